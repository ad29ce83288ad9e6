// Router logits of the gate that stays in BF16 ("clef-omni-fp8" card, section
// "What was quantized"; "clef-omni-NVFP4" card, section "How it was made"),
// read as a linear layer without bias: logits[t, e] = sum_h x[t, h] w[e, h].
//
// A block of 8 waves covers 32 TG tokens x 32 EG experts; each (token group,
// expert group) 32x32 tile (gate_tile, BF16 MFMA with FP32 accumulation) is
// split over KS = 8 / (TG EG) waves along H, and the KS partial tiles are
// added through LDS in wave order (the same order every run).  Below 1024
// tokens TG = EG = 1, KS = 8, so a decode batch still spreads over many waves;
// above, TG = 1, EG = 2, KS = 4.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"
#include "gate.h"
#include "internal.h"

namespace mq {

constexpr int kRouterWaves = 8;

template <int TG, int EG>
__global__ __launch_bounds__(64 * kRouterWaves) void router_logits_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, float *__restrict__ out, int T,
    int H, int E) {
  constexpr int KS = kRouterWaves / (TG * EG);
  static_assert(KS * TG * EG == kRouterWaves, "8 waves per block");
  __shared__ f4 red[KS > 1 ? kRouterWaves : 1][4][64];  // partial tiles (16 floats per lane)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ks = wave % KS, tile = wave / KS;  // k slice; (token group, expert group) tile
  const int t0 = (blockIdx.x * TG + tile / EG) * 32, e0 = (blockIdx.y * EG + tile % EG) * 32;
  const bool live = t0 < T && e0 < E;  // a tile past both ends still takes the barrier
  const int r16 = lane & 15, q16 = lane >> 4;
  const int nchunk = H / 64;
  const int cb = live ? (ks * nchunk) / KS : 0, ce = live ? ((ks + 1) * nchunk) / KS : 0;
  f4 acc[2][2];  // [expert tile][token tile]
  gate_tile(x, w, T, H, E, t0, e0, cb, ce, lane, acc);
  if constexpr (KS > 1) {
    if (ks > 0) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) red[wave][2 * a + b][lane] = acc[a][b];
    }
    __syncthreads();
    if (ks != 0) return;
#pragma unroll
    for (int p = 1; p < KS; ++p)
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const f4 v = red[wave + p][2 * a + b][lane];
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[a][b][i] += v[i];
        }
  }
  // MFMA tile (a, b): lane holds token t0 + 16 b + l % 16 and experts
  // e0 + 16 a + 4 (l / 16) + [0, 4)
  if (!live) return;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int t = t0 + 16 * b + r16;
    if (t >= T) continue;
    float *orow = out + (size_t)t * E;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int e = e0 + 16 * a + 4 * q16;
      if ((E & 3) == 0 && e + 3 < E) {
        *(f4 *)(orow + e) = acc[a][b];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (e + i < E) orow[e + i] = acc[a][b][i];
      }
    }
  }
}

hipError_t launch_router_logits(const uint16_t *x, const uint16_t *w, float *out, int64_t T, int H,
                                int E, hipStream_t s) {
  // Measured at H 2048, E 128 with the 32x32x16 MFMA (us for T = 64 / 4096 /
  // 16384): 32x32 tiles with 8 k slices 9.2 / 18.1 / 68.0; 32x64 with 4
  // slices - / 17.3 / 65.1; 32x128 and 64x64 with 2 slices - / 30.9 / 61.4 and
  // - / 30.3 / 61.9; 64x128 unsplit 57.1 / 57.8 / 60.3.  The 16x16x32 MFMA
  // (64 contiguous bytes per row per load, against 32): 9.2 / 17.1 / 58.9.
  if (T < 1024) {
    const dim3 grid((unsigned)((T + 31) / 32), (unsigned)((E + 31) / 32));
    hipLaunchKernelGGL((router_logits_kernel<1, 1>), grid, dim3(64 * kRouterWaves), 0, s, x, w, out,
                       (int)T, H, E);
  } else {
    const dim3 grid((unsigned)((T + 31) / 32), (unsigned)((E + 63) / 64));
    hipLaunchKernelGGL((router_logits_kernel<1, 2>), grid, dim3(64 * kRouterWaves), 0, s, x, w, out,
                       (int)T, H, E);
  }
  return hipGetLastError();
}

}  // namespace mq

// Router logits of the gate that stays in BF16 ("clef-omni-fp8" card, section
// "What was quantized"; "clef-omni-NVFP4" card, section "How it was made"),
// read as a linear layer without bias: logits[t, e] = sum_h x[t, h] w[e, h].
//
// BF16 MFMA 32x32x16 with FP32 accumulation: every product is exact in FP32
// and only the FP32 sums round.  A block of 8 waves covers 32 TG tokens x
// 32 EG experts; each (token group, expert group) 32x32 tile is split over KS
// = 8 / (TG EG) waves along H, and the KS partial tiles are added through LDS
// in wave order (the same order every run).  Below 1024 tokens TG = EG = 1,
// KS = 8, so a decode batch still spreads over many waves; above, TG = 1,
// EG = 2, KS = 4.  In a wave, lane j = lane % 32 owns expert row
// e0 + j (the MFMA A rows) and token row t0 + j (the B columns).  Per 64-wide
// k chunk c a lane loads 32 values (64 bytes) of each row, k = c + 32 h +
// [0, 32) with h = lane / 32; MFMA s of the chunk takes k = c + 32 h + 8 s +
// [0, 8) on both operands (any k order works when both operands follow it).
// Rows past T or E are clamped on load and never stored.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"
#include "internal.h"

namespace mq {

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));

constexpr int kRouterWaves = 8;

template <int TG, int EG>
__global__ __launch_bounds__(64 * kRouterWaves) void router_logits_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, float *__restrict__ out, int T,
    int H, int E) {
  constexpr int KS = kRouterWaves / (TG * EG);
  static_assert(KS * TG * EG == kRouterWaves, "8 waves per block");
  __shared__ f4 red[KS > 1 ? kRouterWaves : 1][4][64];  // partial tiles (16 floats per lane)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane & 31, hh = lane >> 5;
  const int ks = wave % KS, tile = wave / KS;  // k slice; (token group, expert group) tile
  const int t0 = (blockIdx.x * TG + tile / EG) * 32, e0 = (blockIdx.y * EG + tile % EG) * 32;
  const bool live = t0 < T && e0 < E;  // a tile past both ends still takes the barrier
  const uint16_t *xp = x + (size_t)min(t0 + j, T - 1) * H + 32 * hh;
  const uint16_t *wp = w + (size_t)min(e0 + j, E - 1) * H + 32 * hh;
  const int nchunk = H / 64;
  const int cb = live ? (ks * nchunk) / KS : 0, ce = live ? ((ks + 1) * nchunk) / KS : 0;
  f16v acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll 2
  for (int c = cb * 64; c < ce * 64; c += 64) {
    u4 xa[4], wa[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      xa[q] = *(const u4 *)(xp + c + 8 * q);
      wa[q] = *(const u4 *)(wp + c + 8 * q);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf8, wa[s]),
                                                     __builtin_bit_cast(bf8, xa[s]), acc, 0, 0, 0);
  }
  if constexpr (KS > 1) {
    if (ks > 0) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
        red[wave][g][lane] = f4{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
    }
    __syncthreads();
    if (ks != 0) return;
#pragma unroll
    for (int p = 1; p < KS; ++p)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f4 v = red[wave + p][g][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[4 * g + i] += v[i];
      }
  }
  // lane holds token t0 + j and, in register v, expert e0 + 8 (v / 4) + 4 h + v % 4
  const int t = t0 + j;
  if (!live || t >= T) return;
  float *orow = out + (size_t)t * E;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int e = e0 + 8 * g + 4 * hh;
    if ((E & 3) == 0 && e + 3 < E) {
      *(f4 *)(orow + e) = f4{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (e + i < E) orow[e + i] = acc[4 * g + i];
    }
  }
}

hipError_t launch_router_logits(const uint16_t *x, const uint16_t *w, float *out, int64_t T, int H,
                                int E, hipStream_t s) {
  // Measured at H 2048, E 128 (us for T = 64 / 4096 / 16384): 32x32 tiles
  // with 8 k slices 9.2 / 18.1 / 68.0; 32x64 with 4 slices - / 17.3 / 65.1;
  // 32x128 and 64x64 with 2 slices - / 30.9 / 61.4 and - / 30.3 / 61.9;
  // 64x128 unsplit 57.1 / 57.8 / 60.3.
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

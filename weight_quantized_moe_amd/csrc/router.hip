// Router logits of the gate that stays in BF16 ("clef-omni-fp8" card, section
// "What was quantized"; "clef-omni-NVFP4" card, section "How it was made"),
// read as a linear layer without bias: logits[t, e] = sum_h x[t, h] w[e, h].
//
// BF16 MFMA 32x32x16 with FP32 accumulation: every product is exact in FP32
// and only the FP32 sum rounds.  A block of 4 waves covers 32 tokens x 128
// experts; wave w owns experts 128 by + 32 w + [0, 32) (the MFMA A rows, one
// per lane j = lane % 32) and the block's 32 tokens (the B columns).  Per
// 64-wide k chunk c a lane loads 32 values (64 bytes) of its expert row and of
// its token row, k = c + 32 h + [0, 32) with h = lane / 32; MFMA s of the chunk
// takes k = c + 32 h + 8 s + [0, 8) on both operands (any k order works when
// both operands follow it).  Rows past T or E are clamped on load and never
// stored.  No LDS and no barriers: the weight rows (E x H x 2 bytes, 0.5 MB at
// E = 128, H = 2048) stay in L2 across the token blocks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"
#include "internal.h"

namespace mq {

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t *__restrict__ x,
                                                            const uint16_t *__restrict__ w,
                                                            float *__restrict__ out, int T, int H,
                                                            int E) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane & 31, hh = lane >> 5;
  const int t0 = blockIdx.x * 32, e0 = blockIdx.y * 128 + wave * 32;
  if (e0 >= E) return;  // wave-uniform; the kernel has no barriers
  const uint16_t *xp = x + (size_t)min(t0 + j, T - 1) * H + 32 * hh;
  const uint16_t *wp = w + (size_t)min(e0 + j, E - 1) * H + 32 * hh;
  f16v acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll 2
  for (int c = 0; c < H; c += 64) {
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
  // lane holds token t0 + j and, in register v, expert e0 + 8 (v / 4) + 4 h + v % 4
  const int t = t0 + j;
  if (t >= T) return;
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
  const dim3 grid((unsigned)((T + 31) / 32), (unsigned)((E + 127) / 128)), block(256);
  hipLaunchKernelGGL(router_logits_kernel, grid, block, 0, s, x, w, out, (int)T, H, E);
  return hipGetLastError();
}

}  // namespace mq

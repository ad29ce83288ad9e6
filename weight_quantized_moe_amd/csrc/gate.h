// The router GEMM tile shared by the router-logits kernel and the fused
// router + top-k routing kernel: logits[t, e] = sum_h x[t, h] w[e, h] for the
// BF16 gate that stays unquantized ("clef-omni-fp8" card, section "What was
// quantized"; "clef-omni-NVFP4" card, section "How it was made"), read as a
// linear layer without bias.
//
// BF16 MFMA 16x16x32 with FP32 accumulation: every product is exact in FP32
// and only the FP32 sums round.  One wave computes the partial sum of a 32x32
// (token, expert) tile over a range of 64-wide chunks of H, as 2 x 2 MFMA
// tiles of 16 rows: lane l feeds row l % 16 of a tile with k = 8 (l / 16) +
// [0, 8) of each 32-wide step, so the four lanes of a row read 64 contiguous
// bytes per load (the gate rows are the MFMA A rows, the token rows the B
// columns).  Rows past T or E are clamped on load; the caller never stores
// them.  On return, MFMA tile (a, b) of lane l holds token t0 + 16 b + l % 16
// and experts e0 + 16 a + 4 (l / 16) + [0, 4) (b < NB: a 32x32 tile, or a
// 16-token x 32-expert tile with NB = 1).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"

namespace mq {

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));

template <int NB = 2>  // 16-row token tiles: 32 tokens (2) or 16 tokens (1)
__device__ __forceinline__ void gate_tile(const uint16_t *__restrict__ x,
                                          const uint16_t *__restrict__ w, int T, int H, int E,
                                          int t0, int e0, int cb, int ce, int lane,
                                          f4 (&acc)[2][2]) {
  const int r16 = lane & 15, q16 = lane >> 4;
  const uint16_t *xp[2], *wp[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    xp[i] = x + (size_t)min(t0 + 16 * (i % NB) + r16, T - 1) * H + 8 * q16;
    wp[i] = w + (size_t)min(e0 + 16 * i + r16, E - 1) * H + 8 * q16;
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f4{0.f, 0.f, 0.f, 0.f};
  // operands of one 64-wide chunk: [x, w][tile][32-wide step]
  struct Chunk {
    u4 v[2][2][2];
  };
  auto load = [&](Chunk &ch, int c) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        if (i < NB) ch.v[0][i][s2] = *(const u4 *)(xp[i] + 64 * c + 32 * s2);
        ch.v[1][i][s2] = *(const u4 *)(wp[i] + 64 * c + 32 * s2);
      }
  };
  auto mul = [&](const Chunk &ch) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf8, ch.v[1][a][s2]), __builtin_bit_cast(bf8, ch.v[0][b][s2]),
              acc[a][b], 0, 0, 0);
  };
  // two chunks in registers: the next one loads while the current one
  // multiplies (a plain loop leaves one chunk's loads in flight per wave)
  if (cb >= ce) return;
  Chunk A, B;
  load(A, cb);
  for (int c = cb; c < ce; c += 2) {
    if (c + 1 < ce) load(B, c + 1);
    mul(A);
    if (c + 2 < ce) load(A, c + 2);
    if (c + 1 < ce) mul(B);
  }
}

}  // namespace mq

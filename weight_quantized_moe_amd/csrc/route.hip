// Router top-k + softmax, FP16 staging of the hidden rows, and the stable
// grouping of (token, slot) pairs by expert.
//
// Routing follows the reading documented with the library: the k largest
// logits in descending order, ties to the lower expert id, weights = softmax
// over the selected k.  The router stays an unquantized BF16 layer on the
// model cards ("clef-omni-int4" card, section "Recipe": ignore_layers =
// mlp.gate); its logits arrive as an input.
#include "device.h"
#include "internal.h"

namespace mq {

// Order-preserving map of an IEEE float to an unsigned integer (every bit
// pattern, NaN included, gets a distinct position in a total order).
__device__ __forceinline__ uint32_t ordered_key(float v) {
  uint32_t b = __builtin_bit_cast(uint32_t, v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float from_ordered_key(uint32_t o) {
  uint32_t b = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __builtin_bit_cast(float, b);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = __shfl_xor((uint32_t)v, m, 64);
  uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}

// One wave per token.  Keys pack (ordered logit, ~expert id) so that the wave
// maximum is the largest logit with the lowest id; a selected key is replaced
// by 0, below every real key (the id half of a real key is never 0 because
// E <= 512), so the k winners are always k distinct valid experts.
template <bool kBf16Logits>
__global__ __launch_bounds__(256) void route_kernel(const void *__restrict__ logits,
                                                    const uint16_t *__restrict__ hidden, int T,
                                                    int E, int H, int k, int32_t *__restrict__ ids,
                                                    float *__restrict__ wts,
                                                    _Float16 *__restrict__ x16,
                                                    float *__restrict__ rowscale,
                                                    uint32_t *__restrict__ flags,
                                                    int32_t *__restrict__ p_ids,
                                                    float *__restrict__ p_w) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (blockIdx.x == 0 && threadIdx.x == 0) flags[0] = 0u;
  if (t >= T) return;

  // ---- top-k over the E logits of token t
  constexpr int kPer = kMaxExperts / 64;
  uint64_t key[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = lane + 64 * i;
    key[i] = 0;
    if (e < E) {
      float v;
      if (kBf16Logits)
        v = bf16_to_f32(((const uint16_t *)logits)[(size_t)t * E + e]);
      else
        v = ((const float *)logits)[(size_t)t * E + e];
      key[i] = ((uint64_t)ordered_key(v) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
    }
  }
  float my_v = 0.f;
  int my_id = 0;
  float v_max = 0.f;
  for (int j = 0; j < k; ++j) {   // k <= 64: lane j keeps slot j
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) best = key[i] > best ? key[i] : best;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const uint64_t o = shfl_xor_u64(best, m);
      best = o > best ? o : best;
    }
    const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
    const float v = from_ordered_key((uint32_t)(best >> 32));
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (lane + 64 * i == e) key[i] = 0;
    if (j == 0) v_max = v;
    if (lane == j) {
      my_v = v;
      my_id = e;
    }
  }
  // softmax over the k selected logits
  const float p = lane < k ? expf(my_v - v_max) : 0.f;
  float sum = p;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) sum += __shfl_xor(sum, m, 64);
  if (lane < k) {
    const float w = p / sum;
    ids[(size_t)t * k + lane] = my_id;
    wts[(size_t)t * k + lane] = w;
    if (p_ids) p_ids[(size_t)t * k + lane] = my_id;
    if (p_w) p_w[(size_t)t * k + lane] = w;
  }

  // ---- hidden row -> FP16 scaled by a power of two.  With max|x| mapped into
  // [2^14, 2^15) every BF16 value of the row above max * 2^-31 converts to FP16
  // exactly (BF16 has 8 significant bits, FP16 11, and the FP16 subnormal step
  // there is 2^-24); smaller entries round with an absolute error below
  // max * 2^-39.  The GEMM multiplies its result rows back by 2^s.
  const uint16_t *xr = hidden + (size_t)t * H;
  float m = 0.f;
  for (int c = lane * 8; c < H; c += 512) {
    const u4 v = *(const u4 *)(xr + c);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      m = fmaxf(m, fabsf(bf16_to_f32(v[q] & 0xFFFFu)));
      m = fmaxf(m, fabsf(bf16_to_f32(v[q] >> 16)));
    }
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) m = fmaxf(m, __shfl_xor(m, s, 64));
  int sh = 0;
  if (m > 0.f) {
    const int ex = (int)((__builtin_bit_cast(uint32_t, m) >> 23) & 0xFF) - 127;
    sh = ex - 14;
    sh = sh < -120 ? -120 : (sh > 120 ? 120 : sh);
  }
  const float down = __builtin_bit_cast(float, (uint32_t)(127 - sh) << 23);
  if (lane == 0) rowscale[t] = __builtin_bit_cast(float, (uint32_t)(127 + sh) << 23);
  _Float16 *xo = x16 + (size_t)t * H;
  for (int c = lane * 8; c < H; c += 512) {
    const u4 v = *(const u4 *)(xr + c);
    u4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      h2 hh = {(_Float16)(bf16_to_f32(v[q] & 0xFFFFu) * down),
               (_Float16)(bf16_to_f32(v[q] >> 16) * down)};
      o[q] = as_u32(hh);
    }
    *(u4 *)(xo + c) = o;
  }
}

// ---------------------------------------------------------------------------
// Stable grouping by expert, one workgroup of 1024 threads.
//   1. per-expert counts (LDS atomics);
//   2. exclusive scans: row offsets, prefill M-tile offsets, active experts;
//   3. tokens in chunks of 1024 (16 waves x 64): each wave records, per expert,
//      the 64-bit mask of its lanes routed there; ranks inside the chunk are
//      (rows of earlier waves) + popcount(mask & lanes below me), which keeps
//      token order inside every expert.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void permute_kernel(
    const int32_t *__restrict__ ids, int T, int E, int k, int32_t *__restrict__ offsets,
    int32_t *__restrict__ mtile, int32_t *__restrict__ active, int32_t *__restrict__ sorted_slots,
    int32_t *__restrict__ inv_pos, int32_t *__restrict__ p_offsets,
    int32_t *__restrict__ p_sorted_tok, int32_t *__restrict__ p_inv) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint64_t *mask = (uint64_t *)smem;                      // [16][E]
  int32_t *base = (int32_t *)(mask + 16 * E);              // [16][E]
  int32_t *cnt = base + 16 * E;                            // [E]
  int32_t *cursor = cnt + E;                               // [E]
  int32_t *scan = cursor + E;                              // [3][1024] scratch

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int R = T * k;
  for (int e = tid; e < E; e += 1024) cnt[e] = 0;
  __syncthreads();
  for (int i = tid; i < R; i += 1024) atomicAdd(&cnt[ids[i]], 1);
  __syncthreads();

  // inclusive Hillis-Steele scans of (count, m-tiles, active flag); E <= 1024
  int v0 = 0, v1 = 0, v2 = 0;
  if (tid < E) {
    v0 = cnt[tid];
    v1 = (v0 + kPrefillBM - 1) / kPrefillBM;
    v2 = v0 > 0 ? 1 : 0;
  }
  for (int d = 1; d < 1024; d <<= 1) {
    scan[tid] = v0;
    scan[1024 + tid] = v1;
    scan[2048 + tid] = v2;
    __syncthreads();
    if (tid >= d) {
      v0 += scan[tid - d];
      v1 += scan[1024 + tid - d];
      v2 += scan[2048 + tid - d];
    }
    __syncthreads();
  }
  if (tid < E) {
    const int c = cnt[tid];
    const int ex0 = v0 - c;
    offsets[tid] = ex0;
    if (p_offsets) p_offsets[tid] = ex0;
    mtile[tid] = v1 - (c + kPrefillBM - 1) / kPrefillBM;
    if (c > 0) active[1 + (v2 - 1)] = tid;
    cursor[tid] = ex0;
    if (tid == E - 1) {
      offsets[E] = v0;
      if (p_offsets) p_offsets[E] = v0;
      mtile[E] = v1;
      active[0] = v2;
    }
  }
  __syncthreads();

  for (int c0 = 0; c0 < T; c0 += 1024) {
    for (int i = tid; i < 16 * E; i += 1024) mask[i] = 0ull;
    __syncthreads();
    const int t = c0 + wave * 64 + lane;
    const bool valid = t < T;
    if (valid)
      for (int j = 0; j < k; ++j) atomicOr(&mask[wave * E + ids[(size_t)t * k + j]], 1ull << lane);
    __syncthreads();
    for (int e = tid; e < E; e += 1024) {
      int run = cursor[e];
      for (int w = 0; w < 16; ++w) {
        base[w * E + e] = run;
        run += __popcll(mask[w * E + e]);
      }
      cursor[e] = run;
    }
    __syncthreads();
    if (valid) {
      const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      for (int j = 0; j < k; ++j) {
        const int e = ids[(size_t)t * k + j];
        const int pos = base[wave * E + e] + __popcll(mask[wave * E + e] & below);
        const int slot = t * k + j;
        sorted_slots[pos] = slot;
        inv_pos[slot] = pos;
        if (p_sorted_tok) p_sorted_tok[pos] = t;
        if (p_inv) p_inv[slot] = pos;
      }
    }
    __syncthreads();
  }
}

hipError_t launch_route(const LayerDims &L, const FwdPtrs &P, const Workspace &W, hipStream_t s) {
  char *ws = P.ws;
  dim3 grid((P.T + 3) / 4), block(256);
  if (P.logits_bf16)
    hipLaunchKernelGGL(route_kernel<true>, grid, block, 0, s, P.logits, P.hidden, P.T, L.E, L.H,
                       L.k, (int32_t *)(ws + W.topk_ids), (float *)(ws + W.topk_w),
                       (_Float16 *)(ws + W.x16), (float *)(ws + W.rowscale),
                       (uint32_t *)(ws + W.flags), P.p_ids, P.p_w);
  else
    hipLaunchKernelGGL(route_kernel<false>, grid, block, 0, s, P.logits, P.hidden, P.T, L.E, L.H,
                       L.k, (int32_t *)(ws + W.topk_ids), (float *)(ws + W.topk_w),
                       (_Float16 *)(ws + W.x16), (float *)(ws + W.rowscale),
                       (uint32_t *)(ws + W.flags), P.p_ids, P.p_w);
  return hipGetLastError();
}

hipError_t launch_permute(const LayerDims &L, const FwdPtrs &P, const Workspace &W, hipStream_t s) {
  char *ws = P.ws;
  const size_t lds = (size_t)16 * L.E * 8 + (size_t)16 * L.E * 4 + 2 * (size_t)L.E * 4 + 3 * 1024 * 4;
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(1024), lds, s, (const int32_t *)(ws + W.topk_ids),
                     P.T, L.E, L.k, (int32_t *)(ws + W.offsets), (int32_t *)(ws + W.mtile),
                     (int32_t *)(ws + W.active), (int32_t *)(ws + W.sorted_slots),
                     (int32_t *)(ws + W.inv_pos), P.p_offsets, P.p_sorted_tok, P.p_inv);
  return hipGetLastError();
}

}  // namespace mq

// Router top-k + softmax, FP16 staging of the hidden rows, and the stable
// grouping of (token, slot) pairs by expert.
//
// Routing follows the reading documented with the library: the k largest
// logits in descending order, ties to the lower expert id, weights = softmax
// over the selected k.  The router stays an unquantized BF16 layer on the
// model cards ("clef-omni-int4" card, section "Recipe": ignore_layers =
// mlp.gate); its logits arrive as an input.
//
// Top-k runs on a group of 16 lanes per token (4 tokens per wave): every lane
// holds E/16 keys, and each of the k rounds finds the largest key as two
// 32-bit maxima (the logit half, then the id half among the keys that hold
// it), each a local maximum plus a 4-step DPP all-reduce inside the 16-lane
// row.
#include "device.h"
#include "gate.h"
#include "internal.h"

namespace mq {

// Order-preserving map of an IEEE float to an unsigned integer (every bit
// pattern, NaN included, gets a position in a total order).  -0 maps to the
// key of +0: the two are equal logits, so their order falls to the expert id.
__device__ __forceinline__ uint32_t ordered_key(float v) {
  uint32_t b = __builtin_bit_cast(uint32_t, v);
  if ((b << 1) == 0u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float from_ordered_key(uint32_t o) {
  uint32_t b = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __builtin_bit_cast(float, b);
}

// DPP lane moves inside a 16-lane row (every lane has a valid source).
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, 0xF, 0xF, false);
}
constexpr int kXor1 = 0xB1, kXor2 = 0x4E, kHalfMirror = 0x141, kMirror = 0x140;

__device__ __forceinline__ uint32_t max16_u32(uint32_t v) {
  v = max(v, dpp<kXor1>(v));
  v = max(v, dpp<kXor2>(v));
  v = max(v, dpp<kHalfMirror>(v));
  v = max(v, dpp<kMirror>(v));
  return v;
}
template <int kCtrl>
__device__ __forceinline__ float dppf(float v) {
  return __builtin_bit_cast(float, dpp<kCtrl>(__builtin_bit_cast(uint32_t, v)));
}
__device__ __forceinline__ float sum16(float v) {
  v += dppf<kXor1>(v);
  v += dppf<kXor2>(v);
  v += dppf<kHalfMirror>(v);
  v += dppf<kMirror>(v);
  return v;
}
__device__ __forceinline__ float max16f(float v) {
  v = fmaxf(v, dppf<kXor1>(v));
  v = fmaxf(v, dppf<kXor2>(v));
  v = fmaxf(v, dppf<kHalfMirror>(v));
  v = fmaxf(v, dppf<kMirror>(v));
  return v;
}

// Top-k + softmax of token t on the 16 lanes of one DPP row (li = lane % 16).
// Keys pack (ordered logit, ~expert id): the row maximum is the largest logit
// with the lowest id.  A selected key becomes 0, below every real key (the id
// half of a real key is never 0 since E <= 512), so the k winners are always k
// distinct valid experts.  Results go to ids/wts (and the probe arrays).
template <int kPer, bool kBf16Logits>
__device__ __forceinline__ void topk16_keys(const void *__restrict__ logits, int t, int E, int li,
                                            uint64_t *key) {
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = li + 16 * i;
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
}
template <int kPer>
__device__ __forceinline__ void topk16_select(uint64_t *key, int t, int k, int li,
                                              int32_t *__restrict__ ids, float *__restrict__ wts,
                                              int32_t *__restrict__ p_ids, float *__restrict__ p_w) {
  float sv[4] = {0.f, 0.f, 0.f, 0.f};  // slot j = li + 16 s held by this lane
  int si[4] = {0, 0, 0, 0};
  float vmax = 0.f;
  // The 64-bit maximum taken as two 32-bit ones: the largest ordered logit,
  // then the largest id half among the keys that hold it (32-bit max
  // instructions, no 64-bit compare and select chains).
  uint32_t hi[kPer], lo[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    hi[i] = (uint32_t)(key[i] >> 32);
    lo[i] = (uint32_t)key[i];
  }
  for (int j = 0; j < k; ++j) {
    uint32_t hm = hi[0];
#pragma unroll
    for (int i = 1; i < kPer; ++i) hm = max(hm, hi[i]);
    hm = max16_u32(hm);
    uint32_t lm = 0u;
#pragma unroll
    for (int i = 0; i < kPer; ++i) lm = max(lm, hi[i] == hm ? lo[i] : 0u);
    lm = max16_u32(lm);
    const int e = (int)(0xFFFFFFFFu - lm);
    const float v = from_ordered_key(hm);
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (li + 16 * i == e) hi[i] = lo[i] = 0u;
    if (j == 0) vmax = v;
    if ((j & 15) == li) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
        if ((j >> 4) == s) { sv[s] = v; si[s] = e; }
    }
  }
  float p[4], sum = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    p[s] = (li + 16 * s < k) ? expf(sv[s] - vmax) : 0.f;
    sum += p[s];
  }
  sum = sum16(sum);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int j = li + 16 * s;
    if (j < k) {
      const float w = p[s] / sum;
      ids[(size_t)t * k + j] = si[s];
      wts[(size_t)t * k + j] = w;
      if (p_ids) p_ids[(size_t)t * k + j] = si[s];
      if (p_w) p_w[(size_t)t * k + j] = w;
    }
  }
}
template <int kPer, bool kBf16Logits>
__device__ __forceinline__ void topk16(const void *__restrict__ logits, int t, int E, int k, int li,
                                       int32_t *__restrict__ ids, float *__restrict__ wts,
                                       int32_t *__restrict__ p_ids, float *__restrict__ p_w) {
  uint64_t key[kPer];
  topk16_keys<kPer, kBf16Logits>(logits, t, E, li, key);
  topk16_select<kPer>(key, t, k, li, ids, wts, p_ids, p_w);
}

// Top-k + softmax of token t on all 64 lanes of one wave (batches of at most
// 4 tokens, one per wave; every lane of the wave active).  Lane l holds the
// keys of experts l + 64 i; a round takes the same two 32-bit maxima as
// topk16_select, each a DPP maximum inside the 16-lane rows followed by the
// maximum of the four row results read with v_readlane (wave-uniform).
__device__ __forceinline__ uint32_t max64_u32(uint32_t v) {
  v = max16_u32(v);  // every lane of a row holds the row maximum
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(a, b), max(c, d));
}
__device__ __forceinline__ float sum64f(float v) {
  v = sum16(v);
  const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return ((a + b) + c) + d;
}
template <int kPer64, bool kBf16Logits>
__device__ __forceinline__ void topk64(const void *__restrict__ logits, int t, int E, int k, int lane,
                                       int32_t *__restrict__ ids, float *__restrict__ wts,
                                       int32_t *__restrict__ p_ids, float *__restrict__ p_w) {
  uint32_t hi[kPer64], lo[kPer64];
#pragma unroll
  for (int i = 0; i < kPer64; ++i) {
    const int e = lane + 64 * i;
    hi[i] = lo[i] = 0u;
    if (e < E) {
      const float v = kBf16Logits ? bf16_to_f32(((const uint16_t *)logits)[(size_t)t * E + e])
                                  : ((const float *)logits)[(size_t)t * E + e];
      hi[i] = ordered_key(v);
      lo[i] = 0xFFFFFFFFu - (uint32_t)e;
    }
  }
  float sv = 0.f, vmax = 0.f;  // lane j < k keeps slot j
  int si = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t hm = hi[0];
#pragma unroll
    for (int i = 1; i < kPer64; ++i) hm = max(hm, hi[i]);
    hm = max64_u32(hm);
    uint32_t lm = 0u;
#pragma unroll
    for (int i = 0; i < kPer64; ++i) lm = max(lm, hi[i] == hm ? lo[i] : 0u);
    lm = max64_u32(lm);
    const int e = (int)(0xFFFFFFFFu - lm);
    const float v = from_ordered_key(hm);
#pragma unroll
    for (int i = 0; i < kPer64; ++i)
      if (lane + 64 * i == e) hi[i] = lo[i] = 0u;
    if (j == 0) vmax = v;
    if (j == lane) { sv = v; si = e; }
  }
  const float p = lane < k ? expf(sv - vmax) : 0.f;
  const float sum = sum64f(p);
  if (lane < k) {
    const float w = p / sum;
    ids[(size_t)t * k + lane] = si;
    wts[(size_t)t * k + lane] = w;
    if (p_ids) p_ids[(size_t)t * k + lane] = si;
    if (p_w) p_w[(size_t)t * k + lane] = w;
  }
}

// Hidden rows of the wave's 4 tokens -> FP16 scaled by a power of two each,
// using all 64 lanes per row.  With max|x| mapped into [2^14, 2^15), every BF16
// value of the row above max * 2^-31 converts to FP16 exactly (BF16 has 8
// significant bits, FP16 11, and the FP16 subnormal step there is 2^-24);
// smaller entries round with an absolute error below max * 2^-39.  The GEMMs
// multiply their result rows back by 2^s.  With kPermInt4 every 8 consecutive
// values are stored in the k order of the INT4 unpack ({0,4,1,5,2,6,3,7}, see
// unpack_int4), so INT4 GEMMs use the rows as they are.  Loads of the 4 rows
// are issued together (kChunk per row per round trip).
template <bool kPermInt4, bool kWriteRows = true>
__device__ __forceinline__ void rows_to_f16(const uint16_t *__restrict__ hidden, int t0, int T,
                                            int H, int lane, _Float16 *__restrict__ x16,
                                            float *__restrict__ rowscale) {
  constexpr int kChunk = 4;  // u4 per lane per row per round trip (2048 values)
  float m[4] = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = lane * 8; c0 < H; c0 += 512 * kChunk) {
    u4 v[4][kChunk];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int u = 0; u < kChunk; ++u)
        if (t0 + r < T && c0 + 512 * u < H)
          v[r][u] = *(const u4 *)(hidden + (size_t)(t0 + r) * H + c0 + 512 * u);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int u = 0; u < kChunk; ++u)
        if (t0 + r < T && c0 + 512 * u < H) m[r] = absmax_bf16x8(v[r][u], m[r]);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m[r] = max16f(m[r]);
    m[r] = fmaxf(m[r], __shfl_xor(m[r], 16, 64));
    m[r] = fmaxf(m[r], __shfl_xor(m[r], 32, 64));
  }
  float down[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int sh = row_shift(m[r]);
    down[r] = pow2f(-sh);
    if (lane == 0 && t0 + r < T) rowscale[t0 + r] = pow2f(sh);
  }
  if (!kWriteRows) return;  // the power of two only (decode)
  for (int c0 = lane * 8; c0 < H; c0 += 512 * kChunk) {
    u4 v[4][kChunk];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int u = 0; u < kChunk; ++u)
        if (t0 + r < T && c0 + 512 * u < H)
          v[r][u] = *(const u4 *)(hidden + (size_t)(t0 + r) * H + c0 + 512 * u);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int u = 0; u < kChunk; ++u)
        if (t0 + r < T && c0 + 512 * u < H) {
          const u4 o = bf16x8_to_f16x8(v[r][u], down[r]);
          *(u4 *)(x16 + (size_t)(t0 + r) * H + c0 + 512 * u) = kPermInt4 ? perm_0415(o) : o;
        }
  }
}

// W8A8: the wave's 4 hidden rows as dynamic 1x128 FP8 activations, codes
// [T, H] and FP32 scales [T, H/128].  Each pass covers 512 columns of a row:
// lane l holds columns 8 l + [0, 8), so the 16 lanes of a DPP row hold one
// 128-wide group, whose maximum is a 4-step DPP max.
__device__ __forceinline__ void rows_to_fp8(const uint16_t *__restrict__ hidden, int t0, int T,
                                            int H, int lane, uint8_t *__restrict__ xq,
                                            float *__restrict__ xs) {
  const int G = H / 128;
  for (int r = 0; r < 4; ++r) {
    const int t = t0 + r;
    if (t >= T) break;  // wave-uniform
    for (int c0 = 0; c0 < H; c0 += 512) {
      const int c = c0 + lane * 8;
      const bool ok = c < H;  // whole 16-lane groups (H is a multiple of 128)
      const u4 v = ok ? *(const u4 *)(hidden + (size_t)t * H + c) : u4{0u, 0u, 0u, 0u};
      float f[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_to_f32(v[i] & 0xFFFFu);
        f[2 * i + 1] = bf16_to_f32(v[i] >> 16);
      }
      float m = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
      m = max16f(m);
      const float s = fp8_group_scale(m);
      if (ok) {
        typedef uint32_t u2 __attribute__((ext_vector_type(2)));
        *(u2 *)(xq + (size_t)t * H + c) = u2{e4m3x4(f[0], f[1], f[2], f[3], s), e4m3x4(f[4], f[5], f[6], f[7], s)};
        if ((lane & 15) == 0) xs[(size_t)t * G + c / 128] = s;
      }
    }
  }
}

// W4A4: the wave's 4 hidden rows as NVFP4 activations with global scale g
// (see nvfp4_act_scale), written as the FP16 values e2m1(code) * s into x16
// [T, H] (exact; natural k order, the NVFP4 GEMMs' operand order), with
// rowscale[t] = 1 / g for the GEMM to apply to its sums.  Each pass covers
// 512 columns of a row: lane l holds columns 8 l + [0, 8), so lanes 2i and
// 2i + 1 hold one group of 16.
__device__ __forceinline__ void rows_to_nvfp4(const uint16_t *__restrict__ hidden, int t0, int T,
                                              int H, int lane, float g, _Float16 *__restrict__ x16,
                                              float *__restrict__ rowscale) {
  for (int r = 0; r < 4; ++r) {
    const int t = t0 + r;
    if (t >= T) break;  // wave-uniform
    if (lane == 0) rowscale[t] = 1.f / g;
    for (int c0 = 0; c0 < H; c0 += 512) {
      const int c = c0 + lane * 8;
      const bool ok = c < H;  // whole 2-lane groups (H is a multiple of 128)
      const u4 v = ok ? *(const u4 *)(hidden + (size_t)t * H + c) : u4{0u, 0u, 0u, 0u};
      float f[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_to_f32(v[i] & 0xFFFFu);
        f[2 * i + 1] = bf16_to_f32(v[i] >> 16);
      }
      float m = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
      m = fmaxf(m, __shfl_xor(m, 1, 64));
      const Nvfp4Scale sc = nvfp4_act_scale(m, g);
      u4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const h2 pr = {(_Float16)(e2m1_value(e2m1_code(f[2 * i], g, sc.s)) * sc.s),
                       (_Float16)(e2m1_value(e2m1_code(f[2 * i + 1], g, sc.s)) * sc.s)};
        o[i] = as_u32(pr);
      }
      if (ok) *(u4 *)(x16 + (size_t)t * H + c) = o;
    }
  }
}

// Test entry: FP32 rows [rows, K] -> NVFP4 codes (packed two per byte, low
// nibble first, [rows, K/2]) and E4M3 block scales [rows, K/16], with the
// group arithmetic of rows_to_nvfp4 and the W4A4 gate/up epilogue.  One wave
// per (row, 512-column pass).
__global__ __launch_bounds__(256) void quant_act_nvfp4_kernel(const float *__restrict__ x, int64_t rows,
                                                              int K, float g, uint8_t *__restrict__ codes,
                                                              uint8_t *__restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int passes = (K + 511) / 512;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= rows * passes) return;  // wave-uniform
  const int64_t row = wid / passes;
  const int c = (int)(wid % passes) * 512 + lane * 8;
  const bool ok = c < K;  // K a multiple of 16: lanes 2i and 2i + 1 agree
  float f[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = ok ? x[row * K + c + i] : 0.f;
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
  m = fmaxf(m, __shfl_xor(m, 1, 64));
  const Nvfp4Scale sc = nvfp4_act_scale(m, g);
  uint32_t w = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) w |= e2m1_code(f[i], g, sc.s) << (4 * i);
  if (ok) {
    *(uint32_t *)(codes + row * (K / 2) + c / 2) = w;
    if ((lane & 1) == 0) scales[row * (K / 16) + c / 16] = (uint8_t)sc.code;
  }
}

hipError_t launch_quant_act_nvfp4(const float *x, int64_t rows, int K, float g, uint8_t *codes,
                                  uint8_t *scales, hipStream_t s) {
  const int64_t waves = rows * ((K + 511) / 512);
  hipLaunchKernelGGL(quant_act_nvfp4_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, x, rows,
                     K, g, codes, scales);
  return hipGetLastError();
}

// Test entry: FP32 rows [rows, K] -> dynamic 1x128 FP8 codes and scales, with
// the same group arithmetic as rows_to_fp8 and the W8A8 GEMM epilogue.  One
// wave per (row, 512-column pass).
__global__ __launch_bounds__(256) void quant_act_kernel(const float *__restrict__ x, int64_t rows, int K,
                                                        uint8_t *__restrict__ codes,
                                                        float *__restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int passes = (K + 511) / 512;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= rows * passes) return;  // wave-uniform
  const int64_t row = wid / passes;
  const int c = (int)(wid % passes) * 512 + lane * 8;
  const bool ok = c < K;
  float f[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = ok ? x[row * K + c + i] : 0.f;
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
  m = max16f(m);
  const float s = fp8_group_scale(m);
  if (ok) {
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));
    *(u2 *)(codes + row * K + c) = u2{e4m3x4(f[0], f[1], f[2], f[3], s), e4m3x4(f[4], f[5], f[6], f[7], s)};
    if ((lane & 15) == 0) scales[row * (K / 128) + c / 128] = s;
  }
}

hipError_t launch_quant_act(const float *x, int64_t rows, int K, uint8_t *codes, float *scales,
                            hipStream_t s) {
  const int64_t waves = rows * ((K + 511) / 512);
  hipLaunchKernelGGL(quant_act_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, x, rows, K,
                     codes, scales);
  return hipGetLastError();
}

// Decode: only the power of two of each hidden row (rowscale[t] = 2^s), for
// the wave's 4 tokens (rows of H <= kRowRegsMaxH, read once into registers).  The
// decode gate/up GEMM scales the rows into FP16 itself while staging them.
__device__ __forceinline__ void row_scale_regs(const u4 (&v)[4][4], int t0, int T, int H, int lane,
                                               float *__restrict__ rowscale, float *down = nullptr) {
  float m[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (t0 + r < T && lane * 8 + 512 * u < H) m[r] = absmax_bf16x8(v[r][u], m[r]);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m[r] = max16f(m[r]);
    m[r] = fmaxf(m[r], __shfl_xor(m[r], 16, 64));
    m[r] = fmaxf(m[r], __shfl_xor(m[r], 32, 64));
    const int sh = row_shift(m[r]);
    if (lane == 0 && t0 + r < T) rowscale[t0 + r] = pow2f(sh);
    if (down) down[r] = pow2f(-sh);
  }
}

// General-T routing: 16 lanes per token, 4 tokens per wave, one or four
// waves per block.  Also zeroes the
// flags word and, for the prefill path (stage_rows), stages the hidden rows
// in FP16.
template <int kPer, bool kBf16Logits, bool kPermInt4>
__global__ __launch_bounds__(256) void route_kernel(const void *__restrict__ logits,
                                                    const uint16_t *__restrict__ hidden, int T,
                                                    int E, int H, int k, int32_t *__restrict__ ids,
                                                    float *__restrict__ wts,
                                                    _Float16 *__restrict__ x16,
                                                    float *__restrict__ rowscale,
                                                    uint32_t *__restrict__ flags,
                                                    int32_t *__restrict__ p_ids,
                                                    float *__restrict__ p_w, int stage_rows,
                                                    float act_g) {
  const int lane = threadIdx.x & 63, li = lane & 15;
  const int tpb = blockDim.x >> 4;  // tokens per block: 16 lanes each
  const int t = blockIdx.x * tpb + (threadIdx.x >> 4);
  const int t0 = blockIdx.x * tpb + (threadIdx.x >> 6) * 4;  // first token of this wave
  if (blockIdx.x == 0 && threadIdx.x == 0) flags[0] = 0u;
  if (t0 >= T) return;
  static_assert(kRowRegsMaxH == 4 * 64 * 8, "4 x 16 bytes per lane cover one row");
  if (stage_rows == 3) {  // W8A8: FP8 codes and scales of the hidden rows
    if (t < T) topk16<kPer, kBf16Logits>(logits, t, E, k, li, ids, wts, p_ids, p_w);
    rows_to_fp8(hidden, t0, T, H, lane, (uint8_t *)x16, (float *)((uint8_t *)x16 + (size_t)T * H));
    return;
  }
  if (stage_rows == 4) {  // W4A4: the hidden rows as NVFP4 activations
    if (t < T) topk16<kPer, kBf16Logits>(logits, t, E, k, li, ids, wts, p_ids, p_w);
    rows_to_nvfp4(hidden, t0, T, H, lane, act_g, x16, rowscale);
    return;
  }
  if (stage_rows != 0 && H <= kRowRegsMaxH) {
    // rows of up to 2048 values: the rows' loads and the logits' loads in
    // flight together, each row read once (decode keeps only its scale,
    // prefill also writes the FP16 row)
    uint64_t key[kPer];
    if (t < T) topk16_keys<kPer, kBf16Logits>(logits, t, E, li, key);
    u4 v[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        v[r][u] = t0 + r < T && lane * 8 + 512 * u < H
                      ? *(const u4 *)(hidden + (size_t)(t0 + r) * H + lane * 8 + 512 * u)
                      : u4{0u, 0u, 0u, 0u};
    float down[4];
    row_scale_regs(v, t0, T, H, lane, rowscale, down);
    if (stage_rows == 1) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (t0 + r < T && lane * 8 + 512 * u < H) {
            const u4 o = bf16x8_to_f16x8(v[r][u], down[r]);
            *(u4 *)(x16 + (size_t)(t0 + r) * H + lane * 8 + 512 * u) = kPermInt4 ? perm_0415(o) : o;
          }
    }
    if (t < T) topk16_select<kPer>(key, t, k, li, ids, wts, p_ids, p_w);
    return;
  }
  if (t < T) topk16<kPer, kBf16Logits>(logits, t, E, k, li, ids, wts, p_ids, p_w);
  if (stage_rows) rows_to_f16<kPermInt4>(hidden, t0, T, H, lane, x16, rowscale);
}

// ---------------------------------------------------------------------------
// Router GEMM fused with the top-k: the logits of the BF16 gate (read as a
// linear layer without bias, logits[t, e] = sum_h x[t, h] w[e, h]; the router
// stays unquantized on every card: "clef-omni-int4" card, section "Recipe";
// "clef-omni-NVFP4" card, section "How it was made") are computed for a block
// of 16 or 32 tokens and all E <= 32 EG experts, kept in LDS, and selected there by
// the same 16-lanes-per-token top-k as route_kernel, while the other half of
// the block stages the tokens' hidden rows as route_kernel does.  The logits
// reach HBM only when the caller asks for them (p_logits).
//   GEMM: 16 waves = EG expert groups of 32 x KS = 16 / EG slices of H; each
//   wave computes a 32x32 partial tile (gate_tile, BF16 MFMA, FP32 sums, the
//   next 64-wide chunk loading while one multiplies) and the KS partials of a tile are
//   added through LDS in wave order, so repeated runs are bit-identical.  The
//   16 waves keep enough loads in flight to stream the whole gate through
//   each block (512 KB at 128 experts x 2048).
// ---------------------------------------------------------------------------
constexpr int kGateWaves = 16;

template <int EG, bool kPermInt4, int TB>
__global__ __launch_bounds__(64 * kGateWaves) void gate_route_kernel(
    const uint16_t *__restrict__ hidden, const uint16_t *__restrict__ gate_w, int T, int E, int H,
    int k, int32_t *__restrict__ ids, float *__restrict__ wts, _Float16 *__restrict__ x16,
    float *__restrict__ rowscale, uint32_t *__restrict__ flags, int32_t *__restrict__ p_ids,
    float *__restrict__ p_w, float *__restrict__ p_logits, int stage_rows) {
  constexpr int KS = kGateWaves / EG, kPer = 2 * EG, EP = 32 * EG + 4, NB = TB / 16;
  static_assert(KS >= 2 && (TB == 16 || TB == 32), "H slices per expert group; 16 or 32 tokens");
  __shared__ f4 red[kGateWaves][4][64];  // partial tiles (16 floats per lane)
  __shared__ float lg[TB][EP];           // the block's logits [token][expert]
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ks = wave % KS, eg = wave / KS;
  const int t0 = blockIdx.x * TB, e0 = eg * 32;
  if (blockIdx.x == 0 && threadIdx.x == 0) flags[0] = 0u;
  const bool live = e0 < E;  // an expert group past E still takes the barriers
  const int nchunk = H / 64;
  const int cb = live ? (ks * nchunk) / KS : 0, ce = live ? ((ks + 1) * nchunk) / KS : 0;
  f4 acc[2][2];
  gate_tile<NB>(hidden, gate_w, T, H, E, t0, e0, cb, ce, lane, acc);
  if (ks > 0) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b) red[wave][2 * a + b][lane] = acc[a][b];
  }
  __syncthreads();
  if (ks == 0 && live) {
#pragma unroll
    for (int p = 1; p < KS; ++p)
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const f4 v = red[wave + p][2 * a + b][lane];
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[a][b][i] += v[i];
        }
    // MFMA tile (a, b): token 16 b + l % 16, experts e0 + 16 a + 4 (l / 16) + [0, 4)
    const int r16 = lane & 15, q16 = lane >> 4;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) lg[16 * b + r16][e0 + 16 * a + 4 * q16 + i] = acc[a][b][i];
  }
  __syncthreads();
  if (wave < TB / 4) {
    // top-k of token t0 + tl on the 16 lanes of one DPP row
    const int tl = threadIdx.x >> 4, li = threadIdx.x & 15, t = t0 + tl;
    if (t < T) {
      uint64_t key[kPer];
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int e = li + 16 * i;
        key[i] = e < E ? ((uint64_t)ordered_key(lg[tl][e]) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e) : 0;
      }
      topk16_select<kPer>(key, t, k, li, ids, wts, p_ids, p_w);
      if (p_logits)
        for (int e = li; e < E; e += 16) p_logits[(size_t)t * E + e] = lg[tl][e];
    }
  } else if (wave < TB / 2) {
    // hidden rows of 4 tokens per wave: FP16 rows and their powers of two
    // (prefill), the powers of two alone (decode), or nothing (decode with
    // rows longer than kRowRegsMaxH: the GEMM scans them itself)
    const int tr = t0 + 4 * (wave - TB / 4);
    if (stage_rows == 1)
      rows_to_f16<kPermInt4>(hidden, tr, T, H, lane, x16, rowscale);
    else if (stage_rows == 2)
      rows_to_f16<kPermInt4, false>(hidden, tr, T, H, lane, x16, rowscale);
  }
}

// ---------------------------------------------------------------------------
// Exclusive scan of cnt[0..E) (E <= 512) by one wave; also the prefill
// M-tile counts and the table of active experts.  Writes offsets[E+1],
// mtile[E+1], einfo ({count of active experts, their 16-row chunks}, then one
// {expert, first grouped row, rows, 0} entry per active expert in ascending
// expert order),
// rcp (per active expert, the prefix of the 16-row chunks of the experts
// before it, then the total: [count + 1] entries)
// and, if given, p_offsets.  Lanes hold 8 consecutive experts.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void scan_experts_wave(const int32_t *cnt, int E, int lane,
                                                  int32_t *__restrict__ offsets,
                                                  int32_t *__restrict__ mtile,
                                                  int4 *__restrict__ einfo,
                                                  int32_t *__restrict__ rcp,
                                                  int32_t *__restrict__ p_offsets,
                                                  int32_t *cursor) {
  int c[8], s0 = 0, s1 = 0, s2 = 0, s3 = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int e = lane * 8 + i;
    c[i] = e < E ? cnt[e] : 0;
    s0 += c[i];
    s1 += (c[i] + kPrefillBM - 1) / kPrefillBM;
    s2 += c[i] > 0;
    s3 += (c[i] + 15) >> 4;
  }
  int i0 = s0, i1 = s1, i2 = s2, i3 = s3;  // inclusive wave scans
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int a0 = __shfl_up(i0, d, 64), a1 = __shfl_up(i1, d, 64), a2 = __shfl_up(i2, d, 64);
    const int a3 = __shfl_up(i3, d, 64);
    if (lane >= d) { i0 += a0; i1 += a1; i2 += a2; i3 += a3; }
  }
  int r0 = i0 - s0, r1 = i1 - s1, r2 = i2 - s2, r3 = i3 - s3;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int e = lane * 8 + i;
    if (e < E) {
      offsets[e] = r0;
      if (p_offsets) p_offsets[e] = r0;
      if (cursor) cursor[e] = r0;
      mtile[e] = r1;
      if (c[i] > 0) {
        einfo[1 + r2] = int4{e, r0, c[i], 0};
        rcp[r2] = r3;
      }
    }
    r0 += c[i];
    r1 += (c[i] + kPrefillBM - 1) / kPrefillBM;
    r2 += c[i] > 0;
    r3 += (c[i] + 15) >> 4;
  }
  if (lane == 63) {
    offsets[E] = i0;
    if (p_offsets) p_offsets[E] = i0;
    mtile[E] = i1;
    einfo[0] = int4{i2, i3, 0, 0};
    rcp[i2] = i3;
  }
}

// ---------------------------------------------------------------------------
// T <= kSmallT (and T k <= kSmallRows): grouping in one workgroup of 1024
// threads, after route_kernel's top-k (whose 16-lane-per-token selection is
// VALU work worth spreading over several CUs).  A bit mask of tokens per
// expert (one 64-bit word per 64 tokens) gives the counts (popcounts) and the
// stable rank of every token inside its expert (popcount of the mask bits
// below it).
// ---------------------------------------------------------------------------
// NTH threads of one workgroup group the T k (token, slot) pairs whose experts
// are ids[] (ids, wts and rowscale may be in LDS or global memory).
template <int NTH>
__device__ __forceinline__ void group_small_body(
    const int32_t *ids, const float *wts, const float *rowscale, int T, int E, int k,
    int32_t *__restrict__ offsets, int32_t *__restrict__ mtile, int4 *__restrict__ einfo,
    int32_t *__restrict__ rcp, int32_t *__restrict__ sorted_slots, int4 *__restrict__ rowinfo,
    int32_t *__restrict__ inv_pos, int32_t *__restrict__ p_offsets, int32_t *__restrict__ p_sorted_tok,
    int32_t *__restrict__ p_inv, int32_t *sm_ids) {
  __shared__ uint64_t mask[kMaxExperts * (kSmallT / 64)];  // [E][NW]
  __shared__ int32_t cnt[kMaxExperts];
  __shared__ int32_t off[kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63;
  const int NW = (T + 63) >> 6;  // mask words per expert
  for (int i = tid; i < E * NW; i += NTH) mask[i] = 0ull;
  if (sm_ids != ids)
    for (int i = tid; i < T * k; i += NTH) sm_ids[i] = ids[i];
  __syncthreads();
  for (int i = tid; i < T * k; i += NTH) {
    const int tt = i / k;
    atomicOr(&mask[sm_ids[i] * NW + (tt >> 6)], 1ull << (tt & 63));
  }
  __syncthreads();
  for (int e = tid; e < E; e += NTH) {
    int c = 0;
    for (int w = 0; w < NW; ++w) c += __popcll(mask[e * NW + w]);
    cnt[e] = c;
  }
  __syncthreads();
  if (tid < 64) scan_experts_wave(cnt, E, lane, offsets, mtile, einfo, rcp, p_offsets, off);
  __syncthreads();
  for (int i = tid; i < T * k; i += NTH) {
    const int tt = i / k, e = sm_ids[i], tw = tt >> 6, tb = tt & 63;
    const uint64_t below = tb == 0 ? 0ull : (~0ull >> (64 - tb));
    int pos = off[e] + __popcll(mask[e * NW + tw] & below);
    for (int w = 0; w < tw; ++w) pos += __popcll(mask[e * NW + w]);
    sorted_slots[pos] = i;
    const float rs = rowscale ? rowscale[tt] : 0.f;
    rowinfo[pos] = int4{i, tt, __builtin_bit_cast(int, rs), __builtin_bit_cast(int, wts[i])};
    inv_pos[i] = pos;
    if (p_sorted_tok) p_sorted_tok[pos] = tt;
    if (p_inv) p_inv[i] = pos;
  }
}

__global__ __launch_bounds__(1024) void group_small_kernel(
    const int32_t *__restrict__ ids, const float *__restrict__ wts, const float *__restrict__ rowscale,
    int T, int E, int k, int32_t *__restrict__ offsets, int32_t *__restrict__ mtile,
    int4 *__restrict__ einfo, int32_t *__restrict__ rcp, int32_t *__restrict__ sorted_slots,
    int4 *__restrict__ rowinfo,
    int32_t *__restrict__ inv_pos, int32_t *__restrict__ p_offsets, int32_t *__restrict__ p_sorted_tok,
    int32_t *__restrict__ p_inv) {
  __shared__ int32_t sm_ids[kSmallRows];
  group_small_body<1024>(ids, wts, rowscale, T, E, k, offsets, mtile, einfo, rcp, sorted_slots, rowinfo,
                         inv_pos, p_offsets, p_sorted_tok, p_inv, sm_ids);
}

// ---------------------------------------------------------------------------
// Decode batches of up to kFusedT tokens: routing and grouping in one
// workgroup of 4 waves (one launch less on the latency-bound smallest steps).
// Each wave takes 4 tokens as route_kernel does (top-k on 16 lanes per token,
// and with rows of at most kRowRegsMaxH values the rows' powers of two); with
// at most 4 tokens each wave takes one token on all its lanes (topk64) and
// wave 0 finds the rows' powers of two.  The ids, weights and powers of two
// stay in LDS for the grouping, and are also written out for the kernels
// after it.
// ---------------------------------------------------------------------------
template <int kPer, bool kBf16Logits>
__global__ __launch_bounds__(256) void route_group_kernel(
    const void *__restrict__ logits, const uint16_t *__restrict__ hidden, int T, int E, int H, int k,
    int32_t *__restrict__ ids, float *__restrict__ wts, float *__restrict__ rowscale,
    uint32_t *__restrict__ flags, int32_t *__restrict__ p_ids, float *__restrict__ p_w, int with_scales,
    int32_t *__restrict__ offsets, int32_t *__restrict__ mtile, int4 *__restrict__ einfo,
    int32_t *__restrict__ rcp, int32_t *__restrict__ sorted_slots, int4 *__restrict__ rowinfo,
    int32_t *__restrict__ inv_pos, int32_t *__restrict__ p_offsets, int32_t *__restrict__ p_sorted_tok,
    int32_t *__restrict__ p_inv) {
  __shared__ int32_t s_ids[kFusedT * 64];
  __shared__ float s_wts[kFusedT * 64];
  __shared__ float s_rs[kFusedT];
  const int lane = threadIdx.x & 63, li = lane & 15;
  const int t = threadIdx.x >> 4, t0 = (threadIdx.x >> 6) * 4;
  if (threadIdx.x == 0) flags[0] = 0u;
  if (T <= 4) {
    // one token per wave on all its lanes (wave 0 also finds the rows' powers of two)
    const int wave = threadIdx.x >> 6;
    if (wave == 0 && with_scales) {
      u4 v[4][4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          v[r][u] = r < T && lane * 8 + 512 * u < H ? *(const u4 *)(hidden + (size_t)r * H + lane * 8 + 512 * u)
                                                     : u4{0u, 0u, 0u, 0u};
      row_scale_regs(v, 0, T, H, lane, s_rs);
    }
    if (wave < T) topk64<kPer / 4, kBf16Logits>(logits, wave, E, k, lane, s_ids, s_wts, p_ids, p_w);
  } else if (t0 < T) {
    uint64_t key[kPer];
    if (t < T) topk16_keys<kPer, kBf16Logits>(logits, t, E, li, key);
    if (with_scales) {
      u4 v[4][4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          v[r][u] = t0 + r < T && lane * 8 + 512 * u < H
                        ? *(const u4 *)(hidden + (size_t)(t0 + r) * H + lane * 8 + 512 * u)
                        : u4{0u, 0u, 0u, 0u};
      row_scale_regs(v, t0, T, H, lane, s_rs);
    }
    if (t < T) topk16_select<kPer>(key, t, k, li, s_ids, s_wts, p_ids, p_w);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < T * k; i += 256) {
    ids[i] = s_ids[i];
    wts[i] = s_wts[i];
  }
  if (with_scales && threadIdx.x < T) rowscale[threadIdx.x] = s_rs[threadIdx.x];
  group_small_body<256>(s_ids, s_wts, with_scales ? s_rs : nullptr, T, E, k, offsets, mtile, einfo, rcp,
                        sorted_slots, rowinfo, inv_pos, p_offsets, p_sorted_tok, p_inv, s_ids);
}

// ---------------------------------------------------------------------------
// Stable grouping by expert for larger batches, in three launches over chunks of
// consecutive tokens (at most kMaxChunks chunks):
//   1. hist_kernel:    per-chunk expert counts cnt[c][e];
//   2. scan_kernel:    one workgroup turns them into the exclusive position of
//                      every chunk's first row of expert e,
//                      base[c][e] = offsets[e] + sum_{c' < c} cnt[c'][e],
//                      plus offsets, M-tile prefix and the active-expert list;
//   3. scatter_kernel: ranks inside a chunk, 256 tokens at a time (4 waves x 64
//                      lanes): per wave and expert the 64-bit mask of lanes
//                      routed there; a row's rank is (rows of earlier waves) +
//                      popcount(mask & lanes below it), which keeps token order
//                      inside every expert.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void hist_kernel(const int32_t *__restrict__ ids, int T, int E,
                                                   int k, int chunk, int32_t *__restrict__ cnt) {
  extern __shared__ int32_t sc[];  // [E]
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 256) sc[e] = 0;
  __syncthreads();
  const int t0 = blockIdx.x * chunk, t1 = min(T, t0 + chunk);
  for (int i = t0 * k + tid; i < t1 * k; i += 256) atomicAdd(&sc[ids[i]], 1);
  __syncthreads();
  for (int e = tid; e < E; e += 256) cnt[(size_t)blockIdx.x * E + e] = sc[e];
}

__global__ __launch_bounds__(1024) void scan_kernel(int32_t *__restrict__ cnt, int nc, int E,
                                                    int32_t *__restrict__ offsets,
                                                    int32_t *__restrict__ mtile,
                                                    int4 *__restrict__ einfo,
                                                    int32_t *__restrict__ rcp,
                                                    int32_t *__restrict__ p_offsets) {
  __shared__ int32_t tot[kMaxExperts];
  __shared__ int32_t off[kMaxExperts];
  __shared__ int32_t subpre[kMaxExperts][8];
  const int tid = threadIdx.x, sub = tid & 7;
  // 8 threads per expert, each over a contiguous range of chunks
  const int per = (nc + 7) / 8, c0 = min(nc, sub * per), c1 = min(nc, c0 + per);
  for (int e0 = 0; e0 < E; e0 += 128) {
    const int e = e0 + (tid >> 3);
    int s = 0;
    if (e < E)
      for (int c = c0; c < c1; ++c) s += cnt[(size_t)c * E + e];
    int incl = s;
#pragma unroll
    for (int d = 1; d < 8; d <<= 1) {
      const int v = __shfl_up(incl, d, 8);
      if (sub >= d) incl += v;
    }
    if (e < E) {
      subpre[e][sub] = incl - s;
      if (sub == 7) tot[e] = incl;
    }
  }
  __syncthreads();
  if (tid < 64) scan_experts_wave(tot, E, tid, offsets, mtile, einfo, rcp, p_offsets, off);
  __syncthreads();
  for (int e0 = 0; e0 < E; e0 += 128) {
    const int e = e0 + (tid >> 3);
    if (e >= E) continue;
    int run = off[e] + subpre[e][sub];
    for (int c = c0; c < c1; ++c) {
      const int v = cnt[(size_t)c * E + e];
      cnt[(size_t)c * E + e] = run;
      run += v;
    }
  }
}

__global__ __launch_bounds__(256) void scatter_kernel(
    const int32_t *__restrict__ ids, const float *__restrict__ wts,
    const float *__restrict__ rowscale, int T, int E, int k, int chunk,
    const int32_t *__restrict__ base, int32_t *__restrict__ sorted_slots,
    int4 *__restrict__ rowinfo, int32_t *__restrict__ inv_pos, int32_t *__restrict__ p_sorted_tok,
    int32_t *__restrict__ p_inv) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint64_t *mask = (uint64_t *)smem;              // [4][E]
  int32_t *wbase = (int32_t *)(mask + 4 * E);     // [4][E]
  int32_t *cursor = wbase + 4 * E;                // [E]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int e = tid; e < E; e += 256) cursor[e] = base[(size_t)blockIdx.x * E + e];
  const int t0 = blockIdx.x * chunk, t1 = min(T, t0 + chunk);
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  for (int s0 = t0; s0 < t1; s0 += 256) {
    for (int i = tid; i < 4 * E; i += 256) mask[i] = 0ull;
    __syncthreads();
    const int t = s0 + tid;
    const bool valid = t < t1;
    if (valid)
      for (int j = 0; j < k; ++j) atomicOr(&mask[wave * E + ids[(size_t)t * k + j]], 1ull << lane);
    __syncthreads();
    for (int e = tid; e < E; e += 256) {
      int run = cursor[e];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        wbase[w * E + e] = run;
        run += __popcll(mask[w * E + e]);
      }
      cursor[e] = run;
    }
    __syncthreads();
    if (valid) {
      for (int j = 0; j < k; ++j) {
        const int e = ids[(size_t)t * k + j];
        const int pos = wbase[wave * E + e] + __popcll(mask[wave * E + e] & below);
        const int slot = t * k + j;
        sorted_slots[pos] = slot;
        const float rs = rowscale ? rowscale[t] : 0.f;
        rowinfo[pos] = int4{slot, t, __builtin_bit_cast(int, rs), __builtin_bit_cast(int, wts[slot])};
        inv_pos[slot] = pos;
        if (p_sorted_tok) p_sorted_tok[pos] = t;
        if (p_inv) p_inv[slot] = pos;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
template <int kPer, bool kBf16, bool kPerm>
static hipError_t route_dispatch(const LayerDims &L, const FwdPtrs &P, const Workspace &W,
                                 int stage_rows, hipStream_t s) {
  char *ws = P.ws;
  // decode batches: one wave (4 tokens) per workgroup spreads the row reads
  // over more CUs; otherwise 16 tokens per workgroup
  const int threads = stage_rows == 2 || P.T <= 256 ? 64 : 256, tpb = threads / 16;
  hipLaunchKernelGGL((route_kernel<kPer, kBf16, kPerm>), dim3((P.T + tpb - 1) / tpb), dim3(threads), 0, s,
                     P.logits, P.hidden, P.T, L.E, L.H, L.k, (int32_t *)(ws + W.topk_ids),
                     (float *)(ws + W.topk_w), (_Float16 *)(ws + W.x16), (float *)(ws + W.rowscale),
                     P.flags, P.p_ids, P.p_w, stage_rows, P.act_g13);
  return hipGetLastError();
}

template <int kPer>
static hipError_t route_dispatch2(const LayerDims &L, const FwdPtrs &P, const Workspace &W,
                                  int stage_rows, hipStream_t s) {
  const bool perm = L.fmt == FMT_INT4;
  if (P.logits_bf16)
    return perm ? route_dispatch<kPer, true, true>(L, P, W, stage_rows, s)
                : route_dispatch<kPer, true, false>(L, P, W, stage_rows, s);
  return perm ? route_dispatch<kPer, false, true>(L, P, W, stage_rows, s)
              : route_dispatch<kPer, false, false>(L, P, W, stage_rows, s);
}

template <int kPer>
static hipError_t route_group_dispatch(const LayerDims &L, const FwdPtrs &P, const Workspace &W,
                                       int stage_rows, hipStream_t s) {
  char *ws = P.ws;
  auto k = P.logits_bf16 ? route_group_kernel<kPer, true> : route_group_kernel<kPer, false>;
  hipLaunchKernelGGL(k, dim3(1), dim3(256), 0, s, P.logits, P.hidden, P.T, L.E, L.H, L.k,
                     (int32_t *)(ws + W.topk_ids), (float *)(ws + W.topk_w), (float *)(ws + W.rowscale),
                     P.flags, P.p_ids, P.p_w, stage_rows == 2 ? 1 : 0, (int32_t *)(ws + W.offsets),
                     (int32_t *)(ws + W.mtile), (int4 *)(ws + W.active), (int32_t *)(ws + W.rcpre),
                     (int32_t *)(ws + W.sorted_slots), (int4 *)(ws + W.rowinfo), (int32_t *)(ws + W.inv_pos),
                     P.p_offsets, P.p_sorted_tok, P.p_inv);
  return hipGetLastError();
}

template <int EG, bool kPerm>
static hipError_t gate_route_launch(const LayerDims &L, const FwdPtrs &P, const Workspace &W,
                                    int stage_rows, hipStream_t s) {
  char *ws = P.ws;
  // 16 tokens per block up to 8192 tokens (twice the blocks: the batch then
  // spreads over more CUs), 32 above (half the gate reads from L2)
  if (P.T <= 8192) {
    hipLaunchKernelGGL((gate_route_kernel<EG, kPerm, 16>), dim3((P.T + 15) / 16), dim3(64 * kGateWaves), 0, s,
                       P.hidden, P.gate_w, P.T, L.E, L.H, L.k, (int32_t *)(ws + W.topk_ids),
                       (float *)(ws + W.topk_w), (_Float16 *)(ws + W.x16), (float *)(ws + W.rowscale),
                       P.flags, P.p_ids, P.p_w, P.p_logits, stage_rows);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((gate_route_kernel<EG, kPerm, 32>), dim3((P.T + 31) / 32), dim3(64 * kGateWaves), 0, s, P.hidden,
                     P.gate_w, P.T, L.E, L.H, L.k, (int32_t *)(ws + W.topk_ids), (float *)(ws + W.topk_w),
                     (_Float16 *)(ws + W.x16), (float *)(ws + W.rowscale), P.flags, P.p_ids, P.p_w,
                     P.p_logits, stage_rows);
  return hipGetLastError();
}

template <bool kPerm>
static hipError_t gate_route_dispatch(const LayerDims &L, const FwdPtrs &P, const Workspace &W,
                                      int stage_rows, hipStream_t s) {
  if (L.E <= 32) return gate_route_launch<1, kPerm>(L, P, W, stage_rows, s);
  if (L.E <= 64) return gate_route_launch<2, kPerm>(L, P, W, stage_rows, s);
  if (L.E <= 128) return gate_route_launch<4, kPerm>(L, P, W, stage_rows, s);
  return gate_route_launch<8, kPerm>(L, P, W, stage_rows, s);  // E <= kMaxGateExperts
}

hipError_t launch_route(const LayerDims &L, const FwdPtrs &P, const Workspace &W, bool decode,
                        hipStream_t s) {
  // prefill: FP16 rows and their scales (1); decode with H <= 2048: the
  // scales only (2), the decode gate/up GEMM converts the rows it stages;
  // larger decode rows: the GEMM finds the scales too (0); W8A8: FP8 codes
  // and scales (3); W4A4: NVFP4 values and 1 / g (4)
  const int stage_rows = P.w8a8 ? 3 : P.act_g13 > 0.f ? 4 : !decode ? 1 : L.H <= kRowRegsMaxH ? 2 : 0;
  if (P.gate_w && P.T >= kGateFusedMinT)  // router GEMM fused with the top-k
    return L.fmt == FMT_INT4 ? gate_route_dispatch<true>(L, P, W, stage_rows, s)
                             : gate_route_dispatch<false>(L, P, W, stage_rows, s);
  if (P.gate_w) {
    // small batch: the router logits kernel, then route_kernel on its logits
    FwdPtrs Q = P;
    float *lg = P.p_logits ? P.p_logits : (float *)(P.ws + W.logits);
    hipError_t e = launch_router_logits(P.hidden, P.gate_w, lg, P.T, L.H, L.E, s);
    if (e != hipSuccess) return e;
    Q.logits = lg;
    Q.logits_bf16 = 0;
    Q.gate_w = nullptr;
    return launch_route(L, Q, W, decode, s);
  }
  if (route_groups(L, P, decode)) {
    if (L.E <= 128) return route_group_dispatch<8>(L, P, W, stage_rows, s);
    if (L.E <= 256) return route_group_dispatch<16>(L, P, W, stage_rows, s);
    return route_group_dispatch<32>(L, P, W, stage_rows, s);
  }
  if (L.E <= 128) return route_dispatch2<8>(L, P, W, stage_rows, s);
  if (L.E <= 256) return route_dispatch2<16>(L, P, W, stage_rows, s);
  return route_dispatch2<32>(L, P, W, stage_rows, s);
}

bool route_groups(const LayerDims &L, const FwdPtrs &P, bool decode) {
  (void)L;
  return decode && !P.w8a8 && P.act_g13 == 0.f && P.T <= kFusedT;
}

hipError_t launch_permute(const LayerDims &L, const FwdPtrs &P, const Workspace &W, bool decode,
                          hipStream_t s) {
  char *ws = P.ws;
  if (route_groups(L, P, decode)) return hipSuccess;  // the routing kernel grouped the rows
  if (P.T <= kSmallT && P.T * L.k <= kSmallRows) {
    hipLaunchKernelGGL(group_small_kernel, dim3(1), dim3(1024), 0, s, (const int32_t *)(ws + W.topk_ids),
                       (const float *)(ws + W.topk_w), decode && L.H > kRowRegsMaxH ? (const float *)nullptr : (const float *)(ws + W.rowscale),
                       P.T, L.E, L.k, (int32_t *)(ws + W.offsets), (int32_t *)(ws + W.mtile),
                       (int4 *)(ws + W.active), (int32_t *)(ws + W.rcpre), (int32_t *)(ws + W.sorted_slots),
                       (int4 *)(ws + W.rowinfo),
                       (int32_t *)(ws + W.inv_pos), P.p_offsets, P.p_sorted_tok, P.p_inv);
    return hipGetLastError();
  }
  int nc, chunk;
  permute_chunks(P.T, &nc, &chunk);
  int32_t *cnt = (int32_t *)(ws + W.chunks);
  hipLaunchKernelGGL(hist_kernel, dim3(nc), dim3(256), (size_t)L.E * 4, s,
                     (const int32_t *)(ws + W.topk_ids), P.T, L.E, L.k, chunk, cnt);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, cnt, nc, L.E,
                     (int32_t *)(ws + W.offsets), (int32_t *)(ws + W.mtile),
                     (int4 *)(ws + W.active), (int32_t *)(ws + W.rcpre), P.p_offsets);
  hipLaunchKernelGGL(scatter_kernel, dim3(nc), dim3(256), (size_t)L.E * (4 * 8 + 4 * 4 + 4), s,
                     (const int32_t *)(ws + W.topk_ids), (const float *)(ws + W.topk_w),
                     decode && L.H > kRowRegsMaxH ? nullptr : (const float *)(ws + W.rowscale), P.T, L.E, L.k, chunk,
                     (const int32_t *)cnt, (int32_t *)(ws + W.sorted_slots),
                     (int4 *)(ws + W.rowinfo), (int32_t *)(ws + W.inv_pos), P.p_sorted_tok,
                     P.p_inv);
  return hipGetLastError();
}

}  // namespace mq

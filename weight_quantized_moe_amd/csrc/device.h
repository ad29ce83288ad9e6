// Device helpers for gfx950 (CDNA4): vector types, MFMA wrappers and the
// per-format unpack of packed weight codes into FP16 MFMA operands.
//
// Every unpack path is exact: INT4 codes (c - 8), E4M3 values and E2M1 x E4M3
// block-scale products are all representable in FP16, so the contraction runs
// on FP16 MFMA with FP32 accumulation.  Where the INT4 / FP8 scales enter
// (on the FP32 partial sums in the decode GEMM, folded into the FP16 weight
// operand in the prefill GEMM) is described with the GEMMs.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mq {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

enum Fmt { FMT_INT4 = 1, FMT_FP8 = 2, FMT_NVFP4 = 3 };

__device__ __forceinline__ f4 mfma16(const h8 &a, const h8 &b, const f4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f16v mfma32(const h8 &a, const h8 &b, const f16v &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ h2 as_h2(uint32_t x) { return __builtin_bit_cast(h2, x); }
__device__ __forceinline__ uint32_t as_u32(h2 x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ h8 as_h8(u4 x) { return __builtin_bit_cast(h8, x); }
__device__ __forceinline__ u4 as_u4(h8 x) { return __builtin_bit_cast(u4, x); }

// ---------------------------------------------------------------- INT4
// One 32-bit word holds the 8 nibbles of k = 0..7 (k even in the low nibble of
// each byte, so nibble i sits at bits 4i).  OR-ing a masked nibble into the
// FP16 pattern of 1024.0 gives an exact FP16 integer:
//   (w      & 0x000F000F) | 0x6400 6400 -> (1024 + c0,    1024 + c4)
//   (w      & 0x00F000F0) | 0x6400 6400 -> (1024 + 16 c1, 1024 + 16 c5)
//   (w >> 8 & 0x000F000F) | ...          -> (1024 + c2,    1024 + c6)
//   (w >> 8 & 0x00F000F0) | ...          -> (1024 + 16 c3, 1024 + 16 c7)
// (1024 + 16 c <= 1264 keeps the exponent of 1024, ulp 1).  Then
// x - 1032 = c - 8 and x / 16 - 72 = c - 8, both exact in one packed op.
// The operand order is therefore k = {0,4,1,5,2,6,3,7}; the activation
// operand is stored or permuted to match (perm_0415 below).  9 VALU ops per
// 8 weights: 1 shift, 4 and-or, 4 packed FP16 add/fma.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t bits) {
  uint32_t r;
  // VOP3 on gfx9 takes no literal constants: keep mask and bits in registers
  // so this stays one instruction instead of v_and + v_or.
  asm volatile("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(mask), "v"(bits));
  return r;
}
__device__ __forceinline__ h8 unpack_int4(uint32_t w) {
  const uint32_t m_lo = 0x000F000Fu, m_hi = 0x00F000F0u, magic = 0x64006400u;
  const h2 off = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const h2 off16 = {(_Float16)-72.0f, (_Float16)-72.0f};
  const uint32_t v = w >> 8;
  const h2 p0 = as_h2(and_or(w, m_lo, magic)) + off;
  const h2 p1 = __builtin_elementwise_fma(as_h2(and_or(w, m_hi, magic)), sixteenth, off16);
  const h2 p2 = as_h2(and_or(v, m_lo, magic)) + off;
  const h2 p3 = __builtin_elementwise_fma(as_h2(and_or(v, m_hi, magic)), sixteenth, off16);
  u4 r = {as_u32(p0), as_u32(p1), as_u32(p2), as_u32(p3)};
  return as_h8(r);
}

// Reorder 8 consecutive FP16 values x0..x7 into x0,x4,x1,x5,x2,x6,x3,x7.
__device__ __forceinline__ u4 perm_0415(u4 d) {
  u4 r;
  r.x = __builtin_amdgcn_perm(d.z, d.x, 0x05040100u);  // (x0, x4)
  r.y = __builtin_amdgcn_perm(d.z, d.x, 0x07060302u);  // (x1, x5)
  r.z = __builtin_amdgcn_perm(d.w, d.y, 0x05040100u);  // (x2, x6)
  r.w = __builtin_amdgcn_perm(d.w, d.y, 0x07060302u);  // (x3, x7)
  return r;
}

// ---------------------------------------------------------------- FP8 E4M3
// gfx950 converts two OCP E4M3FN bytes to two FP16 values in one instruction;
// with a scale of 2^0 the conversion is exact (every E4M3 value is an FP16
// value).  w0 holds k = 0..3, w1 k = 4..7 (natural order).
template <bool kHiWord>
__device__ __forceinline__ h2 e4m3x2_to_h2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, kHiWord);
}
__device__ __forceinline__ h8 unpack_fp8(uint32_t w0, uint32_t w1) {
  u4 r = {as_u32(e4m3x2_to_h2<false>(w0)), as_u32(e4m3x2_to_h2<true>(w0)),
          as_u32(e4m3x2_to_h2<false>(w1)), as_u32(e4m3x2_to_h2<true>(w1))};
  return as_h8(r);
}

// ---------------------------------------------------------------- NVFP4
// Two E2M1 nibbles of one byte -> two FP16 values (low nibble first), exact.
__device__ __forceinline__ h2 e2m1x2_to_h2(uint32_t w, int byte_sel) {
  switch (byte_sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  }
}
// Value of one E4M3FN scale byte as FP16 (exact).
__device__ __forceinline__ _Float16 e4m3_to_f16(uint32_t byte) {
  return e4m3x2_to_h2<false>(byte & 0xFFu).x;
}
// 8 nibbles (k = 0..7, natural order) times their block scale s, exact in FP16
// (an E2M1 value has at most 2 significant bits, an E4M3 value 4, and
// |product| <= 6 * 448).
__device__ __forceinline__ h8 unpack_nvfp4(uint32_t w, _Float16 s) {
  const h2 ss = {s, s};
  u4 r = {as_u32(e2m1x2_to_h2(w, 0) * ss), as_u32(e2m1x2_to_h2(w, 1) * ss),
          as_u32(e2m1x2_to_h2(w, 2) * ss), as_u32(e2m1x2_to_h2(w, 3) * ss)};
  return as_h8(r);
}

// ---------------------------------------------------------------- FP8 activations
// Dynamic 1x128 FP8 activation quantization (the W8A8 variant of the FP8
// layer: the "clef-omni-fp8" card, table "What was quantized", runs its
// activations as dynamic FP8 per 1x128 group in engines).  For a group of 128
// values with maximum magnitude m: s = m / 448 (one IEEE FP32 division; m = 0
// gives s = 1 and zero codes) and code = RNE-to-E4M3(v / s), the quotient
// clamped to +-448 first (one IEEE FP32 division per value).  gfx950's
// v_cvt_pk_fp8_f32 encodes OCP E4M3FN with round-to-nearest-even.
__device__ __forceinline__ float fp8_group_scale(float amax) { return amax > 0.f ? amax / 448.f : 1.f; }
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d, float s) {
  const float qa = fminf(fmaxf(a / s, -448.f), 448.f), qb = fminf(fmaxf(b / s, -448.f), 448.f);
  const float qc = fminf(fmaxf(c / s, -448.f), 448.f), qd = fminf(fmaxf(d / s, -448.f), 448.f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(qa, qb, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(qc, qd, w, true);
  return (uint32_t)w;
}

// ---------------------------------------------------------------- NVFP4 activations
// The W4A4 variant of the NVFP4 layer quantizes activations the way the
// weights are quantized: E2M1 values, one E4M3 scale per 16 consecutive
// values, and one FP32 global scale g per projection input, a calibrated
// constant ("clef-flash-NVFP4-Hybrid" card, section "Quantization details").
// For a group with maximum magnitude m:
//   s    = RNE-to-E4M3(min((m * g) / 6, 448))  (FP32 multiply, IEEE division)
//   code = RNE-to-E2M1((x * g) / s)            (FP32 multiply, IEEE division,
//                                               saturated to +-6; s = 0: 0)
// The GEMMs multiply e2m1(code) * s, an exact FP16 number (at most 2 + 4
// significant bits, magnitude within [2^-10, 6 * 448]), and apply 1 / g to
// their FP32 sums.
struct Nvfp4Scale {
  uint32_t code;  // E4M3FN bits
  float s;        // its value
};
__device__ __forceinline__ Nvfp4Scale nvfp4_act_scale(float amax, float g) {
  const float u = fminf((amax * g) / 6.f, 448.f);
  const uint32_t c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(u, 0.f, 0, false) & 0xFFu;
  return {c, (float)e4m3_to_f16(c)};
}
// E2M1 code of (x * g) / s: the magnitude is the count of rounding boundaries
// below |q| (the midpoints of the grid 0, 0.5, 1, 1.5, 2, 3, 4, 6), each tie
// going to the even code; the sign is q's sign bit.
__device__ __forceinline__ uint32_t e2m1_code(float x, float g, float s) {
  if (s == 0.f) return 0u;
  const float q = (x * g) / s;
  const float a = fminf(fabsf(q), 6.f);
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                     (uint32_t)(a > 5.f);
  return c | ((__float_as_uint(q) >> 28) & 8u);
}
// Value of an E2M1 code as FP32.
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t m = c & 7u;
  const float a = m < 4u ? 0.5f * (float)m : m < 6u ? (float)(m - 2u) : m == 6u ? 4.f : 6.f;
  return (c & 8u) ? -a : a;
}

// ---------------------------------------------------------------- misc
// silu(z) = z / (1 + e^-z); the reciprocal is the hardware one (1 ulp), which
// is far below the FP16 rounding of the SwiGLU intermediate it feeds.
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// float -> bfloat16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
  return __builtin_bit_cast(float, b << 16);
}

// Power-of-two row scaling of BF16 activations into FP16: the shift s puts
// max|x| * 2^-s into [2^14, 2^15) (clamped to [-120, 120] so 2^+-s stay normal
// FP32 numbers); then every BF16 value above max * 2^-31 is exact in FP16.
__device__ __forceinline__ int row_shift(float m) {
  if (!(m > 0.f)) return 0;
  const int ex = (int)((__builtin_bit_cast(uint32_t, m) >> 23) & 0xFF) - 127;
  const int sh = ex - 14;
  return sh < -120 ? -120 : (sh > 120 ? 120 : sh);
}
__device__ __forceinline__ float pow2f(int s) {
  return __builtin_bit_cast(float, (uint32_t)(127 + s) << 23);
}
// 8 BF16 values (bits) times a power of two -> 8 FP16 values.
__device__ __forceinline__ u4 bf16x8_to_f16x8(u4 v, float scale) {
  u4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    h2 hh = {(_Float16)(bf16_to_f32(v[q] & 0xFFFFu) * scale),
             (_Float16)(bf16_to_f32(v[q] >> 16) * scale)};
    o[q] = as_u32(hh);
  }
  return o;
}
__device__ __forceinline__ float absmax_bf16x8(u4 v, float m) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    m = fmaxf(m, fabsf(bf16_to_f32(v[q] & 0xFFFFu)));
    m = fmaxf(m, fabsf(bf16_to_f32(v[q] >> 16)));
  }
  return m;
}

}  // namespace mq

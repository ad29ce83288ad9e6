// Device helpers for gfx950 (CDNA4): vector types, MFMA wrappers and the
// per-format unpack of packed weight codes into FP16 MFMA operands.
//
// Every unpack path is exact: INT4 codes (c - 8), E4M3 values and E2M1 x E4M3
// block-scale products are all representable in FP16, so the contraction runs
// on FP16 MFMA with FP32 accumulation and only the FP32 scales round.
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
// each byte, so nibble i sits at bits 4i).  Masking bits {4i, 16+4i} and OR-ing
// the FP16 pattern of 1024.0 yields the pair (1024 + c_i, 1024 + c_{i+4});
// subtracting 1032 gives (c - 8) exactly.  The operand order is therefore
// k = {0,4,1,5,2,6,3,7}; the activation operand is permuted to match
// (perm_0415 below).
__device__ __forceinline__ h8 unpack_int4(uint32_t w) {
  const h2 off = {(_Float16)1032.0f, (_Float16)1032.0f};
  h2 p0 = as_h2((w & 0x000F000Fu) | 0x64006400u) - off;
  h2 p1 = as_h2(((w >> 4) & 0x000F000Fu) | 0x64006400u) - off;
  h2 p2 = as_h2(((w >> 8) & 0x000F000Fu) | 0x64006400u) - off;
  h2 p3 = as_h2(((w >> 12) & 0x000F000Fu) | 0x64006400u) - off;
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

// ---------------------------------------------------------------- misc
__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

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

template <typename T>
__device__ __forceinline__ T ld_nt(const T *p) {
  return __builtin_nontemporal_load(p);
}

}  // namespace mq

// Grouped expert GEMMs with the dequantization fused into the weight-operand
// load, the SwiGLU epilogue of the gate/up projection, the routing-weighted
// epilogue of the down projection, and the slot-ordered combine.
//
// The model cards run the selected experts of a layer as one "dequantize +
// grouped matmul" ("clef-omni-fp8" card, section "How this checkpoint runs";
// "clef-omni-int4" card, section "How this checkpoint runs"; "clef-omni-NVFP4"
// card, section "How it was made").  Here the dequantization never leaves the
// chip: packed codes are unpacked exactly into FP16 MFMA operands, INT4 group
// scales and FP8 block scales multiply the FP32 partial sum of each 128-wide k
// block, and the NVFP4 global scale multiplies the finished sum.
//
// Operand roles (both kernels): the MFMA A operand is activations (rows =
// grouped tokens), the B operand is weights (columns = output features).  A
// lane therefore owns one output column, so a per-column scale is one scalar
// per lane.
#include "device.h"
#include "internal.h"

namespace mq {

struct GemmArgs {
  const uint8_t *w;
  const void *scale;
  const float *gscale;
  int N, K;  // weight matrix [N, K] per expert
  int E, I, H, k;
  const int32_t *active, *offsets, *mtile, *sorted_slots;
  const _Float16 *a_src;  // x16 [T, H] (gate/up) or h [R, I] (down)
  const float *rowscale;  // gate/up: 2^s_t per token
  const float *topk_w;    // down: routing weight per slot
  _Float16 *h_out;        // gate/up output
  float *partial;         // down output [R, H] indexed by slot
  uint32_t *flags;
  int tiles;              // decode: column tiles per expert; prefill: N tiles
};

constexpr int kDecodeKC = 2048;  // k chunk of the activation rows kept in LDS

__device__ __forceinline__ void store_h(const GemmArgs &a, int r, int col, float g, float u) {
  float hv = silu(g) * u;
  if (fabsf(hv) > 65504.f) {
    atomicOr(a.flags, 1u);
    hv = hv > 0.f ? 65504.f : -65504.f;
  }
  a.h_out[(size_t)r * a.I + col] = (_Float16)hv;
}

// ===========================================================================
// Decode path: few rows per expert.  The weights are streamed once from HBM
// straight into MFMA B-operand registers (no LDS round trip); the <= 16 rows
// of one expert sit in LDS and feed the A operand of 16x16x32 MFMAs.
//   lane l: output column n = l % 16, k slice q = l / 16.
//   group g (128 k): lane reads 32 consecutive k of its weight row,
//   k = 128 g + 32 q + [0, 32), and MFMA j in 0..3 consumes k + 8 j + [0, 8).
// Each wave owns two 16-column tiles (gate + matching up columns, or two
// adjacent down columns); KSPLIT waves split the k groups of one tile pair.
// ===========================================================================
template <int FMT>
struct DecodeFrag {
  u4 w[2];
  u4 w2[2];
  float s[2];
  uint32_t sb[2];
};

template <int FMT, int STAGE>
__device__ __forceinline__ void stage_rows(_Float16 *As, int lda, const GemmArgs &a, int rbeg,
                                           int nrows, int kc, int kcn) {
  const int cpr = kcn >> 3;
  for (int idx = threadIdx.x; idx < 16 * cpr; idx += 256) {
    const int m = idx / cpr, c = idx - m * cpr;
    u4 v = {0u, 0u, 0u, 0u};
    if (m < nrows) {
      const _Float16 *src;
      if (STAGE == 0)
        src = a.a_src + (size_t)(a.sorted_slots[rbeg + m] / a.k) * a.K + kc + c * 8;
      else
        src = a.a_src + (size_t)(rbeg + m) * a.K + kc + c * 8;
      v = *(const u4 *)src;
      if (FMT == FMT_INT4) v = perm_0415(v);
    }
    *(u4 *)(As + m * lda + c * 8) = v;
  }
}

template <int FMT, int STAGE, int KSPLIT>
__global__ __launch_bounds__(256) void gemm_decode(GemmArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int CG = 4 / KSPLIT;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int cg = wave / KSPLIT, kp = wave % KSPLIT;
  const int slot_idx = blockIdx.x / a.tiles, tile = blockIdx.x % a.tiles;
  if (slot_idx >= a.active[0]) return;
  const int e = a.active[1 + slot_idx];
  const int r0 = a.offsets[e], ne = a.offsets[e + 1] - r0;
  const int K = a.K, N = a.N, G = K / 128;
  const int KC = K < kDecodeKC ? K : kDecodeKC;
  const int lda = KC + 8;
  _Float16 *As = (_Float16 *)smem;
  float *red = (float *)(smem + (size_t)16 * lda * 2);
  const int q = lane >> 4, nl = lane & 15;

  int row[2];
  if (STAGE == 0) {
    const int n0 = (tile * CG + cg) * 16;
    row[0] = n0 + nl;
    row[1] = a.I + n0 + nl;
  } else {
    const int n0 = (tile * CG + cg) * 32;
    row[0] = n0 + nl;
    row[1] = n0 + 16 + nl;
  }
  const size_t rowbytes = FMT == FMT_FP8 ? (size_t)K : (size_t)K / 2;
  const uint8_t *wrow[2];
  const void *srow[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    wrow[t] = a.w + ((size_t)e * N + row[t]) * rowbytes;
    if (FMT == FMT_INT4)
      srow[t] = (const _Float16 *)a.scale + ((size_t)e * N + row[t]) * G;
    else if (FMT == FMT_FP8)
      srow[t] = (const float *)a.scale + ((size_t)e * (N / 128) + row[t] / 128) * G;
    else
      srow[t] = (const uint8_t *)a.scale + ((size_t)e * N + row[t]) * (K / 16);
  }

  auto load = [&](DecodeFrag<FMT> &f, int g) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (FMT == FMT_FP8) {
        const u4 *p = (const u4 *)(wrow[t] + (size_t)g * 128 + q * 32);
        f.w[t] = ld_nt(p);
        f.w2[t] = ld_nt(p + 1);
        f.s[t] = ((const float *)srow[t])[g];
      } else {
        f.w[t] = ld_nt((const u4 *)(wrow[t] + (size_t)g * 64 + q * 16));
        if (FMT == FMT_INT4)
          f.s[t] = (float)((const _Float16 *)srow[t])[g];
        else
          f.sb[t] = *(const uint16_t *)((const uint8_t *)srow[t] + 8 * g + 2 * q);
      }
    }
  };

  for (int mc = 0; mc < ne; mc += 16) {
    f4 acc[2];
    acc[0] = f4{0.f, 0.f, 0.f, 0.f};
    acc[1] = acc[0];
    for (int kc = 0; kc < K; kc += KC) {
      const int kcn = (K - kc) < KC ? (K - kc) : KC;
      const int gb = kc / 128 + kp, ge = (kc + kcn) / 128;
      DecodeFrag<FMT> cur, nxt;
      if (gb < ge) load(cur, gb);
      __syncthreads();
      stage_rows<FMT, STAGE>(As, lda, a, r0 + mc, (ne - mc) < 16 ? (ne - mc) : 16, kc, kcn);
      __syncthreads();
      for (int g = gb; g < ge; g += KSPLIT) {
        if (g + KSPLIT < ge) load(nxt, g + KSPLIT);
        const _Float16 *ap = As + nl * lda + (g * 128 - kc) + 32 * q;
        f4 tmp[2];
        tmp[0] = f4{0.f, 0.f, 0.f, 0.f};
        tmp[1] = tmp[0];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const h8 av = *(const h8 *)(ap + 8 * j);
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            h8 bv;
            if (FMT == FMT_INT4) {
              bv = unpack_int4(cur.w[t][j]);
            } else if (FMT == FMT_FP8) {
              bv = j < 2 ? unpack_fp8(cur.w[t][2 * j], cur.w[t][2 * j + 1])
                         : unpack_fp8(cur.w2[t][2 * j - 4], cur.w2[t][2 * j - 3]);
            } else {
              bv = unpack_nvfp4(cur.w[t][j], e4m3_to_f16((cur.sb[t] >> (8 * (j >> 1))) & 0xFFu));
            }
            if (FMT == FMT_NVFP4)
              acc[t] = mfma16(av, bv, acc[t]);
            else
              tmp[t] = mfma16(av, bv, tmp[t]);
          }
        }
        if (FMT != FMT_NVFP4) {
#pragma unroll
          for (int t = 0; t < 2; ++t) acc[t] += tmp[t] * cur.s[t];
        }
        cur = nxt;
      }
    }
    if (KSPLIT > 1) {
      if (kp > 0) {
        float *rb = red + (size_t)((kp - 1) * CG + cg) * 512;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) rb[(t * 4 + i) * 64 + lane] = acc[t][i];
      }
      __syncthreads();
      if (kp == 0) {
        for (int p = 1; p < KSPLIT; ++p) {
          const float *rb = red + (size_t)((p - 1) * CG + cg) * 512;
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[t][i] += rb[(t * 4 + i) * 64 + lane];
        }
      }
    }
    if (kp == 0) {
      const float ginv = FMT == FMT_NVFP4 ? 1.0f / a.gscale[e] : 1.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = mc + 4 * q + i;
        if (m >= ne) continue;
        const int r = r0 + m;
        const int slot = a.sorted_slots[r];
        if (STAGE == 0) {
          const float rs = a.rowscale[slot / a.k] * ginv;
          store_h(a, r, row[0], acc[0][i] * rs, acc[1][i] * rs);
        } else {
          const float wt = a.topk_w[slot] * ginv;
          a.partial[(size_t)slot * a.H + row[0]] = acc[0][i] * wt;
          a.partial[(size_t)slot * a.H + row[1]] = acc[1][i] * wt;
        }
      }
    }
  }
}

// ===========================================================================
// Prefill path: tiles of 128 grouped rows x 128 weight columns x 128 k.  The
// weight tile is unpacked once into LDS and shared by the 4 waves (2 x 2, each
// 64 x 64 = 2 x 2 MFMA 32x32x16 tiles).  For the gate/up projection the block
// covers 64 gate columns and the same 64 up columns, so every lane holds the
// gate and up value of one column and SwiGLU runs in registers.
// ===========================================================================
constexpr int kBM = kPrefillBM, kBN = 128, kBK = 128, kLD = kBK + 8;

template <int FMT, int STAGE>
__global__ __launch_bounds__(256, 2) void gemm_prefill(GemmArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  _Float16 *As = (_Float16 *)smem;  // [kBM][kLD]
  _Float16 *Bs = As + kBM * kLD;    // [kBN][kLD]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int mt = blockIdx.x / a.tiles, nt = blockIdx.x % a.tiles;
  if (mt >= a.mtile[a.E]) return;
  int lo = 0, hi = a.E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.mtile[mid] <= mt) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  const int rbeg = a.offsets[e] + (mt - a.mtile[e]) * kBM;
  const int nrows = min(kBM, a.offsets[e + 1] - rbeg);
  const int K = a.K, N = a.N, G = K / 128, nK = K / kBK;
  const size_t rowbytes = FMT == FMT_FP8 ? (size_t)K : (size_t)K / 2;

  // ---- staging assignments
  const int brow = tid >> 1, bhalf = tid & 1;
  const int nb = STAGE == 0 ? nt * 64 : nt * 128;
  const int wrow_g = STAGE == 0 ? (brow < 64 ? nb + brow : a.I + nb + brow - 64) : nb + brow;
  const uint8_t *wsrc = a.w + ((size_t)e * N + wrow_g) * rowbytes;
  const uint8_t *ssrc = FMT == FMT_NVFP4
                            ? (const uint8_t *)a.scale + ((size_t)e * N + wrow_g) * (K / 16)
                            : nullptr;
  const _Float16 *asrc[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int rr = p * 16 + (tid >> 4);
    const int r = rbeg + (rr < nrows ? rr : nrows - 1);
    const size_t arow = STAGE == 0 ? (size_t)(a.sorted_slots[r] / a.k) : (size_t)r;
    asrc[p] = a.a_src + arow * K + (tid & 15) * 8;
  }
  // ---- this lane's output columns (one per 32-wide tile)
  const int j = lane & 31;
  int lrow[2], bbase[2];
#pragma unroll
  for (int tn = 0; tn < 2; ++tn) {
    if (STAGE == 0) {
      bbase[tn] = tn * 64 + wn * 32;
      lrow[tn] = (tn == 0 ? nb : a.I + nb) + wn * 32 + j;
    } else {
      bbase[tn] = wn * 64 + tn * 32;
      lrow[tn] = nb + wn * 64 + tn * 32 + j;
    }
  }

  u4 areg[8], breg[4];
  uint32_t sreg = 0;
  auto gload = [&](int ks) {
    const int kb = ks * kBK;
#pragma unroll
    for (int p = 0; p < 8; ++p) areg[p] = *(const u4 *)(asrc[p] + kb);
    if (FMT == FMT_FP8) {
      const u4 *pw = (const u4 *)(wsrc + kb + bhalf * 64);
#pragma unroll
      for (int c = 0; c < 4; ++c) breg[c] = ld_nt(pw + c);
    } else {
      const u4 *pw = (const u4 *)(wsrc + kb / 2 + bhalf * 32);
      breg[0] = ld_nt(pw);
      breg[1] = ld_nt(pw + 1);
      if (FMT == FMT_NVFP4) sreg = *(const uint32_t *)(ssrc + kb / 16 + 4 * bhalf);
    }
  };

  f16v acc[2][2];
#pragma unroll
  for (int tm = 0; tm < 2; ++tm)
#pragma unroll
    for (int tn = 0; tn < 2; ++tn)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[tm][tn][i] = 0.f;

  gload(0);
  for (int ks = 0; ks < nK; ++ks) {
    __syncthreads();
    // registers -> LDS (A permuted for INT4, B unpacked to FP16 codes)
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      u4 v = areg[p];
      if (FMT == FMT_INT4) v = perm_0415(v);
      *(u4 *)(As + (p * 16 + (tid >> 4)) * kLD + (tid & 15) * 8) = v;
    }
    _Float16 *bdst = Bs + brow * kLD + bhalf * 64;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      h8 v;
      if (FMT == FMT_INT4)
        v = unpack_int4(breg[c >> 2][c & 3]);
      else if (FMT == FMT_FP8)
        v = unpack_fp8(breg[c >> 1][(c & 1) * 2], breg[c >> 1][(c & 1) * 2 + 1]);
      else
        v = unpack_nvfp4(breg[c >> 2][c & 3], e4m3_to_f16((sreg >> (8 * (c >> 1))) & 0xFFu));
      *(h8 *)(bdst + c * 8) = v;
    }
    __syncthreads();
    if (ks + 1 < nK) gload(ks + 1);
    float sc[2] = {1.f, 1.f};
    if (FMT == FMT_INT4) {
#pragma unroll
      for (int tn = 0; tn < 2; ++tn)
        sc[tn] = (float)((const _Float16 *)a.scale)[((size_t)e * N + lrow[tn]) * G + ks];
    } else if (FMT == FMT_FP8) {
#pragma unroll
      for (int tn = 0; tn < 2; ++tn)
        sc[tn] = ((const float *)a.scale)[((size_t)e * (N / 128) + lrow[tn] / 128) * G + ks];
    }
    f16v tmp[2][2];
    if (FMT != FMT_NVFP4) {
#pragma unroll
      for (int tm = 0; tm < 2; ++tm)
#pragma unroll
        for (int tn = 0; tn < 2; ++tn)
#pragma unroll
          for (int i = 0; i < 16; ++i) tmp[tm][tn][i] = 0.f;
    }
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      const int kk = s * 16 + 8 * (lane >> 5);
      h8 av[2], bv[2];
#pragma unroll
      for (int tm = 0; tm < 2; ++tm) av[tm] = *(const h8 *)(As + (wm * 64 + tm * 32 + j) * kLD + kk);
#pragma unroll
      for (int tn = 0; tn < 2; ++tn) bv[tn] = *(const h8 *)(Bs + (bbase[tn] + j) * kLD + kk);
#pragma unroll
      for (int tm = 0; tm < 2; ++tm)
#pragma unroll
        for (int tn = 0; tn < 2; ++tn) {
          if (FMT == FMT_NVFP4)
            acc[tm][tn] = mfma32(av[tm], bv[tn], acc[tm][tn]);
          else
            tmp[tm][tn] = mfma32(av[tm], bv[tn], tmp[tm][tn]);
        }
    }
    if (FMT != FMT_NVFP4) {
#pragma unroll
      for (int tm = 0; tm < 2; ++tm)
#pragma unroll
        for (int tn = 0; tn < 2; ++tn) acc[tm][tn] += tmp[tm][tn] * sc[tn];
    }
  }

  // ---- epilogue.  32x32 accumulator layout: register v of lane l holds
  // row 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32.
  const float ginv = FMT == FMT_NVFP4 ? 1.0f / a.gscale[e] : 1.0f;
#pragma unroll
  for (int tm = 0; tm < 2; ++tm) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = wm * 64 + tm * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      if (row >= nrows) continue;
      const int r = rbeg + row;
      const int slot = a.sorted_slots[r];
      if (STAGE == 0) {
        const float rs = a.rowscale[slot / a.k] * ginv;
        store_h(a, r, lrow[0], acc[tm][0][v] * rs, acc[tm][1][v] * rs);
      } else {
        const float wt = a.topk_w[slot] * ginv;
        a.partial[(size_t)slot * a.H + lrow[0]] = acc[tm][0][v] * wt;
        a.partial[(size_t)slot * a.H + lrow[1]] = acc[tm][1][v] * wt;
      }
    }
  }
}

// ===========================================================================
// Combine: out[t] = bf16(sum_j partial[t*k + j] (+ residual[t])), slots added
// in order j = 0..k-1 so repeated runs are bit-identical.
// ===========================================================================
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ partial,
                                                      const uint16_t *__restrict__ residual,
                                                      uint16_t *__restrict__ out, int T, int H,
                                                      int k) {
  const int per_row = H / 8;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)T * per_row) return;
  const int t = (int)(idx / per_row), c = (int)(idx - (size_t)t * per_row) * 8;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int j = 0; j < k; ++j) {
    const f4 *p = (const f4 *)(partial + ((size_t)t * k + j) * H + c);
    const f4 x0 = p[0], x1 = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[i] += x0[i];
      acc[4 + i] += x1[i];
    }
  }
  if (residual) {
    const u4 rv = *(const u4 *)(residual + (size_t)t * H + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = bf16_to_f32(rv[i] & 0xFFFFu) + acc[2 * i];
      acc[2 * i + 1] = bf16_to_f32(rv[i] >> 16) + acc[2 * i + 1];
    }
  }
  u4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = (uint32_t)f32_to_bf16_rne(acc[2 * i]) | ((uint32_t)f32_to_bf16_rne(acc[2 * i + 1]) << 16);
  *(u4 *)(out + (size_t)t * H + c) = o;
}

// ===========================================================================
// Test entry: dequantize one expert matrix through the same unpack functions.
// One thread per 8 consecutive k of a row.
// ===========================================================================
template <int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t *__restrict__ w,
                                                      const void *__restrict__ scale,
                                                      const float *__restrict__ gscale, int N,
                                                      int K, int e, float *__restrict__ out) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)N * (K / 8)) return;
  const int n = (int)(idx / (K / 8)), k0 = (int)(idx % (K / 8)) * 8;
  float v[8];
  if (FMT == FMT_INT4) {
    const uint32_t word = *(const uint32_t *)(w + ((size_t)e * N + n) * (K / 2) + k0 / 2);
    const h8 c = unpack_int4(word);
    const float s = (float)((const _Float16 *)scale)[((size_t)e * N + n) * (K / 128) + k0 / 128];
    const int order[8] = {0, 4, 1, 5, 2, 6, 3, 7};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[order[i]] = (float)c[i] * s;
  } else if (FMT == FMT_FP8) {
    const uint32_t *p = (const uint32_t *)(w + ((size_t)e * N + n) * K + k0);
    const h8 c = unpack_fp8(p[0], p[1]);
    const float s = ((const float *)scale)[((size_t)e * (N / 128) + n / 128) * (K / 128) + k0 / 128];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)c[i] * s;
  } else {
    const uint32_t word = *(const uint32_t *)(w + ((size_t)e * N + n) * (K / 2) + k0 / 2);
    const uint32_t sb = ((const uint8_t *)scale)[((size_t)e * N + n) * (K / 16) + k0 / 16];
    const h8 c = unpack_nvfp4(word, e4m3_to_f16(sb));
    const float g = gscale[e];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)c[i] / g;
  }
  f4 *o = (f4 *)(out + (size_t)n * K + k0);
  o[0] = f4{v[0], v[1], v[2], v[3]};
  o[1] = f4{v[4], v[5], v[6], v[7]};
}

// ===========================================================================
// Launchers
// ===========================================================================
static GemmArgs make_args(const LayerDims &L, const FwdPtrs &P, const Workspace &W, int stage) {
  GemmArgs a;
  char *ws = P.ws;
  a.E = L.E; a.I = L.I; a.H = L.H; a.k = L.k;
  if (stage == 0) {
    a.w = L.w13; a.scale = L.s13; a.gscale = L.g13; a.N = 2 * L.I; a.K = L.H;
    a.a_src = (const _Float16 *)(ws + W.x16);
  } else {
    a.w = L.w2; a.scale = L.s2; a.gscale = L.g2; a.N = L.H; a.K = L.I;
    a.a_src = (const _Float16 *)(ws + W.h);
  }
  a.active = (const int32_t *)(ws + W.active);
  a.offsets = (const int32_t *)(ws + W.offsets);
  a.mtile = (const int32_t *)(ws + W.mtile);
  a.sorted_slots = (const int32_t *)(ws + W.sorted_slots);
  a.rowscale = (const float *)(ws + W.rowscale);
  a.topk_w = (const float *)(ws + W.topk_w);
  a.h_out = (_Float16 *)(ws + W.h);
  a.partial = (float *)(ws + W.partial);
  a.flags = (uint32_t *)(ws + W.flags);
  a.tiles = 0;
  return a;
}

template <int FMT, int STAGE, int KSPLIT>
static hipError_t run_decode(GemmArgs a, int slots, hipStream_t s) {
  constexpr int CG = 4 / KSPLIT;
  a.tiles = STAGE == 0 ? a.I / (16 * CG) : a.H / (32 * CG);
  const int KC = a.K < kDecodeKC ? a.K : kDecodeKC;
  const size_t lds = (size_t)16 * (KC + 8) * 2 + (size_t)(KSPLIT - 1) * CG * 512 * 4;
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void *)gemm_decode<FMT, STAGE, KSPLIT>,
                        hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    attr_set = true;
  }
  hipLaunchKernelGGL((gemm_decode<FMT, STAGE, KSPLIT>), dim3(slots * a.tiles), dim3(256), lds, s, a);
  return hipGetLastError();
}

template <int FMT, int STAGE>
static hipError_t run_decode_ks(GemmArgs a, int slots, hipStream_t s) {
  // split k across the waves of a block when there are too few column tiles
  // to give every SIMD work
  const long cols = STAGE == 0 ? (long)a.I / 16 : (long)a.H / 32;
  const long waves = (long)slots * cols;
  const int groups = a.K / 128;
  if (waves < 1024 && groups >= 4)
    return run_decode<FMT, STAGE, 4>(a, slots, s);
  if (waves < 2048 && groups >= 2)
    return run_decode<FMT, STAGE, 2>(a, slots, s);
  return run_decode<FMT, STAGE, 1>(a, slots, s);
}

template <int FMT, int STAGE>
static hipError_t run_prefill(GemmArgs a, int64_t R, hipStream_t s) {
  a.tiles = STAGE == 0 ? a.I / 64 : a.H / 128;
  const int64_t max_mt = R / kBM + a.E;  // >= sum_e ceil(n_e / kBM)
  const size_t lds = (size_t)(kBM + kBN) * kLD * 2;
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void *)gemm_prefill<FMT, STAGE>,
                        hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    attr_set = true;
  }
  hipLaunchKernelGGL((gemm_prefill<FMT, STAGE>), dim3((unsigned)(max_mt * a.tiles)), dim3(256), lds,
                     s, a);
  return hipGetLastError();
}

template <int STAGE>
static hipError_t dispatch(const LayerDims &L, const FwdPtrs &P, const Workspace &W, bool decode,
                           hipStream_t s) {
  GemmArgs a = make_args(L, P, W, STAGE);
  const int64_t R = (int64_t)P.T * L.k;
  const int slots = (int)(R < L.E ? R : L.E);
  if (decode) {
    switch (L.fmt) {
      case FMT_INT4: return run_decode_ks<FMT_INT4, STAGE>(a, slots, s);
      case FMT_FP8: return run_decode_ks<FMT_FP8, STAGE>(a, slots, s);
      default: return run_decode_ks<FMT_NVFP4, STAGE>(a, slots, s);
    }
  }
  switch (L.fmt) {
    case FMT_INT4: return run_prefill<FMT_INT4, STAGE>(a, R, s);
    case FMT_FP8: return run_prefill<FMT_FP8, STAGE>(a, R, s);
    default: return run_prefill<FMT_NVFP4, STAGE>(a, R, s);
  }
}

hipError_t launch_gate_up(const LayerDims &L, const FwdPtrs &P, const Workspace &W, bool decode,
                          hipStream_t s) {
  return dispatch<0>(L, P, W, decode, s);
}

hipError_t launch_down(const LayerDims &L, const FwdPtrs &P, const Workspace &W, bool decode,
                       hipStream_t s) {
  return dispatch<1>(L, P, W, decode, s);
}

hipError_t launch_combine(const LayerDims &L, const FwdPtrs &P, const Workspace &W, hipStream_t s) {
  const size_t items = (size_t)P.T * (L.H / 8);
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, s,
                     (const float *)(P.ws + W.partial), P.residual, P.out, P.T, L.H, L.k);
  return hipGetLastError();
}

hipError_t launch_dequantize(const LayerDims &L, int which, int expert, float *out, hipStream_t s) {
  const uint8_t *w = which == 0 ? L.w13 : L.w2;
  const void *sc = which == 0 ? L.s13 : L.s2;
  const float *g = which == 0 ? L.g13 : L.g2;
  const int N = which == 0 ? 2 * L.I : L.H, K = which == 0 ? L.H : L.I;
  const size_t items = (size_t)N * (K / 8);
  const dim3 grid((unsigned)((items + 255) / 256)), block(256);
  switch (L.fmt) {
    case FMT_INT4: hipLaunchKernelGGL(dequant_kernel<FMT_INT4>, grid, block, 0, s, w, sc, g, N, K, expert, out); break;
    case FMT_FP8: hipLaunchKernelGGL(dequant_kernel<FMT_FP8>, grid, block, 0, s, w, sc, g, N, K, expert, out); break;
    default: hipLaunchKernelGGL(dequant_kernel<FMT_NVFP4>, grid, block, 0, s, w, sc, g, N, K, expert, out); break;
  }
  return hipGetLastError();
}

bool use_decode_path(int64_t T, int E, int k) {
  // mean rows per expert <= 16: one 16-row MFMA block per expert on average
  return T * k <= (int64_t)16 * E;
}

}  // namespace mq

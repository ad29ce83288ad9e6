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
#include <algorithm>

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

__device__ __forceinline__ void store_h(const GemmArgs &a, int r, int col, float g, float u) {
  float hv = silu(g) * u;
  if (fabsf(hv) > 65504.f) {
    atomicOr(a.flags, 1u);
    hv = hv > 0.f ? 65504.f : -65504.f;
  }
  a.h_out[(size_t)r * a.I + col] = (_Float16)hv;
}

// ===========================================================================
// Decode path: few rows per expert.  Weights are streamed once from HBM
// straight into MFMA B-operand registers, kD groups ahead of their use; the
// <= 16 activation rows of the expert (FP16, prepared by the routing kernel)
// are copied once per unit into LDS and feed the A operand.
//   16x16x32 MFMA, lane l: output column n = l % 16, k slice q = l / 16, and
//   A row m = l % 16 (a grouped row of the expert; rows >= nrows are never
//   written to LDS and never stored: an MFMA output row depends only on its
//   own A row).  Group g (128 k): lane holds k = 128 g + 32 q + [0, 32); MFMA
//   j in 0..3 consumes k + 8 j + [0, 8).
// A block has kDecodeWaves waves: CG column-tile pairs x KSPLIT k-splits.  Each
// wave owns two 16-column tiles (gate + matching up columns, or two adjacent
// down columns); KSPLIT waves reduce their partial sums through LDS.  The grid
// is persistent: resident blocks loop over (expert, tile group) units.
// ===========================================================================
constexpr int kDecodeWaves = 8;
#ifndef MQ_DECODE_DEPTH
#define MQ_DECODE_DEPTH 4
#endif
constexpr int kD = MQ_DECODE_DEPTH;  // weight groups in flight per wave (even)
static_assert(kD % 2 == 0, "groups are prefetched in pairs");

// Registers of one group in flight.  Scales stay raw until use: a conversion
// at load time would make the compiler wait for that load, and loads retire in
// order, so it would drain every older prefetch as well.
template <int FMT>
struct DecodeFrag {
  u4 w[2];
  u4 w2[2];
  float s[2];       // FP8 block scale
  uint32_t sb[2];   // INT4: FP16 group-scale bits; NVFP4: two E4M3 block-scale bytes
};

template <int FMT, int STAGE, int KSPLIT, int GCT>
__global__ __launch_bounds__(64 * kDecodeWaves) void gemm_decode(GemmArgs a) {
  // GCT > 0: the k groups per row (K / 128) known at compile time; the group
  // loop is then fully unrolled, so every wait on a prefetch is an exact
  // count instead of the conservative merge LLVM makes at a loop header.
  constexpr int CG = kDecodeWaves / KSPLIT;
  constexpr int NGCT = GCT > 0 && GCT % KSPLIT == 0 ? GCT / KSPLIT : 0;
  extern __shared__ __align__(16) unsigned char smem[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int cg = wave / KSPLIT, kp = wave % KSPLIT;
  const int q = lane >> 4, nl = lane & 15;
  const int K = GCT > 0 ? GCT * 128 : a.K, N = a.N, G = K / 128;
  const int lda = K + 8;                                          // halves
  _Float16 *As = (_Float16 *)smem;                                // [16][lda]
  float *red = (float *)(smem + (size_t)16 * lda * 2);            // [KSPLIT-1][CG][512]
  const size_t rowbytes = FMT == FMT_FP8 ? (size_t)K : (size_t)K / 2;
  const int gb = (kp * G) / KSPLIT;                               // groups [gb, gb + ng)
  const int ng = NGCT > 0 ? NGCT : ((kp + 1) * G) / KSPLIT - gb;
  const int n_units = a.active[0] * a.tiles;

  for (int unit = blockIdx.x; unit < n_units; unit += gridDim.x) {
    const int slot_idx = unit / a.tiles, tile = unit - slot_idx * a.tiles;
    const int e = a.active[1 + slot_idx];
    const int r0 = a.offsets[e], ne = a.offsets[e + 1] - r0;
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

    // Groups g and g + 1 (if `two`), issued tile by tile so the two halves of
    // every 128-byte line of a 4-bit row are requested back to back.
    auto load_pair = [&](DecodeFrag<FMT> &fa, DecodeFrag<FMT> &fb, int g, bool two) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if (FMT == FMT_FP8) {
          const u4 *p = (const u4 *)(wrow[t] + (size_t)g * 128 + q * 32);
          fa.w[t] = ld_nt(p);
          fa.w2[t] = ld_nt(p + 1);
          if (two) {
            fb.w[t] = ld_nt(p + 8);
            fb.w2[t] = ld_nt(p + 9);
          }
        } else {
          const u4 *p = (const u4 *)(wrow[t] + (size_t)g * 64 + q * 16);
          fa.w[t] = ld_nt(p);
          if (two) fb.w[t] = ld_nt(p + 4);
        }
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if (FMT == FMT_FP8) {
          fa.s[t] = ((const float *)srow[t])[g];
          if (two) fb.s[t] = ((const float *)srow[t])[g + 1];
        } else if (FMT == FMT_INT4) {
          fa.sb[t] = ((const uint16_t *)srow[t])[g];
          if (two) fb.sb[t] = ((const uint16_t *)srow[t])[g + 1];
        } else {
          fa.sb[t] = *(const uint16_t *)((const uint8_t *)srow[t] + 8 * g + 2 * q);
          if (two) fb.sb[t] = *(const uint16_t *)((const uint8_t *)srow[t] + 8 * (g + 1) + 2 * q);
        }
      }
    };

    for (int mc = 0; mc < ne; mc += 16) {
      const int nrows = (ne - mc) < 16 ? (ne - mc) : 16;
      DecodeFrag<FMT> f[kD];
#pragma unroll
      for (int d = 0; d < kD; d += 2)
        if (d < ng) load_pair(f[d], f[d + 1], gb + d, d + 1 < ng);

      // ---- rows of this expert -> LDS (one pass; gate/up rows arrive in the
      // INT4 k order already, down rows are permuted here)
      __syncthreads();
      {
        const int cpr = K >> 3;
        for (int idx = threadIdx.x; idx < nrows * cpr; idx += 64 * kDecodeWaves) {
          const int m = idx / cpr, c = idx - m * cpr;
          const int r = r0 + mc + m;
          const size_t src_row = STAGE == 0 ? (size_t)(a.sorted_slots[r] / a.k) : (size_t)r;
          u4 v = *(const u4 *)(a.a_src + src_row * K + c * 8);
          if (FMT == FMT_INT4 && STAGE == 1) v = perm_0415(v);
          *(u4 *)(As + m * lda + c * 8) = v;
        }
      }
      __syncthreads();

      f4 acc[2];
      acc[0] = f4{0.f, 0.f, 0.f, 0.f};
      acc[1] = acc[0];
      const _Float16 *abase = As + nl * lda + 32 * q;
      auto compute = [&](const DecodeFrag<FMT> &fr, int g) {
        const _Float16 *ap = abase + g * 128;
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
              bv = unpack_int4(fr.w[t][j]);
            } else if (FMT == FMT_FP8) {
              bv = j < 2 ? unpack_fp8(fr.w[t][2 * j], fr.w[t][2 * j + 1])
                         : unpack_fp8(fr.w2[t][2 * j - 4], fr.w2[t][2 * j - 3]);
            } else {
              bv = unpack_nvfp4(fr.w[t][j], e4m3_to_f16((fr.sb[t] >> (8 * (j >> 1))) & 0xFFu));
            }
            if (FMT == FMT_NVFP4)
              acc[t] = mfma16(av, bv, acc[t]);
            else
              tmp[t] = mfma16(av, bv, tmp[t]);
          }
        }
        if (FMT == FMT_INT4) {
#pragma unroll
          for (int t = 0; t < 2; ++t)
            acc[t] += tmp[t] * (float)__builtin_bit_cast(_Float16, (uint16_t)fr.sb[t]);
        } else if (FMT == FMT_FP8) {
#pragma unroll
          for (int t = 0; t < 2; ++t) acc[t] += tmp[t] * fr.s[t];
        }
      };

      if constexpr (NGCT > 0) {
        // fully unrolled ring of kD groups
#pragma unroll
        for (int i = 0; i < NGCT; i += 2) {
          compute(f[i % kD], gb + i);
          if (i + 1 < NGCT) compute(f[(i + 1) % kD], gb + i + 1);
          if (i + kD < NGCT) {
            load_pair(f[i % kD], f[(i + 1) % kD], gb + i + kD, i + kD + 1 < NGCT);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      } else {
        // steady state: every computed pair of groups is replaced by the pair
        // kD ahead (unconditional: no register merge waits on a load)
        int i = 0;
        for (; i + 2 * kD <= ng; i += kD) {
#pragma unroll
          for (int d = 0; d < kD; d += 2) {
            compute(f[d], gb + i + d);
            compute(f[d + 1], gb + i + d + 1);
            load_pair(f[d], f[d + 1], gb + i + d + kD, true);
            // keep the prefetch here: sunk to the loop end, it would become
            // the youngest load and the next wait would drain the window
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // tail: fewer than 2 kD groups left
#pragma unroll
        for (int d = 0; d < kD; d += 2) {
          if (i + d < ng) compute(f[d], gb + i + d);
          if (i + d + 1 < ng) compute(f[d + 1], gb + i + d + 1);
          if (i + d + kD < ng) load_pair(f[d], f[d + 1], gb + i + d + kD, i + d + kD + 1 < ng);
        }
#pragma unroll
        for (int d = 0; d < kD; ++d)
          if (i + kD + d < ng) compute(f[d], gb + i + kD + d);
      }

      if (KSPLIT > 1) {
        if (kp > 0) {
          float *rb = red + (size_t)((kp - 1) * CG + cg) * 512;
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) rb[(t * 4 + ii) * 64 + lane] = acc[t][ii];
        }
        __syncthreads();
        if (kp == 0) {
          for (int p = 1; p < KSPLIT; ++p) {
            const float *rb = red + (size_t)((p - 1) * CG + cg) * 512;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
              for (int ii = 0; ii < 4; ++ii) acc[t][ii] += rb[(t * 4 + ii) * 64 + lane];
          }
        }
      }
      if (kp == 0) {
        const float ginv = FMT == FMT_NVFP4 ? 1.0f / a.gscale[e] : 1.0f;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int m = 4 * q + ii;
          if (m >= nrows) continue;
          const int r = r0 + mc + m;
          const int slot = a.sorted_slots[r];
          if (STAGE == 0) {
            const float sc = a.rowscale[slot / a.k] * ginv;
            store_h(a, r, row[0], acc[0][ii] * sc, acc[1][ii] * sc);
          } else {
            const float wt = a.topk_w[slot] * ginv;
            a.partial[(size_t)slot * a.H + row[0]] = acc[0][ii] * wt;
            a.partial[(size_t)slot * a.H + row[1]] = acc[1][ii] * wt;
          }
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
      if (FMT == FMT_INT4 && STAGE == 1) v = perm_0415(v);  // gate/up rows come INT4-ordered
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
    // scales of this k step first: the prefetch below retires after them
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
    if (ks + 1 < nK) gload(ks + 1);
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

static int g_num_cus = 0;

static int num_cus() {
  if (g_num_cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      g_num_cus = n;
    else
      g_num_cus = 256;
  }
  return g_num_cus;
}

template <int FMT, int STAGE, int KSPLIT, int GCT>
static hipError_t run_decode_g(GemmArgs a, int slots, hipStream_t s) {
  constexpr int CG = kDecodeWaves / KSPLIT;
  a.tiles = STAGE == 0 ? a.I / (16 * CG) : a.H / (32 * CG);
  const size_t lds = (size_t)16 * (a.K + 8) * 2 + (size_t)(KSPLIT - 1) * CG * 512 * 4;
  // persistent grid: as many blocks as are resident at once (from the
  // kernel's registers and LDS), never more than the number of units
  static int per_cu = 0;
  static size_t per_cu_lds = 0;
  if (per_cu == 0 || per_cu_lds != lds) {
    (void)hipFuncSetAttribute((const void *)gemm_decode<FMT, STAGE, KSPLIT, GCT>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemm_decode<FMT, STAGE, KSPLIT, GCT>,
                                                     64 * kDecodeWaves, lds) != hipSuccess || n < 1)
      n = 1;
    per_cu = n;
    per_cu_lds = lds;
  }
  const long units = (long)slots * a.tiles;
  const long grid = std::min<long>(units, (long)num_cus() * per_cu);
  hipLaunchKernelGGL((gemm_decode<FMT, STAGE, KSPLIT, GCT>), dim3((unsigned)grid),
                     dim3(64 * kDecodeWaves), lds, s, a);
  return hipGetLastError();
}

template <int FMT, int STAGE, int KSPLIT>
static hipError_t run_decode(GemmArgs a, int slots, hipStream_t s) {
  switch (a.K / 128) {  // k groups per row; unrolled variants for common sizes
    case 4: return run_decode_g<FMT, STAGE, KSPLIT, 4>(a, slots, s);
    case 6: return run_decode_g<FMT, STAGE, KSPLIT, 6>(a, slots, s);
    case 8: return run_decode_g<FMT, STAGE, KSPLIT, 8>(a, slots, s);
    case 12: return run_decode_g<FMT, STAGE, KSPLIT, 12>(a, slots, s);
    case 16: return run_decode_g<FMT, STAGE, KSPLIT, 16>(a, slots, s);
    case 32: return run_decode_g<FMT, STAGE, KSPLIT, 32>(a, slots, s);
    default: return run_decode_g<FMT, STAGE, KSPLIT, 0>(a, slots, s);
  }
}

template <int FMT, int STAGE>
static hipError_t run_decode_ks(GemmArgs a, int slots, hipStream_t s) {
  // Smallest k split whose column groups tile the expert exactly and whose
  // wave-tasks (tile pair x k split) cover the resident waves about twice.
  const int cols = STAGE == 0 ? a.I / 16 : a.H / 32;  // tile pairs per expert
  const long waves = (long)num_cus() * 16;
  const int ksplits[4] = {1, 2, 4, 8};
  int pick = 8;
  for (int ks : ksplits) {
    if (cols % (kDecodeWaves / ks) != 0) continue;
    if ((long)slots * cols * ks >= 2 * waves) {
      pick = ks;
      break;
    }
  }
  switch (pick) {
    case 1: return run_decode<FMT, STAGE, 1>(a, slots, s);
    case 2: return run_decode<FMT, STAGE, 2>(a, slots, s);
    case 4: return run_decode<FMT, STAGE, 4>(a, slots, s);
    default: return run_decode<FMT, STAGE, 8>(a, slots, s);
  }
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

bool use_decode_path(int64_t T, int E, int k, int H, int I) {
  // mean rows per expert <= 16: one 16-row MFMA block per expert on average
  (void)H;
  (void)I;
  return T * k <= (int64_t)16 * E;
}

}  // namespace mq

// Grouped expert GEMMs with the dequantization fused into the weight-operand
// load, the SwiGLU epilogue of the gate/up projection, the routing-weighted
// epilogue of the down projection, and the slot-ordered combine.
//
// The model cards run the selected experts of a layer as one "dequantize +
// grouped matmul" ("clef-omni-fp8" card, section "How this checkpoint runs";
// "clef-omni-int4" card, section "How this checkpoint runs"; "clef-omni-NVFP4"
// card, section "How it was made").  Here the dequantization never leaves the
// chip: packed codes are unpacked exactly into FP16 MFMA operands, and the
// NVFP4 global scale multiplies the finished FP32 sum.  The INT4 group scales
// and FP8 block scales are applied differently by the two paths:
//  - decode: they multiply the FP32 partial sum of each 128-wide k block (one
//    FP32 rounding per block);
//  - prefill: each is folded into the FP16 weight operand together with a
//    power of two per weight column (the FP32 scale rounded to FP16, then the
//    product code * scale rounded to FP16: at most about 2^-11 relative per
//    weight beside the FP16 scale's own 2^-11), and the column's accumulator
//    is multiplied back by the power of two at the end.
//
// Operand roles: the decode MFMA takes activations as its A operand (rows =
// grouped tokens) and weights as B (columns = output features), so a lane
// owns one output column and a per-column scale is one scalar per lane; the
// prefill MFMA takes them the other way round (C[n][m], weights as A), so a
// lane ends with four consecutive output columns of one grouped row.
#include <algorithm>
#include <map>
#include <mutex>
#include <set>
#include <tuple>
#include <type_traits>

#include <hip/hip_ext.h>

#include "device.h"
#include "internal.h"

namespace mq {

struct GemmArgs {
  const uint8_t *w;
  const void *scale;
  const float *gscale;
  int N, K;  // weight matrix [N, K] per expert
  int E, I, H, k;
  int T;                // tokens
  const int4 *einfo;    // {count, 16-row chunks}, then {expert, first grouped row, rows, 0} per active expert
  const int32_t *rcp;   // per active expert, prefix of the 16-row chunks; then the total
  const int4 *rowinfo;  // per grouped row: {slot, token, row scale bits, routing weight bits}
  const int32_t *offsets, *mtile;
  const _Float16 *a_src;  // prefill: x16 [T, H] (gate/up) or h [R, I] (down); decode: h
  const uint16_t *hidden; // BF16 [T, H]: the decode gate/up scales its rows itself
  _Float16 *h_out;        // gate/up output
  _Float16 *partial;      // down output [R, H] indexed by slot (FP16, routing-weighted)
  uint32_t *flags;
  int tiles;              // decode: column tiles per expert; prefill: N tiles
  float hq_g;             // W4A4 gate/up: global scale of the NVFP4 quantization of h
  float a_inv;            // down: factor on the sums (W4A4: 1 / the global scale of h; else 1)
  int rc_off;             // decode: byte offset in dynamic LDS of the 16-row-chunk table
                          // (units are 16-row chunks); 0: units are whole experts
  // decode down projection with the combine fused in (a few tokens)
  const int32_t *slot_ids;   // [T k]: expert of slot (t, j)
  const int32_t *slot_pos;   // [T k]: grouped row of slot (t, j)
  const float *slot_w;       // [T k]: routing weight of slot (t, j)
  const uint16_t *residual;  // BF16 [T, H] or null
  uint16_t *out;             // BF16 [T, H]
};

// Saturate to the FP16 range, remembering whether anything was clamped.
__device__ __forceinline__ _Float16 to_f16_sat(float v, uint32_t &sat) {
  const float c = fminf(fmaxf(v, -65504.f), 65504.f);
  sat |= c != v;
  return (_Float16)c;
}

// SwiGLU of one (gate, up) pair into the FP16 intermediate; `sat` remembers a
// clamp (the caller sets the flag word once per wave).
__device__ __forceinline__ void store_h(const GemmArgs &a, int r, int col, float g, float u,
                                        uint32_t &sat) {
  a.h_out[(size_t)r * a.I + col] = to_f16_sat(silu(g) * u, sat);
}

// One flag-word update per wave that saw a saturated value (every lane of the
// wave must reach this call).
__device__ __forceinline__ void flag_saturation(const GemmArgs &a, uint32_t sat) {
  if (__builtin_amdgcn_ballot_w64(sat != 0u) != 0ull && (threadIdx.x & 63) == 0) atomicOr(a.flags, 1u);
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
// is persistent: resident blocks loop over (16-row chunk of an expert's rows,
// tile group) units, so an expert with many rows spreads over many blocks.
// ===========================================================================
constexpr int kDecodeWaves = 8;
constexpr int kD = 4;  // weight groups in flight per wave (even; 6 and 8 measured slower)
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

template <int FMT, int STAGE, int KSPLIT, int GCT, int TPW>
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
  uint32_t *sm_rmax = (uint32_t *)(smem + (size_t)16 * lda * 2);  // [16] row max |x| bits
  float *sm_rscale = (float *)(sm_rmax + 16);                     // [2][16]: 2^s, 2^-s
  float *red = sm_rscale + 32;                                    // [KSPLIT-1][CG][512]
  const size_t rowbytes = FMT == FMT_FP8 ? (size_t)K : (size_t)K / 2;
  const int gb = (kp * G) / KSPLIT;                               // groups [gb, gb + ng)
  const int ng = NGCT > 0 ? NGCT : ((kp + 1) * G) / KSPLIT - gb;
  // Units are whole experts, or, when some expert holds more than 16 rows
  // (more 16-row chunks than active experts) and the launch has room for it,
  // 16-row chunks, through a table in LDS: the grouping's prefix of the active
  // experts' chunks [n_act + 1], then the active-expert records [n_act] (from
  // offset 16 * ceil((E + 1) / 4)).
  const int4 hdr = a.einfo[0];
  const int n_act = hdr.x;
  int *rcpre = a.rc_off && hdr.y > hdr.x ? (int *)(smem + a.rc_off) : nullptr;  // block-uniform
  int4 *einf = (int4 *)(smem + a.rc_off + 16 * ((a.E + 4) / 4));
  if (rcpre) {
    for (int i = threadIdx.x; i <= n_act; i += 64 * kDecodeWaves) {
      if (i < n_act) einf[i] = a.einfo[1 + i];
      rcpre[i] = a.rcp[i];
    }
    __syncthreads();
  }
  const int n_units = (rcpre ? rcpre[n_act] : n_act) * a.tiles;
  // TPW > 1 (down projection with few k groups): each wave streams TPW tile
  // pairs of the unit in one ring, so a unit's ring fill and drain cover more
  // weight bytes
  static_assert(TPW == 1 || (NGCT > 0 && NGCT % 2 == 0 && KSPLIT == 1), "pairs of groups stay in one tile pair");
  constexpr int NGT = NGCT * TPW;  // groups of the wave's ring (unrolled case)

  for (int unit = blockIdx.x; unit < n_units; unit += gridDim.x) {
    const int ui = unit / a.tiles, tile = unit - ui * a.tiles;
    int slot_idx = ui, mcg = 0;
    if (rcpre) {  // ui is a 16-row chunk: find the active expert that holds it
      // (every expert has at least one chunk, so it is at or before slot ui;
      // with up to 16 rows per expert it is slot ui itself)
      int lo = min(ui, n_act - 1);
      int pre = rcpre[lo];
      while (pre > ui) pre = rcpre[--lo];
      slot_idx = lo;
      mcg = ui - pre;
    }
    const int4 ei = rcpre ? einf[slot_idx] : a.einfo[1 + slot_idx];
    // the unit's rows: chunk mcg of the expert (the row loop below then runs
    // once), or all of them
    const int e = ei.x, r0 = ei.y + 16 * mcg, ne = rcpre ? min(16, ei.z - 16 * mcg) : ei.z;
    int row[TPW][2];
#pragma unroll
    for (int p = 0; p < TPW; ++p) {
      if (STAGE == 0) {
        const int n0 = ((tile * TPW + p) * CG + cg) * 16;
        row[p][0] = n0 + nl;
        row[p][1] = a.I + n0 + nl;
      } else {
        const int n0 = ((tile * TPW + p) * CG + cg) * 32;
        row[p][0] = n0 + nl;
        row[p][1] = n0 + 16 + nl;
      }
    }
    const uint8_t *wrow[TPW][2];
    const void *srow[TPW][2];
#pragma unroll
    for (int p = 0; p < TPW; ++p)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        wrow[p][t] = a.w + ((size_t)e * N + row[p][t]) * rowbytes;
        if (FMT == FMT_INT4)
          srow[p][t] = (const _Float16 *)a.scale + ((size_t)e * N + row[p][t]) * G;
        else if (FMT == FMT_FP8)
          srow[p][t] = (const float *)a.scale + ((size_t)e * (N / 128) + row[p][t] / 128) * G;
        else
          srow[p][t] = (const uint8_t *)a.scale + ((size_t)e * N + row[p][t]) * (K / 16);
      }

    // Groups g and g + 1 (if `two`), issued tile by tile so the two halves of
    // every 128-byte line of a 4-bit row are requested back to back.  Plain
    // (cached) loads: measured faster than non-temporal ones here, as the
    // second half of a line then finds the first's fill in L2.
    auto load_pair_p = [&](DecodeFrag<FMT> &fa, DecodeFrag<FMT> &fb, int pp, int g, bool two) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if (FMT == FMT_FP8) {
          const u4 *p = (const u4 *)(wrow[pp][t] + (size_t)g * 128 + q * 32);
          fa.w[t] = p[0];
          fa.w2[t] = p[1];
          if (two) {
            fb.w[t] = p[8];
            fb.w2[t] = p[9];
          }
        } else {
          const u4 *p = (const u4 *)(wrow[pp][t] + (size_t)g * 64 + q * 16);
          fa.w[t] = p[0];
          if (two) fb.w[t] = p[4];
        }
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if (FMT == FMT_FP8) {
          fa.s[t] = ((const float *)srow[pp][t])[g];
          if (two) fb.s[t] = ((const float *)srow[pp][t])[g + 1];
        } else if (FMT == FMT_INT4) {
          fa.sb[t] = ((const uint16_t *)srow[pp][t])[g];
          if (two) fb.sb[t] = ((const uint16_t *)srow[pp][t])[g + 1];
        } else {
          fa.sb[t] = *(const uint16_t *)((const uint8_t *)srow[pp][t] + 8 * g + 2 * q);
          if (two) fb.sb[t] = *(const uint16_t *)((const uint8_t *)srow[pp][t] + 8 * (g + 1) + 2 * q);
        }
      }
    };
    // ring position i -> (tile pair i / NGCT, group i % NGCT) when unrolled
    auto load_pair = [&](DecodeFrag<FMT> &fa, DecodeFrag<FMT> &fb, int i, bool two) {
      if (TPW == 1)
        load_pair_p(fa, fb, 0, i, two);
      else
        load_pair_p(fa, fb, i / NGCT, i % NGCT, two);
    };

    for (int mc = 0; mc < ne; mc += 16) {
      const int nrows = (ne - mc) < 16 ? (ne - mc) : 16;
      DecodeFrag<FMT> f[kD];
#pragma unroll
      for (int d = 0; d < kD; d += 2)
        if (d < ng * TPW) load_pair(f[d], f[d + 1], gb + d, d + 1 < ng * TPW);
      // per-row records of the rows this lane stores (issued early; read in
      // the epilogue)
      int4 rinf[4];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int m = 4 * q + ii;
        rinf[ii] = m < nrows ? a.rowinfo[r0 + mc + m] : int4{0, 0, 0, 0};
      }

      // ---- rows of this expert -> LDS.  Gate/up: the tokens' BF16 hidden
      // rows, each scaled by a power of two into FP16 (max |x| of the row into
      // [2^14, 2^15), so every BF16 value above max * 2^-31 converts exactly)
      // and stored in the INT4 k order for INT4; the epilogue multiplies the
      // row back.  For rows of up to 2048 values the routing kernel has found
      // each row's power of two; longer rows are scanned here first.  Down:
      // the grouped FP16 intermediate rows (permuted here for INT4).
      __syncthreads();
      if (STAGE == 0 && K <= kRowRegsMaxH) {
        // the routing kernel left each row's power of two 2^s in its record
        // (row scale bits); convert with the exact inverse 2^-s
        const int cpr = K >> 3;
        for (int idx = threadIdx.x; idx < nrows * cpr; idx += 64 * kDecodeWaves) {
          const int m = idx / cpr, c = idx - m * cpr;
          const int4 ri = a.rowinfo[r0 + mc + m];
          const float down = __builtin_bit_cast(float, (uint32_t)(254u << 23) - (uint32_t)ri.z);
          u4 v = bf16x8_to_f16x8(*(const u4 *)(a.hidden + (size_t)ri.y * K + c * 8), down);
          if (FMT == FMT_INT4) v = perm_0415(v);
          *(u4 *)(As + m * lda + c * 8) = v;
        }
        if (threadIdx.x < nrows) sm_rscale[threadIdx.x] = __builtin_bit_cast(float, a.rowinfo[r0 + mc + threadIdx.x].z);
      } else {
        const int cpr = K >> 3;
        if (STAGE == 0) {
          if (threadIdx.x < 16) sm_rmax[threadIdx.x] = 0u;
          __syncthreads();
          for (int idx = threadIdx.x; idx < nrows * cpr; idx += 64 * kDecodeWaves) {
            const int m = idx / cpr, c = idx - m * cpr;
            const u4 v = *(const u4 *)(a.hidden + (size_t)a.rowinfo[r0 + mc + m].y * K + c * 8);
            atomicMax(&sm_rmax[m], __builtin_bit_cast(uint32_t, absmax_bf16x8(v, 0.f)));
          }
          __syncthreads();
          if (threadIdx.x < nrows) {
            const int sh = row_shift(__builtin_bit_cast(float, sm_rmax[threadIdx.x]));
            sm_rscale[threadIdx.x] = pow2f(sh);
            sm_rscale[16 + threadIdx.x] = pow2f(-sh);
          }
          __syncthreads();
        }
        for (int idx = threadIdx.x; idx < nrows * cpr; idx += 64 * kDecodeWaves) {
          const int m = idx / cpr, c = idx - m * cpr;
          const int r = r0 + mc + m;
          u4 v;
          if (STAGE == 0) {
            v = bf16x8_to_f16x8(*(const u4 *)(a.hidden + (size_t)a.rowinfo[r].y * K + c * 8),
                                sm_rscale[16 + m]);
            if (FMT == FMT_INT4) v = perm_0415(v);
          } else {
            v = *(const u4 *)(a.a_src + (size_t)r * K + c * 8);
            if (FMT == FMT_INT4) v = perm_0415(v);
          }
          *(u4 *)(As + m * lda + c * 8) = v;
        }
      }
      __syncthreads();

      f4 acc[TPW][2];
#pragma unroll
      for (int p = 0; p < TPW; ++p) acc[p][0] = acc[p][1] = f4{0.f, 0.f, 0.f, 0.f};
      const _Float16 *abase = As + nl * lda + 32 * q;
      // ring position i: group i of tile pair 0, or with TPW > 1 group i % NGCT
      // of tile pair i / NGCT (constants once the ring is unrolled)
      auto compute = [&](const DecodeFrag<FMT> &fr, int i) {
        const int pp = TPW == 1 ? 0 : i / NGCT, g = TPW == 1 ? i : i % NGCT;
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
              acc[pp][t] = mfma16(av, bv, acc[pp][t]);
            else
              tmp[t] = mfma16(av, bv, tmp[t]);
          }
        }
        if (FMT == FMT_INT4) {
#pragma unroll
          for (int t = 0; t < 2; ++t)
            acc[pp][t] += tmp[t] * (float)__builtin_bit_cast(_Float16, (uint16_t)fr.sb[t]);
        } else if (FMT == FMT_FP8) {
#pragma unroll
          for (int t = 0; t < 2; ++t) acc[pp][t] += tmp[t] * fr.s[t];
        }
      };

      if constexpr (NGCT > 0) {
        // fully unrolled ring of kD groups (over TPW tile pairs)
#pragma unroll
        for (int i = 0; i < NGT; i += 2) {
          compute(f[i % kD], gb + i);
          if (i + 1 < NGT) compute(f[(i + 1) % kD], gb + i + 1);
          if (i + kD < NGT) {
            load_pair(f[i % kD], f[(i + 1) % kD], gb + i + kD, i + kD + 1 < NGT);
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
            for (int ii = 0; ii < 4; ++ii) rb[(t * 4 + ii) * 64 + lane] = acc[0][t][ii];
        }
        __syncthreads();
        if (kp == 0) {
          for (int p = 1; p < KSPLIT; ++p) {
            const float *rb = red + (size_t)((p - 1) * CG + cg) * 512;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
              for (int ii = 0; ii < 4; ++ii) acc[0][t][ii] += rb[(t * 4 + ii) * 64 + lane];
          }
        }
      }
      if (kp == 0) {  // wave-uniform
        const float ginv = FMT == FMT_NVFP4 ? 1.0f / a.gscale[e] : 1.0f;
        uint32_t sat = 0u;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int m = 4 * q + ii;
          if (m >= nrows) continue;
          const int r = r0 + mc + m;
          const int slot = rinf[ii].x;
          if (STAGE == 0) {
            const float sc = sm_rscale[m] * ginv;
            store_h(a, r, row[0][0], acc[0][0][ii] * sc, acc[0][1][ii] * sc, sat);
          } else {
            const float wt = __builtin_bit_cast(float, rinf[ii].w) * ginv;
#pragma unroll
            for (int p = 0; p < TPW; ++p) {
              a.partial[(size_t)slot * a.H + row[p][0]] = to_f16_sat(acc[p][0][ii] * wt, sat);
              a.partial[(size_t)slot * a.H + row[p][1]] = to_f16_sat(acc[p][1][ii] * wt, sat);
            }
          }
        }
        flag_saturation(a, sat);
      }
    }
  }
}

// ===========================================================================
// Streaming decode gate/up GEMM (4 to 16 rows per expert on average,
// K = H <= 2048).  The work is a list of units (one 16-row chunk of an
// expert's grouped rows x 128 gate columns and the matching 128 up columns),
// dealt to one persistent block per CU in contiguous ranges, so that
// consecutive units of a block mostly share their activation rows.  Each of
// the 8 waves owns 16 gate and the 16 matching up rows of a unit (two 16-row
// tiles) and streams them 128 bytes of k at a time (a 4 KB chunk) from global
// memory straight into a private LDS ring, kDSDepth chunks ahead of their use
// and across unit boundaries: no register ring, no block barrier for the
// weights, and every copy instruction moves 8 rows x 128 contiguous bytes.  A
// chunk is unpacked from LDS into the B operand of the 16x16x32 FP16 MFMA,
// whose A operand is the unit's hidden rows, copied (BF16) into LDS by the
// same copies whenever the row chunk changes and converted there to FP16 with
// the power of two the routing kernel found for each row.
// INT4 / FP8 scales multiply each 128-wide k block's FP32 partial sum, as in
// gemm_decode.  A chunk's scales travel the same way, by one more copy into a
// per-wave LDS slot: the loop issues no load whose result lands in registers,
// so nothing but the explicit waits holds a wave back (a register load in the
// mix would make the compiler wait for every copy in flight).
//   Lane l: MFMA column (weight row) l % 16 of a tile, k slice q = l / 16;
//   result rows (activation rows) 4 q + [0, 4).  Ring chunk layout: local row
//   lr (0..31) x 8 pieces of 16 bytes, piece pc of row lr at slot
//   8 lr + (pc ^ ((lr >> 1) & 7)), so 16 rows reading one piece hit distinct
//   banks.
// ===========================================================================
constexpr int kDSMaxK = 2048;         // activation rows staged whole in LDS
constexpr int kDSDepth = 2;           // chunks in flight per wave
constexpr int kDSChunk = 32 * 128;    // bytes: 32 weight rows x 128 bytes of k
constexpr size_t kDSAsBytes = (size_t)16 * (kDSMaxK + 8) * 2;
constexpr int kDSScB = 1024;          // bytes of scale slot per wave and chunk (NVFP4; others use 256)
// dynamic LDS (every copy target): the weight rings, the scale slots, the
// activation rows; the tables are static
constexpr size_t kDSLds = (size_t)8 * kDSDepth * (kDSChunk + kDSScB) + kDSAsBytes;
static_assert(kDSLds + (size_t)(kMaxExperts + 1) * 4 + (size_t)kMaxExperts * 16 + 16 * 16 <= kMaxLdsBytes,
              "streaming decode GEMM fits in LDS");

typedef __attribute__((address_space(3))) void lds_void_t;
__device__ __forceinline__ void copy16_lds(const void *g, unsigned char *lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t *)lds, 16, 0, 0);
}
// 4 bytes per lane: lane i's dword lands at lds + 4 i
__device__ __forceinline__ void copy4_lds(const void *g, unsigned char *lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t *)lds, 4, 0, 0);
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int FMT>
__global__ __launch_bounds__(512) void gemm_decode_stream(GemmArgs a) {
  // Every copy target is in the dynamic LDS array, which the compiler does
  // not match against the copies in flight (for copies into a static array it
  // would wait for all of them before any read of that array): the explicit
  // waits below are what orders each read after its copy.
  extern __shared__ __align__(16) unsigned char ring[];                 // [8 waves][kDSDepth][4 KB]
  constexpr int SCB = FMT == FMT_NVFP4 ? kDSScB : 256;
  unsigned char *scs = ring + (size_t)8 * kDSDepth * kDSChunk;          // [8 waves][kDSDepth][SCB]
  _Float16 *As = (_Float16 *)(scs + (size_t)8 * kDSDepth * SCB);        // [16][K + 8]
  __shared__ int rcpre[kMaxExperts + 1];                                // [active + 1]
  __shared__ int4 einf[kMaxExperts];                                    // [active]: the expert table
  __shared__ int4 rinf[16];                                             // the unit's row records
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int col = lane & 15, q = lane >> 4;
  const int K = a.K, N = a.N, lda = K + 8, G = K / 128;
  const int RB = FMT == FMT_FP8 ? K : K / 2;  // bytes per weight row
  const int CPU = RB / 128;                   // chunks per unit and wave
  constexpr int NGC = FMT == FMT_FP8 ? 1 : 2; // 128-wide k groups per chunk

  // ---- the expert table and the grouping's prefix of its 16-row chunks, in
  // LDS (global loads consumed in the loop would make the wave wait for every
  // copy in flight); count, records and prefix in one round trip (the
  // workspace holds E + 1 of each; entries past the count are not kept)
  // (.w: the NVFP4 expert's 1 / global scale)
  constexpr int NU = (kMaxExperts + 512) / 512;
  int4 ev[NU];
  int pv[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int i = threadIdx.x + 512 * u;
    if (i < a.E) ev[u] = a.einfo[1 + i];
    if (i <= a.E) pv[u] = a.rcp[i];
  }
  const int n_act = __builtin_amdgcn_readfirstlane(a.einfo[0].x);
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int i = threadIdx.x + 512 * u;
    if (i < n_act) {
      int4 ei = ev[u];
      if (FMT == FMT_NVFP4) ei.w = __builtin_bit_cast(int, 1.0f / a.gscale[ei.x]);
      einf[i] = ei;
    }
    if (i <= n_act) rcpre[i] = pv[u];
  }
  __syncthreads();
  const int UPE = a.tiles;
  // Contiguous unit ranges of L = ceil(units / blocks) units.  When L divides
  // the units of one row chunk, ranges start at multiples of L, so no range
  // crosses a chunk (one row staging per block); otherwise ranges are spread
  // proportionally (at most one more unit than the fewest).
  const int64_t n_units = (int64_t)rcpre[n_act] * UPE;
  const int64_t L = (n_units + gridDim.x - 1) / gridDim.x;
  int u0, u1;
  if (L > 0 && UPE % L == 0) {
    u0 = (int)min<int64_t>((int64_t)blockIdx.x * L, n_units);
    u1 = (int)min<int64_t>(u0 + L, n_units);
  } else {
    u0 = (int)((int64_t)blockIdx.x * n_units / gridDim.x);
    u1 = (int)((int64_t)(blockIdx.x + 1) * n_units / gridDim.x);
  }
  if (u0 >= u1) return;  // block-uniform

  struct Unit {
    int e, r0, nr, tile, rc;
    float ginv;
  };
  auto unit_of = [&](int u) {
    Unit x;
    x.rc = u / UPE;
    x.tile = u - x.rc * UPE;
    int lo = 0, hi = n_act - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (rcpre[mid] <= x.rc) lo = mid; else hi = mid - 1;
    }
    const int4 ei = einf[lo];
    const int mc = x.rc - rcpre[lo];
    x.e = ei.x;
    x.r0 = ei.y + 16 * mc;
    x.nr = min(16, ei.z - 16 * mc);
    x.ginv = FMT == FMT_NVFP4 ? __builtin_bit_cast(float, ei.w) : 1.0f;
    return x;
  };
  // global weight row of local row lr (0..31) of this wave in unit x (gate
  // rows, then the matching up rows); rows past the end read row 0 of the
  // expert and are never stored
  auto wrow = [&](const Unit &x, int lr) {
    const int hc = x.tile * 128 + 16 * wave + (lr & 15);
    return hc < a.I ? (lr < 16 ? hc : a.I + hc) : 0;
  };
  // scales of a chunk, one copy into the wave's scale slot: INT4 the two FP16
  // group scales of row lane % 32 (dword 4 lr), NVFP4 its 16 E4M3 bytes
  // (16 lr + 8 g + 2 q: the pair of k slice q in group g), FP8 the block scale
  // of tile lane % 2 (dword 4 t); lanes 32..63 repeat lanes 0..31
  auto issue_sc = [&](const Unit &x, int c, int sl) {
    unsigned char *dst = scs + ((size_t)wave * kDSDepth + sl) * SCB;
    if (FMT == FMT_INT4) {
      const int n = wrow(x, lane & 31);
      copy4_lds((const uint16_t *)a.scale + ((size_t)x.e * N + n) * G + 2 * c, dst);
    } else if (FMT == FMT_NVFP4) {
      const int n = wrow(x, lane & 31);
      copy16_lds((const uint8_t *)a.scale + ((size_t)x.e * N + n) * (K / 16) + 16 * c, dst);
    } else {
      const int nb = wrow(x, 16 * (lane & 1));  // the tile's 16 rows share a block
      copy4_lds((const float *)a.scale + ((size_t)x.e * (N / 128) + nb / 128) * G + c, dst);
    }
  };
  auto issue_w = [&](const Unit &x, int c, int sl) {
    unsigned char *dst = ring + ((size_t)wave * kDSDepth + sl) * kDSChunk;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int lr = 8 * q4 + (lane >> 3), pc = (lane & 7) ^ ((lr >> 1) & 7);
      copy16_lds(a.w + ((size_t)x.e * N + wrow(x, lr)) * RB + 128 * c + 16 * pc, dst + 1024 * q4);
    }
  };
  // the unit's row records into rinf, then its BF16 hidden rows (by token)
  // into As (all waves), by copies of up to 1 KB; once its copies have landed
  // each lane converts the 16 bytes it copied in place: FP16 scaled by the
  // row's 2^-s (the routing kernel's power of two, whose 2^s is the record's
  // row scale; exact reciprocal of a power of two), in the INT4 unpack's k
  // order for INT4, as the routing kernel stages rows for the prefill GEMMs.
  // Leaves every copy of the wave complete; the caller's barrier publishes As.
  auto stage_rows = [&](const Unit &x) {
    if (threadIdx.x < 16) rinf[threadIdx.x] = threadIdx.x < x.nr ? a.rowinfo[x.r0 + threadIdx.x] : int4{0, 0, 0, 0};
    __syncthreads();
    const int rowb = 2 * K, pieces = (rowb + 1023) >> 10;
    for (int idx = wave; idx < x.nr * pieces; idx += 8) {
      const int m = idx / pieces, pc = idx - m * pieces;
      const int src_row = __builtin_amdgcn_readfirstlane(rinf[m].y);
      const int off = pc * 1024 + 16 * lane;
      if (off < rowb)
        copy16_lds((const unsigned char *)a.hidden + (size_t)src_row * rowb + off,
                   (unsigned char *)As + (size_t)m * lda * 2 + pc * 1024);
    }
    wait_vmcnt<0>();  // this wave's row copies (and every chunk it has in flight)
    for (int idx = wave; idx < x.nr * pieces; idx += 8) {
      const int m = idx / pieces, pc = idx - m * pieces;
      const int off = pc * 1024 + 16 * lane;
      if (off < rowb) {
        u4 *p = (u4 *)((unsigned char *)As + (size_t)m * lda * 2 + off);
        const float down = __builtin_bit_cast(float, (uint32_t)(254u << 23) - (uint32_t)rinf[m].z);
        u4 v = bf16x8_to_f16x8(*p, down);
        if (FMT == FMT_INT4) v = perm_0415(v);
        *p = v;
      }
    }
  };

  f4 acc[2];
  acc[0] = acc[1] = f4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const Unit &x, int c, int sl) {
    const unsigned char *wb = ring + ((size_t)wave * kDSDepth + sl) * kDSChunk;
    const unsigned char *sb = scs + ((size_t)wave * kDSDepth + sl) * SCB;
#pragma unroll
    for (int gi = 0; gi < NGC; ++gi) {
      const int gk = (NGC * c + gi) * 128;
      h8 av[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) av[j] = *(const h8 *)(As + col * lda + gk + 32 * q + 8 * j);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int lr = 16 * t + col, sw = (lr >> 1) & 7;
        uint32_t sv = 0u;
        float sf = 0.f;
        if (FMT == FMT_INT4)
          sv = (*(const uint32_t *)(sb + 4 * lr) >> (16 * gi)) & 0xFFFFu;
        else if (FMT == FMT_NVFP4)
          sv = *(const uint16_t *)(sb + 16 * lr + 8 * gi + 2 * q);
        else
          sf = *(const float *)(sb + 4 * t);
        u4 w0, w1;
        if (FMT == FMT_FP8) {
          w0 = *(const u4 *)(wb + 16 * (8 * lr + ((2 * q) ^ sw)));
          w1 = *(const u4 *)(wb + 16 * (8 * lr + ((2 * q + 1) ^ sw)));
        } else {
          w0 = *(const u4 *)(wb + 16 * (8 * lr + ((4 * gi + q) ^ sw)));
        }
        f4 tmp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          h8 bv;
          if (FMT == FMT_INT4)
            bv = unpack_int4(w0[j]);
          else if (FMT == FMT_FP8)
            bv = j < 2 ? unpack_fp8(w0[2 * j], w0[2 * j + 1]) : unpack_fp8(w1[2 * j - 4], w1[2 * j - 3]);
          else
            bv = unpack_nvfp4(w0[j], e4m3_to_f16((sv >> (8 * (j >> 1))) & 0xFFu));
          if (FMT == FMT_NVFP4)
            acc[t] = mfma16(av[j], bv, acc[t]);
          else
            tmp = mfma16(av[j], bv, tmp);
        }
        if (FMT == FMT_INT4)
          acc[t] += tmp * (float)__builtin_bit_cast(_Float16, (uint16_t)sv);
        else if (FMT == FMT_FP8)
          acc[t] += tmp * sf;
      }
    }
  };
  auto epilogue = [&](const Unit &x) {
    const float ginv = x.ginv;
    uint32_t sat = 0u;
    const int hc = x.tile * 128 + 16 * wave + col;
    if (x.tile * 128 + 16 * wave < a.I) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = 4 * q + v;
        if (m < x.nr) {
          const float rs = __builtin_bit_cast(float, rinf[m].z) * ginv;
          a.h_out[(size_t)(x.r0 + m) * a.I + hc] = to_f16_sat(silu(acc[0][v] * rs) * (acc[1][v] * rs), sat);
        }
      }
    }
    flag_saturation(a, sat);
    acc[0] = acc[1] = f4{0.f, 0.f, 0.f, 0.f};
  };

  // ---- the chunk sequence of this block: s -> unit u0 + s / CPU, chunk s % CPU
  const int S = (u1 - u0) * CPU;
  Unit iss = unit_of(u0);
  int iss_u = u0, iss_c = 0, issued = 0;
  auto issue_next = [&](int sl) {
    issue_sc(iss, iss_c, sl);
    issue_w(iss, iss_c, sl);
    ++issued;
    if (++iss_c == CPU && issued < S) {
      iss_c = 0;
      iss = unit_of(++iss_u);
    }
  };
  static_assert(kDSDepth == 2, "the loop below alternates two ring slots");
  issue_next(0);
  if (issued < S) issue_next(1);
  Unit cur = unit_of(u0);
  int cur_u = u0, staged_rc = -1;
  // wait for this wave's chunk s with `later` newer chunks in flight: each
  // chunk is five copies (scales, then four of weights) and copies complete in
  // issue order, so at most five outstanding means chunk s is in LDS (stores
  // of a finished unit, also counted, only make the wait stricter)
  auto wait_chunk = [&](int later) {
    if (later) wait_vmcnt<5>(); else wait_vmcnt<0>();
  };
  auto step = [&](int s, int sl) {
    const int c = s - (cur_u - u0) * CPU;
    if (c == 0 && cur.rc != staged_rc) {
      // every wave is done reading the previous rows and records (no wait
      // for the weight copies in flight)
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      stage_rows(cur);
      __syncthreads();
      staged_rc = cur.rc;
    }
    wait_chunk(issued - s - 1);
    compute(cur, c, sl);
    // the slot's LDS reads are complete before its refill is issued
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    if (issued < S) issue_next(sl);
    if (c == CPU - 1) {
      epilogue(cur);
      if (cur_u + 1 < u1) cur = unit_of(++cur_u);
    }
  };
  for (int s = 0; s < S; s += 2) {
    step(s, 0);
    if (s + 1 < S) step(s + 1, 1);
  }
}

// ===========================================================================
// Prefill path (many rows per expert).  Tiles of 128 grouped rows of one
// expert; weight codes become FP16 MFMA operands that carry their group /
// block scale, multiplied by a power of two 2^p per weight column chosen from
// the column's largest scale so the values sit high in FP16 range, and the
// accumulator of that column is multiplied by 2^-p at the end.  INT4: the FP16
// group scale times 2^p is exact, so (c - 8) * s is rounded once to FP16
// (relative error <= 2^-11).  FP8: the FP32 block scale times 2^p is rounded
// to FP16 first, then the product e4m3 * s (two roundings, relative error
// below 2^-10).  NVFP4 e2m1 * e4m3 products are exact in FP16; its global
// scale divides the finished sum.
//
// Tiles are numbered (M-tile, N-tile) with N fastest and dealt to the 8 XCDs
// in contiguous ranges (blocks are dispatched to XCDs round robin), so tiles
// that share activation rows or an expert's weights run on the same L2.
// ===========================================================================
constexpr int kBM = kPrefillBM;  // grouped rows per M tile

// Power of two that maps a row's largest weight magnitude `m` to [2^14, 2^15).
__device__ __forceinline__ float row_pow2(float m, float *inv) {
  const int sh = -row_shift(m);  // row_shift maps m * 2^-s into [2^14, 2^15)
  *inv = pow2f(-sh);
  return pow2f(sh);
}

// Weights in registers.  A block of WPB waves covers 128 grouped rows of one
// expert; each wave owns TN 32-column weight tiles and all 128 rows, a TN x 4
// grid of MFMA 32x32x16 tiles.  TN = 2 (the one launched): 128 accumulators
// per lane, two waves per SIMD (gate/up: one 8-wave block per CU; down: two
// 4-wave blocks); TN = 4: 256 accumulators in the accumulation registers, one
// wave per SIMD.  Only the FP16 activation tile goes through LDS (written
// once by the block, read by all its waves); every wave streams the packed codes of its own columns into registers one k step
// ahead and unpacks them straight into the MFMA A operand with the column's
// scale folded in.
//
// Per k step of 64 a lane holds 32 k values of its column: FP8 bytes
// 16 h + [0, 16) and 32 + 16 h + [0, 16) of the step (h = lane / 32), INT4 and
// NVFP4 bytes 16 h + [0, 16) (k 32 h + [0, 32)).  MFMA s of the step takes the
// lane's 8 values s; the activation fragment of lane half h reads the same k
// offsets (any k order works when both operands follow it).
//
// gate/up (STAGE 0): wave w of column tile nt holds gate columns
// 16 TN (WPB nt + w) + [0, 16 TN) in tiles [0, TN/2) and the matching up
// columns in the others, so SwiGLU runs in registers (STAGE 2: the same, with
// h quantized to NVFP4 activations for the W4A4 layer).  down (STAGE 1): wave w
// holds output columns 32 TN (WPB nt + w) + [0, 32 TN); its rows go to
// scattered partial slots through an LDS transpose.  A wave whose columns lie
// past the end (I or H not a multiple of the block width) stages activations
// and takes the barriers but multiplies and stores nothing.
// ===========================================================================
constexpr int kWK = 64;  // k step

// Shape of a variant with TN 32-column tiles per wave and WPB waves per block:
// SPB k steps per activation buffer (one barrier each), LDS row stride in halves,
// bytes of one buffer, weight columns per block, dynamic LDS per block, and
// the activation staging passes (each thread stages 16 bytes of one row per
// pass; a pass covers 8 WPB rows).
template <int TN, int WPB, int SPB_>
struct WideShape {
  static constexpr int SPB = SPB_;
  static constexpr int LD = SPB * kWK + 8;
  static constexpr size_t ABUF = (size_t)kBM * LD * 2;
  static constexpr int BC = WPB * 32 * TN;
  static constexpr size_t LDS = 2 * ABUF + 2 * BC * sizeof(float) + kBM * 16;
  static constexpr int AP = kBM / (8 * WPB);
};

template <int FMT, int TN>
struct WideRegs {
  uint32_t w[TN][FMT == FMT_FP8 ? 8 : 4];  // codes of column tile tn
  uint32_t s[TN];  // INT4: FP16 scale bits; FP8: FP32 scale bits; NVFP4: two E4M3 bytes
};

template <int FMT>
__device__ __forceinline__ int wide_koff(int s, int hh) {
  return FMT == FMT_FP8 ? 16 * hh + 8 * (s & 1) + 32 * (s >> 1) : 32 * hh + 8 * s;
}

template <int FMT, int TN, int WPB, int STAGE, int SPB_>
__global__ __launch_bounds__(64 * WPB) __attribute__((amdgpu_waves_per_eu(4 / TN, 4 / TN)))
void gemm_prefill_wide(GemmArgs a) {
  using Shape = WideShape<TN, WPB, SPB_>;
  constexpr int SPB = Shape::SPB, LD = Shape::LD, BC = Shape::BC, AP = Shape::AP;
  constexpr int WC = 32 * TN, TH = TN / 2;  // columns per wave; gate (and up) tiles per wave
  constexpr size_t ABUF = Shape::ABUF;
  extern __shared__ __align__(16) unsigned char smem[];
  float *colinv = (float *)(smem + 2 * ABUF);  // [BC]: 2^-p of each weight column (not NVFP4)
  float *rowfs = colinv + BC;                  // [BC]: 2^p
  int4 *rmeta = (int4 *)(rowfs + BC);          // [kBM]: the tile's grouped-row records
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int j = lane & 31, hh = lane >> 5;
  // ---- tile of this block
  const int NT = a.tiles;
  const int n_tiles = a.mtile[a.E] * NT;
  const int per_xcd = (n_tiles + 7) >> 3;
  const int xslot = blockIdx.x >> 3;
  if (xslot >= per_xcd) return;
  const int L = (blockIdx.x & 7) * per_xcd + xslot;
  if (L >= n_tiles) return;
  const int mt = L / NT, nt = L - mt * NT;
  int lo = 0, hi = a.E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.mtile[mid] <= mt) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  const int rbeg = a.offsets[e] + (mt - a.mtile[e]) * kBM;
  const int nrows = min(kBM, a.offsets[e + 1] - rbeg);
  const int K = a.K, N = a.N, G = K / 128, nK = K / kWK;
  const size_t rowbytes = FMT == FMT_FP8 ? (size_t)K : (size_t)K / 2;

  // ---- the wave's columns: global weight row of this lane in each tile
  // gate/up: first gate (h) column of the wave; down: first output column
  const int cb = STAGE != 1 ? nt * (BC / 2) + wave * (WC / 2) : nt * BC + wave * WC;
  const bool wvalid = cb < (STAGE != 1 ? a.I : N);  // wave-uniform
  int gr[TN];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
    const int c = STAGE != 1 ? (tn < TH ? cb : a.I + cb) + (tn % TH) * 32 + j : cb + tn * 32 + j;
    gr[tn] = wvalid ? c : j;  // a row that exists; never stored
  }

  // ---- power of two of each column (from its largest scale): lane half hh
  // takes tiles TN/2 hh + [0, TN/2), shared through LDS
  if (FMT != FMT_NVFP4) {
#pragma unroll
    for (int q = 0; q < TH; ++q) {
      const int tn = hh * TH + q;
      float m = 0.f;
      for (int g0 = 0; g0 < G; g0 += 8) {
        float sv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int g = min(g0 + u, G - 1);
          sv[u] = FMT == FMT_INT4 ? (float)((const _Float16 *)a.scale)[((size_t)e * N + gr[tn]) * G + g]
                                  : ((const float *)a.scale)[((size_t)e * (N / 128) + gr[tn] / 128) * G + g];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) m = fmaxf(m, fabsf(sv[u]));
      }
      float inv;
      rowfs[wave * WC + tn * 32 + j] = row_pow2(m * (FMT == FMT_INT4 ? 8.f : 448.f), &inv);
      colinv[wave * WC + tn * 32 + j] = inv;
    }
  }

  // ---- the epilogue's per-row data (slot, scale, routing weight), read now
  // so that the epilogue issues no global load (each would wait for every
  // store before it)
  if (tid < kBM) rmeta[tid] = tid < nrows ? a.rowinfo[rbeg + tid] : int4{0, 0, 0, 0};
  const float ginv = FMT == FMT_NVFP4 ? 1.0f / a.gscale[e] : 1.0f;

  // ---- activation staging: row (tid >> 3) + 8 WPB p, 16-byte chunk tid & 7
  const _Float16 *asrc[AP];
#pragma unroll
  for (int p = 0; p < AP; ++p) {
    const int rr = (tid >> 3) + 8 * WPB * p;
    const int r = rbeg + (rr < nrows ? rr : nrows - 1);
    // gate/up: the token's x16 row; down: the grouped h row
    asrc[p] = a.a_src + (STAGE != 1 ? (size_t)a.rowinfo[r].y : (size_t)r) * K + (tid & 7) * 8;
  }
  // ---- weight and scale streams of the lane's TN columns
  const uint8_t *wsrc[TN];
  const uint8_t *ssrc[TN];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
    wsrc[tn] = a.w + ((size_t)e * N + gr[tn]) * rowbytes + 16 * hh;
    if (FMT == FMT_INT4)
      ssrc[tn] = (const uint8_t *)((const uint16_t *)a.scale + ((size_t)e * N + gr[tn]) * G);
    else if (FMT == FMT_FP8)
      ssrc[tn] = (const uint8_t *)((const float *)a.scale + ((size_t)e * (N / 128) + gr[tn] / 128) * G);
    else
      ssrc[tn] = (const uint8_t *)a.scale + ((size_t)e * N + gr[tn]) * (K / 16) + 2 * hh;
  }

  auto load_a = [&](u4 (&ar)[AP], int ks) {
#pragma unroll
    for (int p = 0; p < AP; ++p) ar[p] = *(const u4 *)(asrc[p] + ks * kWK);
  };
  auto write_a = [&](const u4 (&ar)[AP], int buf, int sub) {
    _Float16 *As = (_Float16 *)(smem + buf * ABUF) + sub * kWK;
#pragma unroll
    for (int p = 0; p < AP; ++p) {
      // INT4: x16 is stored INT4-ordered, h in natural order
      *(u4 *)(As + ((tid >> 3) + 8 * WPB * p) * LD + (tid & 7) * 8) = FMT == FMT_INT4 && STAGE == 1 ? perm_0415(ar[p]) : ar[p];
    }
  };
  auto load_w = [&](WideRegs<FMT, TN> &R, int ks) {
    const int kb = ks * kWK;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      if (FMT == FMT_FP8) {
        const u4 v0 = *(const u4 *)(wsrc[tn] + kb);
        const u4 v1 = *(const u4 *)(wsrc[tn] + kb + 32);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          R.w[tn][q] = v0[q];
          R.w[tn][4 + q] = v1[q];
        }
      } else {
        const u4 v = *(const u4 *)(wsrc[tn] + kb / 2);
#pragma unroll
        for (int q = 0; q < 4; ++q) R.w[tn][q] = v[q];
      }
    }
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      if (FMT == FMT_INT4)
        R.s[tn] = ((const uint16_t *)ssrc[tn])[kb >> 7];
      else if (FMT == FMT_FP8)
        R.s[tn] = ((const uint32_t *)ssrc[tn])[kb >> 7];
      else
        R.s[tn] = *(const uint16_t *)(ssrc[tn] + kb / 16);
    }
  };

  __syncthreads();  // rowfs / colinv
  float rowf[TN];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) rowf[tn] = 1.f;
  if (FMT != FMT_NVFP4) {
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) rowf[tn] = rowfs[wave * WC + tn * 32 + j];
  }

  f16v acc[TN][4];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn)
#pragma unroll
    for (int tm = 0; tm < 4; ++tm)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[tn][tm][i] = 0.f;

  // NV: 32-row M subtiles that hold rows of the expert (block-uniform; 0 for
  // a wave past the last column)
  auto compute = [&](auto nv_c, const WideRegs<FMT, TN> &R, int buf, int sub) {
    constexpr int NV = decltype(nv_c)::value;
    if constexpr (NV > 0) {
      const _Float16 *As = (const _Float16 *)(smem + buf * ABUF) + sub * kWK;
      h2 sc[TN];
      if (FMT != FMT_NVFP4) {
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const float sv = FMT == FMT_INT4 ? (float)__builtin_bit_cast(_Float16, (uint16_t)R.s[tn])
                                           : __builtin_bit_cast(float, R.s[tn]);
          const _Float16 s16 = (_Float16)(sv * rowf[tn]);
          sc[tn] = h2{s16, s16};
        }
      }
      // activation fragments of sub-step s + 1 are read while sub-step s
      // multiplies; the compiler interleaves the unpack with the MFMAs of the
      // k step (an explicit one-MFMA-per-unpack-share interleave measured 2-4%
      // slower on every format)
      h8 afc[NV], afn[NV];
#pragma unroll
      for (int tm = 0; tm < NV; ++tm) afc[tm] = *(const h8 *)(As + (tm * 32 + j) * LD + wide_koff<FMT>(0, hh));
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (s < 3) {
#pragma unroll
          for (int tm = 0; tm < NV; ++tm)
            afn[tm] = *(const h8 *)(As + (tm * 32 + j) * LD + wide_koff<FMT>(s + 1, hh));
        }
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          h8 wf;
          if (FMT == FMT_INT4) {
            wf = unpack_int4(R.w[tn][s]);
          } else if (FMT == FMT_FP8) {
            wf = unpack_fp8(R.w[tn][2 * s], R.w[tn][2 * s + 1]);
          } else {
            wf = unpack_nvfp4(R.w[tn][s], e4m3_to_f16((R.s[tn] >> (8 * (s >> 1))) & 0xFFu));
          }
          if (FMT != FMT_NVFP4) {
            u4 w = as_u4(wf);
#pragma unroll
            for (int q = 0; q < 4; ++q) w[q] = as_u32(as_h2(w[q]) * sc[tn]);
            wf = as_h8(w);
          }
#pragma unroll
          for (int tm = 0; tm < NV; ++tm) acc[tn][tm] = mfma32(wf, afc[tm], acc[tn][tm]);
        }
        if (s < 3) {
#pragma unroll
          for (int tm = 0; tm < NV; ++tm) afc[tm] = afn[tm];
        }
      }
    }
  };
  // One barrier per SPB k steps: an LDS buffer holds the activations of
  // SPB steps, and while the block multiplies from one buffer it fills the
  // other one k step at a time (so the staging registers hold one step).
  // Weights for k step t + 1 load while step t multiplies.
  auto main_loop = [&](auto nv_c) {
    WideRegs<FMT, TN> R[2];
    u4 ar[AP], a0[SPB][AP];
    // same load order as in the loop (activations of a later step, then
    // weights), so that the loop's first LDS write waits for the activation
    // loads alone
#pragma unroll
    for (int u = 0; u < SPB; ++u) load_a(a0[u], u);
    load_a(ar, min(SPB, nK - 1));
    __builtin_amdgcn_sched_barrier(0);
    load_w(R[0], 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < SPB; ++u) write_a(a0[u], 0, u);
    for (int t = 0; t < nK; t += SPB) {  // nK is a multiple of SPB (checked by the launcher)
      const int q = (t / SPB) & 1;
      __syncthreads();
#pragma unroll
      for (int u = 0; u < SPB; ++u) {
        // k step t + u from buffer q; stage step t + SPB + u into the other
        // (past the end: a repeat of the last step, never read)
        write_a(ar, q ^ 1, u);
        load_a(ar, min(t + SPB + u + 1, nK - 1));
        __builtin_amdgcn_sched_barrier(0);
        load_w(R[(u + 1) & 1], min(t + u + 1, nK - 1));
        // keep the loads ahead of the MFMAs (left alone, the scheduler sinks
        // them to the end of the step and the next step waits for them)
        __builtin_amdgcn_sched_barrier(0);
        compute(nv_c, R[u & 1], q, u);
      }
    }
  };
  const int nv = wvalid ? min(4, (nrows + 31) / 32) : 0;
  switch (nv) {
    case 4: main_loop(std::integral_constant<int, 4>{}); break;
    case 3: main_loop(std::integral_constant<int, 3>{}); break;
    case 2: main_loop(std::integral_constant<int, 2>{}); break;
    case 1: main_loop(std::integral_constant<int, 1>{}); break;
    default: main_loop(std::integral_constant<int, 0>{}); break;
  }

  // ---- epilogue: lane l holds grouped row m = 32 tm + l % 32 and, in
  // register v of tile tn, column 8 (v / 4) + 4 (l / 32) + v % 4 of the tile
  const int cl = 4 * hh;
  const float *cinv = colinv + wave * WC;
  uint32_t sat = 0u;
  typedef uint32_t u2 __attribute__((ext_vector_type(2)));
  if constexpr (STAGE == 0) {
    if (wvalid) {
#pragma unroll
      for (int tm = 0; tm < 4; ++tm) {
        const int row = tm * 32 + j;
        if (row >= nrows) continue;
        const int r = rbeg + row;
        const float rsc = __builtin_bit_cast(float, rmeta[row].z) * ginv;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int c4 = 8 * g4 + cl;
#pragma unroll
          for (int tn = 0; tn < TH; ++tn) {
            // column inverses (NVFP4: all 1, not applied)
            f4 ig = {1.f, 1.f, 1.f, 1.f}, iu = ig;
            if (FMT != FMT_NVFP4) {
              ig = *(const f4 *)(cinv + tn * 32 + c4);
              iu = *(const f4 *)(cinv + (tn + TH) * 32 + c4);
            }
            h2 o[2];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float gv = acc[tn][tm][4 * g4 + i] * (FMT == FMT_NVFP4 ? rsc : rsc * ig[i]);
              const float uv = acc[tn + TH][tm][4 * g4 + i] * (FMT == FMT_NVFP4 ? rsc : rsc * iu[i]);
              const float hv = silu(gv) * uv;
              const float hc = fminf(fmaxf(hv, -65504.f), 65504.f);
              sat |= hc != hv;
              o[i >> 1][i & 1] = (_Float16)hc;
            }
            *(u2 *)(a.h_out + (size_t)r * a.I + cb + tn * 32 + c4) = u2{as_u32(o[0]), as_u32(o[1])};
          }
        }
      }
    }
  } else if constexpr (STAGE == 2) {
    // W4A4 (NVFP4 only): h quantized to NVFP4 with global scale a.hq_g, stored
    // as the FP16 values e2m1(code) * s (exact, never saturating).  A 32-wide
    // slice of h holds two groups of 16: columns [0, 16) in registers g4 = 0,
    // 1 and [16, 32) in g4 = 2, 3 of lanes j and j + 32 (the same row, so both
    // lanes skip or keep a row together).
    static_assert(FMT == FMT_NVFP4, "W4A4 is the NVFP4 layer's variant");
    if (wvalid) {
#pragma unroll
      for (int tm = 0; tm < 4; ++tm) {
        const int row = tm * 32 + j;
        if (row >= nrows) continue;
        const int r = rbeg + row;
        const float rsc = __builtin_bit_cast(float, rmeta[row].z) * ginv;
#pragma unroll
        for (int tn = 0; tn < TH; ++tn) {
          float hv[16];
#pragma unroll
          for (int v = 0; v < 16; ++v)
            hv[v] = silu(acc[tn][tm][v] * rsc) * (acc[tn + TH][tm][v] * rsc);
          float m0 = 0.f, m1 = 0.f;
#pragma unroll
          for (int v = 0; v < 8; ++v) {
            m0 = fmaxf(m0, fabsf(hv[v]));
            m1 = fmaxf(m1, fabsf(hv[8 + v]));
          }
          m0 = fmaxf(m0, __shfl_xor(m0, 32, 64));
          m1 = fmaxf(m1, __shfl_xor(m1, 32, 64));
          const float s0 = nvfp4_act_scale(m0, a.hq_g).s, s1 = nvfp4_act_scale(m1, a.hq_g).s;
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const float sg = g4 < 2 ? s0 : s1;
            h2 o[2];
#pragma unroll
            for (int i = 0; i < 4; ++i)
              o[i >> 1][i & 1] = (_Float16)(e2m1_value(e2m1_code(hv[4 * g4 + i], a.hq_g, sg)) * sg);
            *(u2 *)(a.h_out + (size_t)r * a.I + cb + tn * 32 + 8 * g4 + cl) = u2{as_u32(o[0]), as_u32(o[1])};
          }
        }
      }
    }
  } else {
    // down: the rows go to scattered slots of the partial buffer, so each
    // 32-row slice of the wave's tile is converted and transposed through LDS
    // and stored 16 bytes per lane, WC * 2 contiguous bytes per row
    constexpr int TL = WC + 8;     // LDS row stride, halves
    constexpr int LPR = WC / 8;    // lanes per row
    constexpr int RPI = 64 / LPR;  // rows per store instruction
    static_assert(WPB * 32 * TL * 2 <= (int)(2 * ABUF), "transpose buffers fit the activation buffers");
    _Float16 *tb = (_Float16 *)smem + wave * 32 * TL;
    float vmax = 0.f;   // largest |value| before the FP16 clamp
    bool vnan = false;  // some value is NaN
    // the lane's column inverses, read once (NVFP4: all 1, not applied);
    // read inside the row loop they would be re-read after every transpose
    // store, which the compiler cannot tell apart from them
    f4 icr[TN][4];
    if (FMT != FMT_NVFP4) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) icr[tn][g4] = *(const f4 *)(cinv + tn * 32 + 8 * g4 + cl);
    }
    __syncthreads();  // every wave is done with the activation buffers
    if (wvalid) {
#pragma unroll
      for (int tm = 0; tm < 4; ++tm) {
        if (tm * 32 >= nrows) break;
        const int row = tm * 32 + j;
        float rsc = 0.f;  // rows past the expert's end: zeros, never stored
        if (row < nrows) rsc = __builtin_bit_cast(float, rmeta[row].w) * ginv * a.a_inv;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int c4 = 8 * g4 + cl;
#pragma unroll
          for (int tn = 0; tn < TN; ++tn) {
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
              v[i] = acc[tn][tm][4 * g4 + i] * (FMT == FMT_NVFP4 ? rsc : rsc * icr[tn][g4][i]);
            vmax = fmaxf(vmax, fmaxf(fabsf(v[0]), fabsf(v[1])));
            vmax = fmaxf(vmax, fmaxf(fabsf(v[2]), fabsf(v[3])));
            vnan |= __builtin_isunordered(v[0], v[1]) | __builtin_isunordered(v[2], v[3]);
            h2 o[2];
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i >> 1][i & 1] = (_Float16)fminf(fmaxf(v[i], -65504.f), 65504.f);
            *(u2 *)(tb + j * TL + tn * 32 + c4) = u2{as_u32(o[0]), as_u32(o[1])};
          }
        }
        // the wave reads back what its own lanes wrote (in-order LDS queue)
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_wave_barrier();
        const int ch = lane % LPR;
#pragma unroll
        for (int it = 0; it < 32 / RPI; ++it) {
          const int rr = it * RPI + lane / LPR;
          const int orow = tm * 32 + rr;
          const u4 v = *(const u4 *)(tb + rr * TL + ch * 8);
          if (orow < nrows)
            *(u4 *)(a.partial + (size_t)rmeta[orow].x * a.H + cb + ch * 8) = v;
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_wave_barrier();
      }
    }
    sat |= !(vmax <= 65504.f) || vnan;  // NaN counts as saturated
  }
  flag_saturation(a, sat);
}

// ===========================================================================
// Decode down projection with the combine fused in, for a few tokens
// (T <= kTokDownMaxT, where the expert-major GEMM and the combine are two
// short latency-bound launches).  One block per (token t, CB output columns);
// wave j takes the token's slots j, j + 8, ...: expert ids[t k + j], its
// grouped intermediate row inv_pos[t k + j] and routing weight.  Lane l is
// column l % CB of the block and k part l / CB; a part takes every (64 / CB)-th
// 64-wide k chunk (each inside one 128-wide scale group), converts the
// column's codes of the chunk to exact FP16 values and takes FP32 dot products
// with the h row (two products per instruction).  INT4 / FP8 scales multiply
// each chunk's sum in FP32, as in gemm_decode; NVFP4 block scales each 16-wide
// block's sum, 1/g the slot's total.  The parts are added across lanes, the
// slot's CB values times its routing weight go to LDS, and CB threads add the
// slots in order j = 0..k-1 (then the residual) into the BF16 output.  The
// slot values stay FP32: no FP16 partials, no partial buffer, no combine.
// A lane loads the codes and h of up to kTDBatch chunks before it multiplies.
// ===========================================================================
constexpr int kTokDownMaxT = 2;
constexpr int kTDBatch = 3;

template <int FMT, int CB>
__global__ __launch_bounds__(512) void gemm_decode_down_tok(GemmArgs a) {
  constexpr int QP = 64 / CB;                        // k parts per column
  constexpr int WQ = FMT == FMT_FP8 ? 4 : 2;         // 16-byte code loads per chunk
  __shared__ float red[64][CB];                      // [slot][column], k <= 64
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int c = lane % CB, qp = lane / CB;
  const int t = blockIdx.y, n0 = blockIdx.x * CB, n = n0 + c;
  const int K = a.K, N = a.N, G = K / 128, NCH = K / 64, k = a.k;
  const size_t RB = FMT == FMT_FP8 ? (size_t)K : (size_t)K / 2;
  for (int j = wave; j < k; j += 8) {
    const int slot = t * k + j;
    const int e = __builtin_amdgcn_readfirstlane(a.slot_ids[slot]);
    const int r = __builtin_amdgcn_readfirstlane(a.slot_pos[slot]);
    const float wt = a.slot_w[slot] * (FMT == FMT_NVFP4 ? 1.0f / a.gscale[e] : 1.0f);
    const uint8_t *wrow = a.w + ((size_t)e * N + n) * RB;
    const _Float16 *hrow = a.a_src + (size_t)r * K;
    float acc = 0.f;
    for (int cb = qp; cb < NCH; cb += kTDBatch * QP) {
      u4 wv[kTDBatch][WQ], hv[kTDBatch][8];
      uint32_t sv[kTDBatch];
#pragma unroll
      for (int b = 0; b < kTDBatch; ++b) {
        const int ch = cb + b * QP;
        if (ch < NCH) {
#pragma unroll
          for (int i = 0; i < WQ; ++i) wv[b][i] = *(const u4 *)(wrow + (size_t)ch * (16 * WQ) + 16 * i);
#pragma unroll
          for (int i = 0; i < 8; ++i) hv[b][i] = *(const u4 *)(hrow + ch * 64 + 8 * i);
          if (FMT == FMT_INT4)
            sv[b] = ((const uint16_t *)a.scale)[((size_t)e * N + n) * G + ch / 2];
          else if (FMT == FMT_FP8)
            sv[b] = ((const uint32_t *)a.scale)[((size_t)e * (N / 128) + n / 128) * G + ch / 2];
          else
            sv[b] = *(const uint32_t *)((const uint8_t *)a.scale + ((size_t)e * N + n) * (K / 16) + ch * 4);
        }
      }
#pragma unroll
      for (int b = 0; b < kTDBatch; ++b) {
        if (cb + b * QP >= NCH) break;
        float sum = 0.f;
        if (FMT == FMT_NVFP4) {
#pragma unroll
          for (int sb = 0; sb < 4; ++sb) {  // 16-wide blocks: words 2 sb, 2 sb + 1
            float bs = 0.f;
#pragma unroll
            for (int ww = 2 * sb; ww < 2 * sb + 2; ++ww) {
              const uint32_t word = wv[b][ww >> 2][ww & 3];
#pragma unroll
              for (int bs8 = 0; bs8 < 4; ++bs8)
                bs = __builtin_amdgcn_fdot2(e2m1x2_to_h2(word, bs8), as_h2(hv[b][ww][bs8]), bs, false);
            }
            sum += bs * (float)e4m3_to_f16((sv[b] >> (8 * sb)) & 0xFFu);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) {  // k 8 i + [0, 8) of the chunk
            h8 wf;
            u4 hp = hv[b][i];
            if (FMT == FMT_INT4) {
              wf = unpack_int4(wv[b][i >> 2][i & 3]);
              hp = perm_0415(hp);  // the unpack's k order 0, 4, 1, 5, ...
            } else {
              wf = unpack_fp8(wv[b][(2 * i) >> 2][(2 * i) & 3], wv[b][(2 * i + 1) >> 2][(2 * i + 1) & 3]);
            }
            const u4 wu = as_u4(wf);
#pragma unroll
            for (int q = 0; q < 4; ++q) sum = __builtin_amdgcn_fdot2(as_h2(wu[q]), as_h2(hp[q]), sum, false);
          }
          sum *= FMT == FMT_INT4 ? (float)__builtin_bit_cast(_Float16, (uint16_t)sv[b])
                                 : __builtin_bit_cast(float, sv[b]);
        }
        acc += sum;
      }
    }
    // the k parts of a column, added in a fixed pattern (every lane ends
    // with the same value)
#pragma unroll
    for (int d = CB; d < 64; d <<= 1) acc += __shfl_xor(acc, d, 64);
    if (qp == 0) red[j][c] = acc * wt;
  }
  __syncthreads();
  if (threadIdx.x < CB) {
    float o = 0.f;
    for (int j = 0; j < k; ++j) o += red[j][threadIdx.x];
    const size_t oi = (size_t)t * a.H + n0 + threadIdx.x;
    if (a.residual) o = bf16_to_f32(a.residual[oi]) + o;
    a.out[oi] = f32_to_bf16_rne(o);
  }
}

// ===========================================================================
// Combine: out[t] = bf16(sum_j partial[t*k + j] (+ residual[t])), the FP16
// partials widened to FP32 and added in order j = 0..k-1 so repeated runs are
// bit-identical.  kStream: non-temporal partial loads, for a partial buffer
// larger than the 256 MiB last-level cache (NVFP4 Zipf T=16384, 537 MB:
// 107 -> 88 us); a smaller one is still partly cached from the down GEMM's
// writes, and plain loads read it faster (FP8 T=4096, 134 MB: 23.5 against
// 24.7 us).
// ===========================================================================
template <bool kStream>
__global__ __launch_bounds__(256) void combine_kernel(const _Float16 *__restrict__ partial,
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
  // the partials of up to 8 slots are loaded together, then summed in slot order
  for (int j0 = 0; j0 < k; j0 += 8) {
    h8 x[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
      if (j0 + jj < k) {
        const u4 *src = (const u4 *)(partial + ((size_t)t * k + j0 + jj) * H + c);
        x[jj] = as_h8(kStream ? __builtin_nontemporal_load(src) : *src);
      }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
      if (j0 + jj < k) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += (float)x[jj][i];
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
  GemmArgs a{};
  char *ws = P.ws;
  a.E = L.E; a.I = L.I; a.H = L.H; a.k = L.k; a.T = P.T;
  if (stage == 0) {
    a.w = L.w13; a.scale = L.s13; a.gscale = L.g13; a.N = 2 * L.I; a.K = L.H;
    a.a_src = (const _Float16 *)(ws + W.x16);
  } else {
    a.w = L.w2; a.scale = L.s2; a.gscale = L.g2; a.N = L.H; a.K = L.I;
    a.a_src = (const _Float16 *)(ws + W.h);
  }
  a.hidden = P.hidden;
  a.einfo = (const int4 *)(ws + W.active);
  a.rcp = (const int32_t *)(ws + W.rcpre);
  a.rowinfo = (const int4 *)(ws + W.rowinfo);
  a.offsets = (const int32_t *)(ws + W.offsets);
  a.mtile = (const int32_t *)(ws + W.mtile);
  a.h_out = (_Float16 *)(ws + W.h);
  a.partial = (_Float16 *)(ws + W.partial);
  a.flags = P.flags;
  a.tiles = 0;
  a.hq_g = P.act_g2;
  a.a_inv = stage == 1 && P.act_g2 > 0.f ? 1.f / P.act_g2 : 1.f;
  a.slot_ids = (const int32_t *)(ws + W.topk_ids);
  a.slot_pos = (const int32_t *)(ws + W.inv_pos);
  a.slot_w = (const float *)(ws + W.topk_w);
  a.residual = P.residual;
  a.out = P.out;
  return a;
}

// Launch-shape caches, shared by every host thread that launches: compute
// units per device, resident blocks per CU per (kernel, device, LDS bytes),
// and the (kernel, device) pairs whose dynamic-LDS limit has been raised.
static std::mutex g_launch_mu;
static std::map<int, int> g_num_cus;
static std::map<std::tuple<const void *, int, size_t>, int> g_per_cu;
static std::set<std::pair<const void *, int>> g_lds_raised;

static int current_device() {
  int dev = 0;
  (void)hipGetDevice(&dev);
  return dev;
}

static int num_cus() {
  const int dev = current_device();
  std::lock_guard<std::mutex> lk(g_launch_mu);
  auto it = g_num_cus.find(dev);
  if (it != g_num_cus.end()) return it->second;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    n = 256;
  g_num_cus[dev] = n;
  return n;
}

// Allow up to 160 KiB of dynamic LDS for kernel f on the current device (once).
void raise_lds_limit(const void *f) {
  const int dev = current_device();
  std::lock_guard<std::mutex> lk(g_launch_mu);
  if (g_lds_raised.insert({f, dev}).second) {
    // the dynamic limit is what the kernel's static LDS leaves of the CU's
    hipFuncAttributes fa{};
    const size_t stat = hipFuncGetAttributes(&fa, f) == hipSuccess ? fa.sharedSizeBytes : 0;
    (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)(kMaxLdsBytes - stat));
  }
}

// Workgroups of kernel f resident per CU at `threads` threads and `lds` bytes.
template <typename F>
static int blocks_per_cu(F f, int threads, size_t lds) {
  raise_lds_limit((const void *)f);
  const int dev = current_device();
  const auto key = std::make_tuple((const void *)f, dev, lds);
  {
    std::lock_guard<std::mutex> lk(g_launch_mu);
    auto it = g_per_cu.find(key);
    if (it != g_per_cu.end()) return it->second;
  }
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, threads, lds) != hipSuccess || n < 1) n = 1;
  std::lock_guard<std::mutex> lk(g_launch_mu);
  g_per_cu[key] = n;
  return n;
}

template <int FMT, int STAGE, int KSPLIT, int GCT, int TPW>
static hipError_t run_decode_t(GemmArgs a, int slots, const GemmLaunch &s) {
  constexpr int CG = kDecodeWaves / KSPLIT;
  a.tiles = STAGE == 0 ? a.I / (16 * CG * TPW) : a.H / (32 * CG * TPW);
  size_t lds = decode_lds_bytes(a.K, KSPLIT);
  static_assert(CG == 8 / KSPLIT && kDecodeWaves == 8, "decode_lds_bytes assumes 8 waves");
  if (lds > kMaxLdsBytes) return hipErrorInvalidValue;  // init rejects such shapes
  // units of 16 rows (an expert with many rows spreads over blocks) where the
  // chunk prefix fits after the staging buffers
  const size_t rc_off = (lds + 15) & ~(size_t)15;
  a.rc_off = 0;
  const size_t table = (size_t)16 * ((a.E + 4) / 4) + (size_t)16 * a.E;
  // with at most 16 tokens no expert holds more than 16 rows (a token's k
  // experts are distinct): whole experts are the same units, without the table
  if (a.T > 16 && rc_off + table <= kMaxLdsBytes) {
    a.rc_off = (int)rc_off;
    lds = rc_off + table;
  }
  // persistent grid: as many blocks as are resident at once (from the
  // kernel's registers and LDS), never more than the number of units
  const int per_cu = blocks_per_cu(gemm_decode<FMT, STAGE, KSPLIT, GCT, TPW>, 64 * kDecodeWaves, lds);
  const long units = (long)slots * a.tiles;
  const long grid = std::min<long>(units, (long)num_cus() * per_cu);
  hipExtLaunchKernelGGL((gemm_decode<FMT, STAGE, KSPLIT, GCT, TPW>), dim3((unsigned)grid),
                        dim3(64 * kDecodeWaves), (uint32_t)lds, s.stream, s.start, s.stop, 0u, a);
  return hipGetLastError();
}

// Down projection with an even number of k groups up to 8 per wave: two tile
// pairs per wave when they tile H and the halved unit count still gives every
// CU two units (a unit's ring then streams twice the bytes).
template <int FMT, int STAGE, int KSPLIT, int GCT>
static hipError_t run_decode_g(GemmArgs a, int slots, const GemmLaunch &s) {
  constexpr int CG = kDecodeWaves / KSPLIT;
  if constexpr (STAGE == 1 && KSPLIT == 1 && GCT > 0 && GCT % 2 == 0 && GCT <= 8) {
    if (a.H % (32 * CG * 2) == 0 && (long)slots * (a.H / (32 * CG * 2)) >= 2L * num_cus())
      return run_decode_t<FMT, STAGE, KSPLIT, GCT, 2>(a, slots, s);
  }
  return run_decode_t<FMT, STAGE, KSPLIT, GCT, 1>(a, slots, s);
}

template <int FMT, int STAGE, int KSPLIT>
static hipError_t run_decode(GemmArgs a, int slots, const GemmLaunch &s) {
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
static hipError_t run_decode_ks(GemmArgs a, int slots, const GemmLaunch &s) {
  // Smallest k split (at most 4) whose column groups tile the expert exactly
  // and whose wave-tasks (tile pair x k split) cover the resident waves
  // (16 per CU): measured on the decode workloads, splitting k further only
  // adds reduction cost.
  const int cols = STAGE == 0 ? a.I / 16 : a.H / 32;  // tile pairs per expert
  const long waves = (long)num_cus() * 16;
  const int ksplits[3] = {1, 2, 4};
  int pick = 0;
  for (int ks : ksplits) {
    if (cols % (kDecodeWaves / ks) != 0) continue;
    if (pick == 0 || (long)slots * cols * pick < waves) pick = ks;
    if ((long)slots * cols * ks >= waves) break;
  }
  if (pick == 0) pick = 8;  // only KS = 8 (one column group) tiles the expert
  switch (pick) {
    case 1: return run_decode<FMT, STAGE, 1>(a, slots, s);
    case 2: return run_decode<FMT, STAGE, 2>(a, slots, s);
    case 4: return run_decode<FMT, STAGE, 4>(a, slots, s);
    default: return run_decode<FMT, STAGE, 8>(a, slots, s);
  }
}

template <int FMT, int TN, int WPB, int STAGE, int SPB>
static hipError_t run_prefill_wide1(GemmArgs a, int64_t R, const GemmLaunch &s) {
  using Shape = WideShape<TN, WPB, SPB>;
  constexpr int BC = Shape::BC;
  if (a.K % (Shape::SPB * kWK) != 0) return hipErrorInvalidValue;  // K fills whole LDS buffers
  a.tiles = STAGE != 1 ? (a.I + BC / 2 - 1) / (BC / 2) : (a.H + BC - 1) / BC;
  const int64_t max_mt = R / kBM + a.E;  // >= sum_e ceil(n_e / kBM)
  const int64_t grid = 8 * ((max_mt * a.tiles + 7) / 8);
  constexpr size_t lds = Shape::LDS;  // above the default limit
  static_assert(lds <= kMaxLdsBytes, "prefill tile fits in LDS");
  raise_lds_limit((const void *)gemm_prefill_wide<FMT, TN, WPB, STAGE, SPB>);
  hipExtLaunchKernelGGL((gemm_prefill_wide<FMT, TN, WPB, STAGE, SPB>), dim3((unsigned)grid), dim3(64 * WPB),
                        (uint32_t)lds, s.stream, s.start, s.stop, 0u, a);
  return hipGetLastError();
}

// gate/up (one 8-wave block per CU, so its LDS is free to take): activation
// buffers of four k steps, one barrier per four steps, where K allows;
// otherwise, and for the down projection (two blocks per CU), two.
template <int FMT, int TN, int WPB, int STAGE>
static hipError_t run_prefill_wide(GemmArgs a, int64_t R, const GemmLaunch &s) {
  if constexpr (STAGE != 1 && TN == 2 && WPB == 8) {
    if (a.K % (4 * kWK) == 0) return run_prefill_wide1<FMT, TN, WPB, STAGE, 4>(a, R, s);
  }
  return run_prefill_wide1<FMT, TN, WPB, STAGE, TN == 4 ? 4 : 2>(a, R, s);
}

template <int FMT>
static hipError_t run_decode_down_tok(GemmArgs a, const GemmLaunch &s) {
  // one token: 8 columns per block (H / 8 blocks); more: 16
  if (a.T == 1)
    hipExtLaunchKernelGGL((gemm_decode_down_tok<FMT, 8>), dim3((unsigned)(a.N / 8), 1u), dim3(512), 0u,
                          s.stream, s.start, s.stop, 0u, a);
  else
    hipExtLaunchKernelGGL((gemm_decode_down_tok<FMT, 16>), dim3((unsigned)(a.N / 16), (unsigned)a.T), dim3(512),
                          0u, s.stream, s.start, s.stop, 0u, a);
  return hipGetLastError();
}

bool down_writes_output(const LayerDims &L, const FwdPtrs &P, bool decode) {
  return decode && !P.w8a8 && P.act_g13 == 0.f && P.T <= kTokDownMaxT && L.H % 16 == 0 && L.I % 64 == 0;
}

template <int FMT>
static hipError_t run_decode_stream(GemmArgs a, const GemmLaunch &s) {
  if (a.K > kDSMaxK || a.K % 256) return hipErrorInvalidValue;
  a.tiles = (a.I + 127) / 128;  // units per 16-row chunk
  raise_lds_limit((const void *)gemm_decode_stream<FMT>);
  hipExtLaunchKernelGGL((gemm_decode_stream<FMT>), dim3((unsigned)num_cus()), dim3(512),
                        (uint32_t)kDSLds, s.stream, s.start, s.stop, 0u, a);
  return hipGetLastError();
}

template <int STAGE>
static hipError_t dispatch(const LayerDims &L, const FwdPtrs &P, const Workspace &W, bool decode,
                           const GemmLaunch &s) {
  GemmArgs a = make_args(L, P, W, STAGE);
  const int64_t R = (int64_t)P.T * L.k;
  const int slots = (int)(R < L.E ? R : L.E);
  if constexpr (STAGE == 0) {
    if (decode && use_decode_stream(L.H, L.E, L.k, P.T)) {
      switch (L.fmt) {
        case FMT_INT4: return run_decode_stream<FMT_INT4>(a, s);
        case FMT_FP8: return run_decode_stream<FMT_FP8>(a, s);
        default: return run_decode_stream<FMT_NVFP4>(a, s);
      }
    }
  }
  if constexpr (STAGE == 1) {
    if (down_writes_output(L, P, decode)) {
      switch (L.fmt) {
        case FMT_INT4: return run_decode_down_tok<FMT_INT4>(a, s);
        case FMT_FP8: return run_decode_down_tok<FMT_FP8>(a, s);
        default: return run_decode_down_tok<FMT_NVFP4>(a, s);
      }
    }
  }
  if (decode) {
    switch (L.fmt) {
      case FMT_INT4: return run_decode_ks<FMT_INT4, STAGE>(a, slots, s);
      case FMT_FP8: return run_decode_ks<FMT_FP8, STAGE>(a, slots, s);
      default: return run_decode_ks<FMT_NVFP4, STAGE>(a, slots, s);
    }
  }
  // Two 32-column tiles per wave, two waves per SIMD.  gate/up: 8 waves per
  // block, so each staged activation tile feeds 512 weight columns (FP8
  // T=4096 gate/up 260 -> 246 us, NVFP4 Zipf 834 -> 806 us against 4 waves);
  // down (K = I = 768): 4 waves per block, two blocks per CU, whose prologue
  // and epilogue overlap each other (8 waves measured slower there).
  constexpr int WPB = STAGE == 0 ? 8 : 4;
  if constexpr (STAGE == 0) {
    if (P.act_g13 > 0.f) {  // W4A4: h quantized in the epilogue
      if (L.fmt != FMT_NVFP4) return hipErrorInvalidValue;
      return run_prefill_wide<FMT_NVFP4, 2, WPB, 2>(a, R, s);
    }
  }
  switch (L.fmt) {
    case FMT_INT4: return run_prefill_wide<FMT_INT4, 2, WPB, STAGE>(a, R, s);
    case FMT_FP8: return run_prefill_wide<FMT_FP8, 2, WPB, STAGE>(a, R, s);
    default: return run_prefill_wide<FMT_NVFP4, 2, WPB, STAGE>(a, R, s);
  }
}

hipError_t launch_gate_up(const LayerDims &L, const FwdPtrs &P, const Workspace &W, bool decode,
                          const GemmLaunch &s) {
  return dispatch<0>(L, P, W, decode, s);
}

hipError_t launch_down(const LayerDims &L, const FwdPtrs &P, const Workspace &W, bool decode,
                       const GemmLaunch &s) {
  return dispatch<1>(L, P, W, decode, s);
}

hipError_t launch_combine(const LayerDims &L, const FwdPtrs &P, const Workspace &W, hipStream_t s) {
  const size_t items = (size_t)P.T * (L.H / 8);
  const bool stream = (size_t)P.T * L.k * L.H * sizeof(_Float16) > ((size_t)256 << 20);
  const dim3 grid((unsigned)((items + 255) / 256)), block(256);
  const _Float16 *partial = (const _Float16 *)(P.ws + W.partial);
  if (stream)
    hipLaunchKernelGGL(combine_kernel<true>, grid, block, 0, s, partial, P.residual, P.out, P.T, L.H, L.k);
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, block, 0, s, partial, P.residual, P.out, P.T, L.H, L.k);
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

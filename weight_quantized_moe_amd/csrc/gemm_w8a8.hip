// W8A8 block FP8 grouped GEMMs: the FP8 layer with dynamic 1x128 FP8
// activations.  The "clef-omni-fp8" card, table "What was quantized", runs the
// thinker experts' activations as "dynamic FP8 per 1x128 group in engines";
// the weights are the card's E4M3 codes with one FP32 scale per 128x128 block.
//
// Both operands are E4M3 codes, so the contraction runs on gfx950's FP8
// matrix instruction (32x32x64, twice the FP16 rate) with no unpack.  For a
// 128-wide k block g, with activation scale sa[row, g] and weight scale
// sw[n / 128, g]:
//     acc[n, row] += (sum_{k in g} a[row, k] w[n, k]) * (sa[row, g] * sw[n / 128, g])
// the inner sum from two MFMAs in FP32 (products of E4M3 values are exact in
// FP32), the scale product one FP32 multiply, the update one FMA.
//
// Block: 8 waves over 128 grouped rows of one expert; wave (cg, rh) = (w % 4,
// w / 4) owns rows 64 rh + [0, 64) (two 32-row subtiles) and two 32-column
// weight tiles:
//   gate/up: gate columns 32 cg + [0, 32) of the block's 128 and the matching
//            up columns, so SwiGLU runs in registers and the block's 128 h
//            columns are exactly one 128-wide quantization group of h;
//   down:    output columns 64 cg + [0, 64) of the block's 256.
// The activation codes of a 128-wide k step go through LDS (written once by
// the block, two buffers); each wave streams its weight codes from global
// memory into registers one k step ahead.  MFMA operand layout (both
// operands the same): lane l holds row l % 32 and the 32 bytes k = 32 (l / 32)
// + [0, 32) of a 64-wide sub-step.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device.h"
#include "internal.h"

namespace mq {

typedef int i8v __attribute__((ext_vector_type(8)));

struct W8Args {
  const uint8_t *w;       // E4M3 weights [E, N, K]
  const float *wscale;    // [E, N/128, K/128]
  int N, K, E, I, H;
  const int32_t *offsets, *mtile;
  const int4 *rowinfo;    // {slot, token, -, routing weight bits} per grouped row
  const uint8_t *a;       // activation codes: gate/up x [T, H] by token; down h [R, I] by grouped row
  const float *as;        // their scales [., K/128]
  uint8_t *hq;            // gate/up output: h codes [R, I]
  float *hs;              // and scales [R, I/128]
  _Float16 *partial;      // down output [R, H] by slot (FP16, routing-weighted)
  uint32_t *flags;
  int tiles;              // N tiles of a launch
};

constexpr int kW8BM = 128;   // grouped rows per M tile (= kPrefillBM: the mtile prefix)
constexpr int kW8K = 128;    // k step = one scale block
constexpr int kW8LD = 144;   // LDS row stride of the activation tile, bytes
constexpr int kW8MaxG = kMaxGemmK / 128;
static_assert(kW8BM == kPrefillBM, "tiles follow the grouping's M-tile prefix");

__device__ __forceinline__ f16v mfma_fp8(const i8v &a, const i8v &b, const f16v &c) {
  // E8M0 scale 127 = 2^0 on both operands: the plain E4M3 x E4M3 product
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

template <int STAGE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_w8a8(W8Args a) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint8_t *abuf = smem;                                         // [2][128][kW8LD]
  float *rsc = (float *)(smem + 2 * kW8BM * kW8LD);             // [128][G] activation scales of the tile rows
  float *hmax = rsc + kW8BM * kW8MaxG;                          // [4][128] (gate/up)
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int cg = wave & 3, rh = wave >> 2, j = lane & 31, hh = lane >> 5;
  // ---- tile of this block (dealt to the 8 XCDs in contiguous ranges)
  const int NT = a.tiles;
  const int n_tiles = a.mtile[a.E] * NT;
  const int per_xcd = (n_tiles + 7) >> 3;
  const int xslot = blockIdx.x >> 3;
  if (xslot >= per_xcd) return;
  const int Lt = (blockIdx.x & 7) * per_xcd + xslot;
  if (Lt >= n_tiles) return;
  const int mt = Lt / NT, nt = Lt - mt * NT;
  int lo = 0, hi = a.E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.mtile[mid] <= mt) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  const int rbeg = a.offsets[e] + (mt - a.mtile[e]) * kW8BM;
  const int nrows = min(kW8BM, a.offsets[e + 1] - rbeg);
  const int K = a.K, N = a.N, G = K / kW8K, nK = G;

  // ---- the wave's weight rows
  const int cb = STAGE == 0 ? nt * 128 + cg * 32 : nt * 256 + cg * 64;  // gate/up: first h column
  const bool wvalid = cb < (STAGE == 0 ? a.I : N);                      // wave-uniform
  int gr[2];
#pragma unroll
  for (int tn = 0; tn < 2; ++tn) {
    const int c = STAGE == 0 ? (tn == 0 ? cb : a.I + cb) + j : cb + 32 * tn + j;
    gr[tn] = wvalid ? c : j;  // a row that exists; never stored
  }
  const uint8_t *wsrc[2];
  const float *wsc[2];  // block scales of the tile's 128-row weight block (wave-uniform)
#pragma unroll
  for (int tn = 0; tn < 2; ++tn) {
    wsrc[tn] = a.w + ((size_t)e * N + gr[tn]) * K + 32 * hh;
    const int n0 = STAGE == 0 ? (tn == 0 ? cb : a.I + cb) : cb + 32 * tn;
    wsc[tn] = a.wscale + ((size_t)e * (N / 128) + (wvalid ? n0 : 0) / 128) * G;
  }

  // ---- activation rows of the tile: row (tid >> 3) + 64 p, 16-byte chunk tid & 7
  const uint8_t *asrc[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int rr = (tid >> 3) + 64 * p;
    const int r = rbeg + (rr < nrows ? rr : nrows - 1);
    asrc[p] = a.a + (STAGE == 0 ? (size_t)a.rowinfo[r].y : (size_t)r) * K + (tid & 7) * 16;
  }
  // activation scales of the tile's rows into LDS
  for (int idx = tid; idx < kW8BM * G; idx += 512) {
    const int rr = idx / G, g = idx - rr * G;
    const int r = rbeg + (rr < nrows ? rr : nrows - 1);
    rsc[rr * G + g] = a.as[(STAGE == 0 ? (size_t)a.rowinfo[r].y : (size_t)r) * G + g];
  }

  auto load_a = [&](u4 (&ar)[2], int ks) {
#pragma unroll
    for (int p = 0; p < 2; ++p) ar[p] = *(const u4 *)(asrc[p] + (size_t)ks * kW8K);
  };
  auto write_a = [&](const u4 (&ar)[2], int buf) {
#pragma unroll
    for (int p = 0; p < 2; ++p)
      *(u4 *)(abuf + (size_t)buf * kW8BM * kW8LD + ((tid >> 3) + 64 * p) * kW8LD + (tid & 7) * 16) = ar[p];
  };
  // weight codes of one k step: [tile][sub-step] x 32 bytes
  struct WRegs {
    i8v v[2][2];
  };
  auto load_w = [&](WRegs &R, int ks) {
#pragma unroll
    for (int tn = 0; tn < 2; ++tn)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const u4 *p = (const u4 *)(wsrc[tn] + (size_t)ks * kW8K + 64 * s);
        const u4 x0 = p[0], x1 = p[1];
        R.v[tn][s] = i8v{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                         (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
      }
  };

  f16v acc[2][2];
#pragma unroll
  for (int tn = 0; tn < 2; ++tn)
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[tn][tm][i] = 0.f;
  // 32-row subtiles of the wave that hold rows of the expert (wave-uniform)
  const int nsub = wvalid ? max(0, min(2, (nrows - 64 * rh + 31) / 32)) : 0;

  // one k step from LDS buffer `buf`: the 2 x 2 tiles' eight MFMAs first
  // (two per tile, 64 k each, into a per-step partial), then the scale FMAs,
  // which overlap the later MFMAs; NS = 32-row subtiles with rows
  auto compute = [&](auto ns_c, const WRegs &R, int buf, int ks) {
    constexpr int NS = decltype(ns_c)::value;
    if constexpr (NS > 0) {
      const uint8_t *As = abuf + (size_t)buf * kW8BM * kW8LD + 32 * hh;
      i8v b[NS][2];
#pragma unroll
      for (int tm = 0; tm < NS; ++tm)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const u4 *p = (const u4 *)(As + (64 * rh + 32 * tm + j) * kW8LD + 64 * s);
          const u4 x0 = p[0], x1 = p[1];
          b[tm][s] = i8v{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
        }
      float sa[NS];
#pragma unroll
      for (int tm = 0; tm < NS; ++tm) sa[tm] = rsc[(64 * rh + 32 * tm + j) * G + ks];
      const float s0 = wsc[0][ks], s1 = wsc[1][ks];
      f16v z;
#pragma unroll
      for (int i = 0; i < 16; ++i) z[i] = 0.f;
      f16v tmp[2][NS];
#pragma unroll
      for (int tm = 0; tm < NS; ++tm)
#pragma unroll
        for (int tn = 0; tn < 2; ++tn) tmp[tn][tm] = mfma_fp8(R.v[tn][0], b[tm][0], z);
#pragma unroll
      for (int tm = 0; tm < NS; ++tm)
#pragma unroll
        for (int tn = 0; tn < 2; ++tn) tmp[tn][tm] = mfma_fp8(R.v[tn][1], b[tm][1], tmp[tn][tm]);
#pragma unroll
      for (int tm = 0; tm < NS; ++tm) {
        const float f0 = sa[tm] * s0, f1 = sa[tm] * s1;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          acc[0][tm][i] = __builtin_fmaf(tmp[0][tm][i], f0, acc[0][tm][i]);
          acc[1][tm][i] = __builtin_fmaf(tmp[1][tm][i], f1, acc[1][tm][i]);
        }
      }
    }
  };

  // ---- main loop: stage k step t + 1 while step t multiplies.  Unrolled by
  // two so the two weight register sets keep fixed names (selected by a
  // runtime index, the compiler would place them in scratch memory).
  auto main_loop = [&](auto ns_c) {
    WRegs R0, R1;
    u4 ar[2];
    load_a(ar, 0);
    load_w(R0, 0);
    write_a(ar, 0);
    if (nK > 1) load_a(ar, 1);
    for (int t = 0; t < nK; t += 2) {
      __syncthreads();  // buffer 0 holds step t; buffer 1 is free
      if (t + 1 < nK) {
        write_a(ar, 1);
        if (t + 2 < nK) load_a(ar, t + 2);
        load_w(R1, t + 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      compute(ns_c, R0, 0, t);
      if (t + 1 < nK) {
        __syncthreads();  // buffer 1 holds step t + 1; buffer 0 is free
        if (t + 2 < nK) {
          write_a(ar, 0);
          if (t + 3 < nK) load_a(ar, t + 3);
          load_w(R0, t + 2);
        }
        __builtin_amdgcn_sched_barrier(0);
        compute(ns_c, R1, 1, t + 1);
      }
    }
  };
  switch (nsub) {
    case 2: main_loop(std::integral_constant<int, 2>{}); break;
    case 1: main_loop(std::integral_constant<int, 1>{}); break;
    default: main_loop(std::integral_constant<int, 0>{}); break;
  }

  uint32_t sat = 0u;
  typedef uint32_t u2 __attribute__((ext_vector_type(2)));
  if constexpr (STAGE == 0) {
    // ---- SwiGLU, then 1x128 FP8 quantization of h: the block's 128 h columns
    // are one group, so a row's maximum is the max over the 4 column waves
    float hv[2][16];
#pragma unroll
    for (int tm = 0; tm < 2; ++tm) {
      float m = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        hv[tm][i] = silu(acc[0][tm][i]) * acc[1][tm][i];
        m = fmaxf(m, fabsf(hv[tm][i]));
      }
      m = fmaxf(m, __shfl_xor(m, 32, 64));  // lanes l and l + 32 hold the same row
      if (hh == 0) hmax[cg * kW8BM + 64 * rh + 32 * tm + j] = wvalid ? m : 0.f;
    }
    __syncthreads();
    if (wvalid) {
      const int Ig = a.I / 128;
#pragma unroll
      for (int tm = 0; tm < 2; ++tm) {
        const int row = 64 * rh + 32 * tm + j;
        if (row >= nrows) continue;
        float m = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) m = fmaxf(m, hmax[c * kW8BM + row]);
        const float s = fp8_group_scale(m);
        const int r = rbeg + row;
        // register v holds column 8 (v / 4) + 4 (l / 32) + v % 4 of the tile
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *(uint32_t *)(a.hq + (size_t)r * a.I + cb + 8 * g4 + 4 * hh) =
              e4m3x4(hv[tm][4 * g4], hv[tm][4 * g4 + 1], hv[tm][4 * g4 + 2], hv[tm][4 * g4 + 3], s);
        if (cg == 0 && hh == 0) a.hs[(size_t)r * Ig + nt] = s;
      }
    }
  } else {
    // ---- down: routing-weighted FP16 partials, each 32-row slice of the
    // wave's tile transposed through LDS and stored 16 bytes per lane
    constexpr int TL = 64 + 8;  // LDS row stride, halves
    static_assert(8 * 32 * TL * 2 <= 2 * kW8BM * kW8LD, "transpose buffers fit the activation buffers");
    _Float16 *tb = (_Float16 *)smem + wave * 32 * TL;
    float vmax = 0.f, vnan = 0.f;
    __syncthreads();  // every wave is done with the activation buffers
    if (wvalid) {
#pragma unroll
      for (int tm = 0; tm < 2; ++tm) {
        if (64 * rh + 32 * tm >= nrows) break;
        const int row = 64 * rh + 32 * tm + j;
        const float wt = row < nrows ? __builtin_bit_cast(float, a.rowinfo[rbeg + row].w) : 0.f;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
          for (int tn = 0; tn < 2; ++tn) {
            h2 o[2];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float v = acc[tn][tm][4 * g4 + i] * wt;
              vmax = fmaxf(vmax, fabsf(v));
              vnan = __builtin_fmaf(v, 0.f, vnan);
              o[i >> 1][i & 1] = (_Float16)fminf(fmaxf(v, -65504.f), 65504.f);
            }
            *(u2 *)(tb + j * TL + tn * 32 + 8 * g4 + 4 * hh) = u2{as_u32(o[0]), as_u32(o[1])};
          }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the wave reads what it wrote
        __builtin_amdgcn_wave_barrier();
        const int ch = lane & 7;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int rr = it * 8 + (lane >> 3);
          const int orow = 64 * rh + 32 * tm + rr;
          const u4 v = *(const u4 *)(tb + rr * TL + ch * 8);
          if (orow < nrows) *(u4 *)(a.partial + (size_t)a.rowinfo[rbeg + orow].x * a.H + cb + ch * 8) = v;
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_wave_barrier();
      }
    }
    sat |= !(vmax <= 65504.f) || vnan != 0.f;
  }
  if (__builtin_amdgcn_ballot_w64(sat != 0u) != 0ull && lane == 0) atomicOr(a.flags, 1u);
}

static size_t w8a8_lds(int) {
  return (size_t)2 * kW8BM * kW8LD + (size_t)kW8BM * kW8MaxG * 4 + (size_t)4 * kW8BM * 4;
}

template <int STAGE>
static hipError_t run_w8a8(const LayerDims &L, const FwdPtrs &P, const Workspace &W, const GemmLaunch &s) {
  char *ws = P.ws;
  W8Args a;
  a.E = L.E; a.I = L.I; a.H = L.H;
  const int64_t T = P.T, R = T * L.k;
  if (STAGE == 0) {
    a.w = L.w13; a.wscale = (const float *)L.s13; a.N = 2 * L.I; a.K = L.H;
    a.a = (const uint8_t *)(ws + W.x16);
    a.as = (const float *)(ws + W.x16 + (size_t)T * L.H);
    a.tiles = (L.I + 127) / 128;
  } else {
    a.w = L.w2; a.wscale = (const float *)L.s2; a.N = L.H; a.K = L.I;
    a.a = (const uint8_t *)(ws + W.h);
    a.as = (const float *)(ws + W.h + (size_t)R * L.I);
    a.tiles = (L.H + 255) / 256;
  }
  a.hq = (uint8_t *)(ws + W.h);
  a.hs = (float *)(ws + W.h + (size_t)R * L.I);
  a.offsets = (const int32_t *)(ws + W.offsets);
  a.mtile = (const int32_t *)(ws + W.mtile);
  a.rowinfo = (const int4 *)(ws + W.rowinfo);
  a.partial = (_Float16 *)(ws + W.partial);
  a.flags = P.flags;
  const int64_t max_mt = R / kW8BM + L.E;  // >= sum_e ceil(n_e / 128)
  const int64_t grid = 8 * ((max_mt * a.tiles + 7) / 8);
  const size_t lds = w8a8_lds(a.K);
  static_assert(2 * kW8BM * kW8LD + kW8BM * kW8MaxG * 4 + 4 * kW8BM * 4 <= kMaxLdsBytes, "LDS");
  raise_lds_limit((const void *)gemm_w8a8<STAGE>);
  hipExtLaunchKernelGGL((gemm_w8a8<STAGE>), dim3((unsigned)grid), dim3(512), (uint32_t)lds, s.stream, s.start,
                        s.stop, 0u, a);
  return hipGetLastError();
}

hipError_t launch_w8a8_gate_up(const LayerDims &L, const FwdPtrs &P, const Workspace &W,
                               const GemmLaunch &s) {
  return run_w8a8<0>(L, P, W, s);
}
hipError_t launch_w8a8_down(const LayerDims &L, const FwdPtrs &P, const Workspace &W,
                            const GemmLaunch &s) {
  return run_w8a8<1>(L, P, W, s);
}

}  // namespace mq

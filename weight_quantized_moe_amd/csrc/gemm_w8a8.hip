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
constexpr int kW8BN = 256;   // weight rows per block (gate/up: 128 gate + 128 up; down: 256 outputs)
constexpr int kW8K = 128;    // k step = one scale block
constexpr int kW8Stages = 3; // k steps in flight through LDS
// one stage: activation codes [128 rows][128 B], weight codes [256 rows][128 B],
// activation scales [128]
constexpr int kW8ABytes = kW8BM * kW8K;
constexpr int kW8WBytes = kW8BN * kW8K;
constexpr int kW8StageBytes = kW8ABytes + kW8WBytes + kW8BM * 4;
static_assert(kW8BM == kPrefillBM, "tiles follow the grouping's M-tile prefix");
constexpr int kW8MaxG = kMaxGemmK / kW8K;
constexpr int kW8Lds = kW8Stages * kW8StageBytes + 4 * kW8BM * 4 + 2 * kW8MaxG * 4 + kW8BM * 16;
static_assert(kW8Lds <= kMaxLdsBytes, "stages fit in LDS");

__device__ __forceinline__ f16v mfma_fp8(const i8v &a, const i8v &b, const f16v &c) {
  // E8M0 scale 127 = 2^0 on both operands: the plain E4M3 x E4M3 product
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// LDS position (16-byte slot) of chunk c (16 bytes of k) of row r of a stage
// array: rows of 8 slots, the chunk index XOR-swizzled by bits 1..3 of the row
// so that 16 consecutive rows reading the same chunk hit distinct banks.
__device__ __forceinline__ int w8_slot(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

typedef __attribute__((address_space(3))) void lds_void;
// Asynchronous copy of 16 (or 4) bytes per lane from global memory into LDS
// at lds + 16 (4) * lane; completion is tracked by the wave's vmcnt.
__device__ __forceinline__ void dma16(const void *g, unsigned char *lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void *)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void *g, unsigned char *lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void *)lds, 4, 0, 0);
}
// s_waitcnt vmcnt(n), other counters left alone
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Main loop: k step t's operands (activation codes and scales, weight codes)
// are copied into stage t % 3 by the block's waves, global memory straight
// into LDS, two k steps ahead of their use; one barrier per k step, after
// which every wave reads its MFMA operands from the stage.  Per k step a wave
// issues 2 activation and 4 weight copies of 1 KB (waves 0 and 1 one more of
// 256 B for the activation scales).
template <int STAGE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_w8a8(W8Args a) {
  extern __shared__ __align__(16) unsigned char smem[];
  float *hmax = (float *)(smem + kW8Stages * kW8StageBytes);   // [4][128] (gate/up)
  float *sws = hmax + 4 * kW8BM;                                // [2][G]: the block's weight scales
  int4 *rmeta = (int4 *)(sws + 2 * kW8MaxG);                    // [128]: the tile's row records (down)
  // the wave index as a scalar, so that per-wave addresses and the weight
  // scale loads stay in scalar registers
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
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

  // ---- the wave's weight rows (stage-local 0..255) and their block scales
  // gate/up: wave cg holds h columns cb + [0, 32): gate rows 32 cg + [0, 32),
  // up rows 128 + 32 cg + [0, 32) of the stage; down: rows 64 cg + [0, 64)
  const int cb = STAGE == 0 ? nt * 128 + cg * 32 : nt * 256 + cg * 64;
  const bool wvalid = cb < (STAGE == 0 ? a.I : N);  // wave-uniform
  int wrow[2], wblk[2];  // stage row of each tile; its 128-row weight block (0 or 1) of the block's two
#pragma unroll
  for (int tn = 0; tn < 2; ++tn) {
    wrow[tn] = STAGE == 0 ? 128 * tn + 32 * cg : 64 * cg + 32 * tn;
    wblk[tn] = STAGE == 0 ? tn : cg >> 1;
  }
  // the block's two weight blocks' scales [2][G] into LDS (gate/up: the gate
  // block of h columns nt * 128 + [0, 128) and its up block; down: weight
  // rows nt * 256 + [0, 128) and [128, 256)); blocks past the end read as 0
  for (int idx = tid; idx < 2 * G; idx += 512) {
    const int b = idx / G, g = idx - b * G;
    const int n0 = STAGE == 0 ? (b == 0 ? nt * 128 : a.I + nt * 128) : nt * 256 + 128 * b;
    const bool ok = STAGE == 0 ? nt * 128 < a.I : n0 < N;
    sws[idx] = ok ? a.wscale[((size_t)e * (N / 128) + n0 / 128) * G + g] : 0.f;
  }

  // the down epilogue's row records (slot, routing weight), read now so that
  // the epilogue issues no global load between its stores
  if (STAGE == 1 && tid < kW8BM) rmeta[tid] = tid < nrows ? a.rowinfo[rbeg + tid] : int4{0, 0, 0, 0};

  // ---- copy sources of this lane: activation copies q = 2 wave + [0, 2)
  // and weight copies q = 4 wave + [0, 4) of each k step; copy q's lane i
  // fills slot 64 q + i, i.e. row 8 q + i / 8 at swizzled chunk i % 8
  const int csl = lane & 7;
  const uint8_t *asrc[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int r = 8 * (2 * wave + p) + (lane >> 3);
    const int c = csl ^ ((r >> 1) & 7);
    const int rr = rbeg + (r < nrows ? r : nrows - 1);
    asrc[p] = a.a + (STAGE == 0 ? (size_t)a.rowinfo[rr].y : (size_t)rr) * K + 16 * c;
  }
  const uint8_t *wsrc[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int r = 8 * (4 * wave + p) + (lane >> 3);  // stage weight row 0..255
    const int c = csl ^ ((r >> 1) & 7);
    int n;
    if (STAGE == 0) {
      const int hc = nt * 128 + (r & 127);            // h column of this gate or up row
      n = hc < a.I ? (r < 128 ? hc : a.I + hc) : 0;   // rows past I: any row, never stored
    } else {
      n = nt * 256 + r;
      n = n < N ? n : 0;
    }
    wsrc[p] = a.w + ((size_t)e * N + n) * K + 16 * c;
  }
  // activation scales: waves 0 and 1 copy rows 64 wave + lane
  const float *ssrc = a.as;
  if (wave < 2) {
    const int r = 64 * wave + lane;
    const int rr = rbeg + (r < nrows ? r : nrows - 1);
    ssrc = a.as + (STAGE == 0 ? (size_t)a.rowinfo[rr].y : (size_t)rr) * G;
  }
  auto issue = [&](int ks) {
    unsigned char *st = smem + (ks % kW8Stages) * kW8StageBytes;
#pragma unroll
    for (int p = 0; p < 2; ++p) dma16(asrc[p] + (size_t)ks * kW8K, st + 1024 * (2 * wave + p));
#pragma unroll
    for (int p = 0; p < 4; ++p) dma16(wsrc[p] + (size_t)ks * kW8K, st + kW8ABytes + 1024 * (4 * wave + p));
    if (wave < 2) dma4(ssrc + ks, st + kW8ABytes + kW8WBytes + 256 * wave);
  };
  // wait for this wave's copies of the k step before the newest `later` steps
  auto wait_step = [&](int later) {
    if (wave < 2) {
      if (later) wait_vm<7>(); else wait_vm<0>();
    } else {
      if (later) wait_vm<6>(); else wait_vm<0>();
    }
  };
  static_assert(kW8Stages == 3, "wait_step counts one later k step in flight");

  f16v acc[2][2];
#pragma unroll
  for (int tn = 0; tn < 2; ++tn)
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[tn][tm][i] = 0.f;
  // 32-row subtiles of the wave that hold rows of the expert (wave-uniform)
  const int nsub = wvalid ? max(0, min(2, (nrows - 64 * rh + 31) / 32)) : 0;

  // one k step from its stage: the 2 x 2 tiles' eight MFMAs first (two per
  // tile, 64 k each, into a per-step partial), then the scale FMAs, which
  // overlap the later MFMAs; NS = 32-row subtiles with rows
  auto compute = [&](auto ns_c, int ks) {
    constexpr int NS = decltype(ns_c)::value;
    if constexpr (NS > 0) {
      const float s0 = sws[wblk[0] * G + ks], s1 = sws[wblk[1] * G + ks];
      const unsigned char *st = smem + (ks % kW8Stages) * kW8StageBytes;
      const unsigned char *Ws = st + kW8ABytes;
      const float *Ss = (const float *)(st + kW8ABytes + kW8WBytes);
      i8v w[2][2], b[NS][2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int c0 = 4 * s + 2 * hh;
#pragma unroll
        for (int tn = 0; tn < 2; ++tn) {
          const int r = wrow[tn] + j;
          const u4 x0 = *(const u4 *)(Ws + 16 * w8_slot(r, c0));
          const u4 x1 = *(const u4 *)(Ws + 16 * w8_slot(r, c0 + 1));
          w[tn][s] = i8v{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
        }
#pragma unroll
        for (int tm = 0; tm < NS; ++tm) {
          const int r = 64 * rh + 32 * tm + j;
          const u4 x0 = *(const u4 *)(st + 16 * w8_slot(r, c0));
          const u4 x1 = *(const u4 *)(st + 16 * w8_slot(r, c0 + 1));
          b[tm][s] = i8v{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
        }
      }
      float sa[NS];
#pragma unroll
      for (int tm = 0; tm < NS; ++tm) sa[tm] = Ss[64 * rh + 32 * tm + j];
      f16v z;
#pragma unroll
      for (int i = 0; i < 16; ++i) z[i] = 0.f;
      f16v tmp[2][NS];
#pragma unroll
      for (int tm = 0; tm < NS; ++tm)
#pragma unroll
        for (int tn = 0; tn < 2; ++tn) tmp[tn][tm] = mfma_fp8(w[tn][0], b[tm][0], z);
#pragma unroll
      for (int tm = 0; tm < NS; ++tm)
#pragma unroll
        for (int tn = 0; tn < 2; ++tn) tmp[tn][tm] = mfma_fp8(w[tn][1], b[tm][1], tmp[tn][tm]);
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

  auto main_loop = [&](auto ns_c) {
    for (int s = 0; s < kW8Stages - 1 && s < nK; ++s) issue(s);
    for (int t = 0; t < nK; ++t) {
      wait_step(t + 1 < nK);
      // step t is in its stage; every wave is done with step t - 1's.  A bare
      // barrier: __syncthreads' fence would also wait for the copies of step
      // t + 1, which are meant to stay in flight
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (t + kW8Stages - 1 < nK) issue(t + kW8Stages - 1);
      compute(ns_c, t);
    }
  };
  __syncthreads();  // the weight scales
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
    static_assert(8 * 32 * TL * 2 <= kW8Stages * kW8StageBytes, "transpose buffers fit the stages");
    _Float16 *tb = (_Float16 *)smem + wave * 32 * TL;
    float vmax = 0.f, vnan = 0.f;
    __syncthreads();  // every wave is done with the activation buffers
    if (wvalid) {
#pragma unroll
      for (int tm = 0; tm < 2; ++tm) {
        if (64 * rh + 32 * tm >= nrows) break;
        const int row = 64 * rh + 32 * tm + j;
        const float wt = row < nrows ? __builtin_bit_cast(float, rmeta[row].w) : 0.f;
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
          if (orow < nrows) *(u4 *)(a.partial + (size_t)rmeta[orow].x * a.H + cb + ch * 8) = v;
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_wave_barrier();
      }
    }
    sat |= !(vmax <= 65504.f) || vnan != 0.f;
  }
  if (__builtin_amdgcn_ballot_w64(sat != 0u) != 0ull && lane == 0) atomicOr(a.flags, 1u);
}

static size_t w8a8_lds(int) { return (size_t)kW8Lds; }

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

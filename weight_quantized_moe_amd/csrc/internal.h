// Internal declarations shared by the host ABI and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>

#include "../../include/moe_quant.h"
#include <stddef.h>
#include <stdint.h>

namespace mq {

constexpr int kMaxExperts = 512;
// Grouping in one workgroup (token bit masks per expert) up to these sizes.
constexpr int kSmallT = 256;      // tokens
constexpr int kSmallRows = 4096;  // routed rows T k
constexpr int kFusedT = 16;       // decode: routing and grouping in one launch up to this many tokens
constexpr int kMaxGateExperts = 256;  // experts the fused router + top-k kernel holds in LDS
// Batches of at least this many tokens route from the gate's weight with the
// fused router + top-k kernel; smaller ones run the router-logits kernel into
// the workspace, then the routing kernel (measured faster there: the fused
// kernel's block runs its GEMM, top-k and row staging back to back).
constexpr int64_t kGateFusedMinT = 4096;
constexpr int kPrefillBM = 128;  // token rows per prefill M-tile
constexpr int kMaxChunks = 256;  // token chunks of the three-launch grouping
// Hidden rows of at most this many values are read whole into the registers
// of one wave by the routing kernel, which then also finds each row's power of
// two (and, for prefill, writes the FP16 row); longer rows are scanned by the
// GEMM that stages them (decode) or in two passes (prefill).
constexpr int kRowRegsMaxH = 2048;

// LDS of one workgroup on gfx950 (bytes).
constexpr size_t kMaxLdsBytes = 160 * 1024;
constexpr int kDecodeRows = 16;  // rows of one decode unit staged in LDS

// Dynamic LDS of the decode GEMM for input dimension K and k split ks: the
// unit's FP16 rows [16][K + 8], row scales, and the k-split reduction tiles.
constexpr size_t decode_lds_bytes(int K, int ks) {
  return (size_t)kDecodeRows * (K + 8) * 2 + 48 * 4 + (size_t)(ks - 1) * (8 / ks) * 512 * 4;
}
// Whether the decode GEMM's LDS fits for input dimension K at every k split.
constexpr bool decode_fits(int K) {
  for (int ks = 1; ks <= 8; ks *= 2)
    if (decode_lds_bytes(K, ks) > kMaxLdsBytes) return false;
  return true;
}

constexpr int kMaxGemmK = 4608;
static_assert(decode_lds_bytes(kMaxGemmK, 8) <= kMaxLdsBytes &&
                  decode_lds_bytes(kMaxGemmK + 128, 8) > kMaxLdsBytes,
              "kMaxGemmK is the largest multiple of 128 the decode GEMM can stage");

// Chunks of the grouping: at most kMaxChunks, each a multiple of 256 tokens.
inline void permute_chunks(int64_t T, int *nc, int *chunk) {
  int64_t n = (T + 255) / 256;
  if (n > kMaxChunks) n = kMaxChunks;
  if (n < 1) n = 1;
  int64_t c = (T + n - 1) / n;
  c = (c + 255) / 256 * 256;
  *chunk = (int)c;
  *nc = (int)((T + c - 1) / c);
}

// Workspace carve-up for one forward call over T tokens (offsets in bytes).
struct Workspace {
  size_t topk_ids, topk_w;     // int32 [R], float [R]            (R = T*k)
  size_t offsets;              // int32 [E+1]
  size_t active;               // int4 [1 + E]: {count, 16-row chunks}, then {expert, first row, rows, 0} per active expert
  size_t rowinfo;              // int4 [R]: {slot, token, row scale bits, routing weight bits} per grouped row
  size_t mtile;                // int32 [E+1]: prefix of ceil(n_e / kPrefillBM)
  size_t rcpre;                // int32 [E+1]: per active expert, prefix of its 16-row chunks ceil(n_e / 16)
  size_t sorted_slots;         // int32 [R]: slot t*k+j of each grouped row
  size_t inv_pos;              // int32 [R]
  size_t x16;                  // fp16 [T, H]: hidden rows scaled by 2^-s_t (INT4: k order of the unpack)
  size_t rowscale;             // float [T]: 2^s_t
  size_t logits;               // float [T, E]: router logits computed in-library (small batches)
  size_t h;                    // fp16 [R, I]
  size_t partial;              // fp16 [R, H]: routing-weighted expert outputs per slot
  size_t chunks;               // int32 [kMaxChunks, E]: per-chunk expert counts, then bases
  size_t flags;                // uint32 [4] at offset 0: bit 0 = an FP16 intermediate saturated
  size_t total;
};

Workspace workspace_layout(int64_t T, int E, int H, int I, int k);

struct LayerDims {
  int E, H, I, k, fmt;
  const uint8_t *w13, *w2;
  const void *s13, *s2;
  const float *g13, *g2;
};

struct FwdPtrs {
  const void *logits;
  int logits_bf16;
  const uint16_t *gate_w;  // BF16 router weight [E, H]: logits computed in-library (else null)
  float *p_logits;         // probe: the in-library logits [T, E] (may be null)
  int w8a8;                // FP8 layer with dynamic 1x128 FP8 activations
  float act_g13, act_g2;   // NVFP4 W4A4: global scales of the gate/up and down inputs (0: W4A16)
  const uint16_t *hidden;
  const uint16_t *residual;
  uint16_t *out;
  char *ws;
  uint32_t *flags;  // saturation flag word (the workspace's first word, or the caller's)
  int T;
  // probe outputs (may be null)
  int32_t *p_ids, *p_offsets, *p_sorted_tok, *p_inv;
  float *p_w;
  uint16_t *p_h;
};

// launchers (return hipGetLastError() after the launch)
hipError_t launch_route(const LayerDims &L, const FwdPtrs &P, const Workspace &W, bool decode,
                        hipStream_t s);
hipError_t launch_permute(const LayerDims &L, const FwdPtrs &P, const Workspace &W, bool decode,
                          hipStream_t s);
// Stream of a GEMM launch, and optional events that the runtime records at
// the start and the end of the kernel's own execution (null: none).
struct GemmLaunch {
  hipStream_t stream;
  hipEvent_t start, stop;
};
hipError_t launch_gate_up(const LayerDims &L, const FwdPtrs &P, const Workspace &W, bool decode,
                          const GemmLaunch &s);
hipError_t launch_down(const LayerDims &L, const FwdPtrs &P, const Workspace &W, bool decode,
                       const GemmLaunch &s);
hipError_t launch_combine(const LayerDims &L, const FwdPtrs &P, const Workspace &W, hipStream_t s);
// True when launch_down writes the layer output itself (the decode down
// projection with the combine fused in, for a few tokens): no combine launch.
bool down_writes_output(const LayerDims &L, const FwdPtrs &P, bool decode);
// True when launch_route also groups the rows (a few decode tokens): then
// launch_permute launches nothing.
bool route_groups(const LayerDims &L, const FwdPtrs &P, bool decode);
hipError_t launch_dequantize(const LayerDims &L, int which, int expert, float *out, hipStream_t s);
hipError_t launch_import_expert(const LayerDims &L, int e, const mq_src_proj &gate,
                                const mq_src_proj &up, const mq_src_proj &down, int gptq_offset,
                                uint32_t *bad, hipStream_t st);
// Allow up to 160 KiB of dynamic LDS for kernel f on the current device (once
// per device; thread safe).
void raise_lds_limit(const void *f);
hipError_t launch_quant_act(const float *x, int64_t rows, int K, uint8_t *codes, float *scales,
                            hipStream_t s);
hipError_t launch_quant_act_nvfp4(const float *x, int64_t rows, int K, float g, uint8_t *codes,
                                  uint8_t *scales, hipStream_t s);
hipError_t launch_w8a8_gate_up(const LayerDims &L, const FwdPtrs &P, const Workspace &W,
                               const GemmLaunch &s);
hipError_t launch_w8a8_down(const LayerDims &L, const FwdPtrs &P, const Workspace &W,
                            const GemmLaunch &s);
hipError_t launch_router_logits(const uint16_t *x, const uint16_t *w, float *out, int64_t T, int H,
                                int E, hipStream_t s);

// The forward path behind moe_quant_forward and its allocation-free variant:
// host checks, then the launch sequence on `stream`.  `flags` (nullable) is
// the saturation word to use instead of the workspace's first word.
mq_status forward_impl(const mq_layer *L, const void *router_logits, int32_t logits_dtype,
                       const uint16_t *hidden_bf16, const uint16_t *residual_bf16,
                       int64_t num_tokens, uint16_t *out_bf16, void *workspace,
                       size_t workspace_bytes, const mq_probe *probe, uint32_t *flags,
                       hipStream_t stream, const uint16_t *gate_w = nullptr,
                       float *logits_out = nullptr, int w8a8 = 0, float act_g13 = 0.f,
                       float act_g2 = 0.f);
// Record a status and its one-line explanation for moe_quant_last_error().
mq_status fail(mq_status s, const char *fmt, ...);
void clear_error();
// Bytes of workspace one forward over T tokens needs for layer L.
size_t workspace_bytes(const mq_layer *L, int64_t T);
constexpr int64_t kMaxTokens = 1 << 22;

// Rows per expert at or below which the decode (weight-streaming) GEMMs run.
bool use_decode_path(int64_t T, int E, int k, int H, int I);
// Decode batches whose gate/up projection runs the streaming decode GEMM: H
// (its K) a multiple of 256 and at most 2048, and at least 4 rows per expert
// on average (T = 64 at 128 experts, top-8; below that the register-streaming
// decode GEMM is faster, and for the down projection at every size).
inline bool use_decode_stream(int H, int E, int k, int64_t T) {
  return H <= 2048 && H % 256 == 0 && T * k >= (int64_t)4 * E;
}

}  // namespace mq

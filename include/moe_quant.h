/*
 * moe_quant.h - C ABI of libmoe_quant.so: the routed MoE expert layer with
 * block-quantized expert weights on AMD Instinct MI355X (gfx950).
 *
 * What the layer computes.  The model cards describe the thinker's routed
 * experts kept packed in GPU memory and dequantized per layer "just in time"
 * for one grouped matmul ("clef-omni-fp8" card, section "How this checkpoint
 * runs"; "clef-omni-int4" card, section "How this checkpoint runs";
 * "clef-omni-NVFP4" card, section "How it was made").  For T tokens with
 * hidden states x[T, H] and router logits l[T, E]:
 *
 *   ids[t, 0..k)  = the k largest logits of token t, in descending order, ties
 *                   to the lower expert id;
 *   w[t, j]       = softmax over the k selected logits;
 *   y[t]          = sum_j w[t, j] * W2[e] (silu(G) * U),   e = ids[t, j],
 *                   [G; U] = W13[e] x[t]  (gate rows first, then up rows),
 *                   silu(z) = z / (1 + exp(-z));
 *   out[t]        = bf16(y[t])  or  bf16(residual[t] + y[t]).
 *
 * W13[e] is [2I, H], W2[e] is [H, I]; both are stored per expert, stacked over
 * experts, row major with the input dimension K contiguous, in one of three
 * packed formats (see mq_wformat).  The router itself is not part of the
 * path: it stays a BF16 linear layer on every card ("clef-omni-int4" card,
 * section "Recipe": ignore_layers=mlp.gate); moe_quant_forward takes its
 * logits as an input, and moe_quant_forward_with_router computes them from
 * the gate's weight in the same kernel as the top-k.
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers, owned by the caller, row major
 *    and contiguous.  The library never allocates device memory, never copies
 *    weights and keeps no device state: init only borrows the weight pointers
 *    for the lifetime of the handle.
 *  - Every entry point returns an mq_status.  Argument checks run on the host
 *    before anything is enqueued; on failure nothing is enqueued and
 *    moe_quant_last_error() holds a one-line explanation (thread local).
 *    Nothing is printed and no exception crosses the ABI.
 *  - Work is enqueued asynchronously on the caller's HIP stream (a
 *    hipStream_t, passed as struct ihipStream_t *; NULL is the default stream).
 *  - A handle is immutable after init: concurrent forward calls, from any host
 *    threads, on different streams are safe as long as each uses its own
 *    workspace (the library's launch-shape caches are guarded by a lock).
 */
#ifndef MOE_QUANT_H
#define MOE_QUANT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_QUANT_ABI_VERSION 1u

struct ihipStream_t; /* hipStream_t */
struct ihipEvent_t;  /* hipEvent_t  */

typedef enum {
  MQ_OK = 0,
  MQ_E_NULL = 1,      /* a required pointer is NULL                                  */
  MQ_E_SHAPE = 2,     /* a dimension is out of range or not a multiple of the block  */
  MQ_E_ALIGN = 3,     /* a pointer is not aligned as required                        */
  MQ_E_FORMAT = 4,    /* unknown weight format                                       */
  MQ_E_DTYPE = 5,     /* unknown logits dtype                                        */
  MQ_E_WORKSPACE = 6, /* workspace NULL or smaller than moe_quant_workspace_size()   */
  MQ_E_ABI = 7,       /* descriptor built against another MOE_QUANT_ABI_VERSION      */
  MQ_E_HIP = 8,       /* a HIP launch or runtime call failed                         */
  MQ_E_OVERFLOW = 9   /* an FP16 intermediate saturated (moe_quant_check)           */
} mq_status;

/*
 * Packed weight formats.  N is a projection's output dim and K its input dim
 * (W13: N = 2I, K = H; W2: N = H, K = I).  4-bit codes are packed two per
 * byte, the even k in the low nibble.
 *
 * MQ_W_INT4_G128  INT4 W4A16, symmetric, one scale per 128 consecutive k of a
 *                 row ("clef-omni-int4" card, intro and section "What was
 *                 quantized").
 *     w      uint8   [E, N, K/2]    nibble c = q + 8 (offset binary)
 *     scale  float16 [E, N, K/128]
 *     weight = (c - 8) * scale[n, k/128]
 *
 * MQ_W_FP8_B128   FP8 E4M3 (OCP E4M3FN: bias 7, max 448, 0x7F/0xFF NaN) with
 *                 one FP32 scale per 128x128 block ("clef-omni-fp8" card,
 *                 sections "What was quantized" and "Recipe"; the stored scale
 *                 is weight_scale_inv, the dequantization multiplier).
 *     w      uint8   [E, N, K]      E4M3FN bits
 *     scale  float32 [E, N/128, K/128]
 *     weight = e4m3(w) * scale[n/128, k/128]
 *
 * MQ_W_NVFP4_G16  NVFP4: FP4 E2M1 values, one E4M3 scale per 16 weights along
 *                 k, one FP32 global scale per expert matrix
 *                 ("clef-omni-NVFP4" card, section "How it was made"; gate and
 *                 up are one concatenated matrix and share its global scale).
 *     w      uint8   [E, N, K/2]    E2M1 nibbles (bit 3 = sign)
 *     scale  uint8   [E, N, K/16]   E4M3FN bits
 *     gscale float32 [E]            global scale g = 448*6/amax
 *     weight = e2m1(c) * e4m3(scale[n, k/16]) / gscale[e]
 *
 * Dimension limits of this version: H and I multiples of 128 for every format,
 * 128 <= H, I <= 4608 (the decode GEMM stages 16 whole input rows of a
 * projection in the 160 KiB LDS of one workgroup), 1 <= k <= E <= 512, k <= 64.
 * The NVFP4 format itself only needs multiples of 16; this version's GEMM
 * tiles (128-wide k blocks and 128-row weight tiles) take multiples of 128
 * for NVFP4 too, which every Clef shape satisfies (hidden 2048, intermediate
 * 768).
 */
typedef enum { MQ_W_INT4_G128 = 1, MQ_W_FP8_B128 = 2, MQ_W_NVFP4_G16 = 3 } mq_wformat;

/* Router-logit element type; BF16 logits are widened exactly to FP32. */
typedef enum { MQ_F32 = 0, MQ_BF16 = 1 } mq_dtype;

typedef struct {
  uint32_t abi_version; /* must equal MOE_QUANT_ABI_VERSION                      */
  int32_t num_experts;  /* E                                                      */
  int32_t hidden;       /* H                                                      */
  int32_t intermediate; /* I (per expert)                                         */
  int32_t top_k;        /* k                                                      */
  int32_t format;       /* mq_wformat                                             */
  const void *w13;      /* gate_up weights [E, 2I, .], 16-byte aligned            */
  const void *w13_scale;/* its scales, 16-byte aligned                            */
  const float *w13_gscale; /* NVFP4 only: [E]; must be NULL for the other formats */
  const void *w2;       /* down weights [E, H, .], 16-byte aligned                */
  const void *w2_scale;
  const float *w2_gscale;
} mq_layer_desc;

typedef struct mq_layer mq_layer; /* opaque host object */

/* Stages of one forward call, in launch order (for mq_probe.events). */
enum {
  MQ_STAGE_ROUTE = 0,   /* top-k + softmax + FP16 staging of the hidden rows */
  MQ_STAGE_PERMUTE = 1, /* histogram, scan and stable grouping by expert     */
  MQ_STAGE_GATE_UP = 2, /* grouped gate/up GEMM with SwiGLU epilogue         */
  MQ_STAGE_DOWN = 3,    /* grouped down GEMM, routing-weighted per slot      */
  MQ_STAGE_COMBINE = 4, /* slot-ordered sum (+ residual), BF16 rounding      */
  MQ_NUM_STAGES = 5
};

/*
 * Optional extra outputs of a forward call, for tests and profiling.  Every
 * field may be NULL.  Device arrays are written in stream order:
 *   topk_ids         int32 [T, k]   selected experts, descending logit
 *   topk_w           float [T, k]   routing weights
 *   expert_offsets   int32 [E + 1]  grouped row range of each expert
 *   sorted_token_ids int32 [T * k]  token of each grouped row (experts
 *                                   ascending, tokens ascending inside one)
 *   inv_pos          int32 [T * k]  grouped row of slot t * k + j
 *   h                uint16 [T*k, I] FP16 bits of the SwiGLU intermediate in
 *                                   grouped row order
 * events[2 * s] / events[2 * s + 1] (hipEvent_t, created by the caller) are
 * recorded on the stream right before / after stage s; for the two GEMM
 * stages the runtime takes them at the start and the end of the GEMM kernel
 * itself (hipExtLaunchKernel), so they exclude the gap before its dispatch.
 */
typedef struct {
  int32_t *topk_ids;
  float *topk_w;
  int32_t *expert_offsets;
  int32_t *sorted_token_ids;
  int32_t *inv_pos;
  uint16_t *h;
  struct ihipEvent_t *events[2 * MQ_NUM_STAGES];
} mq_probe;

/*
 * Validate a layer descriptor and create a handle.  Host only: no HIP call is
 * made.  On MQ_OK *out holds a handle to release with moe_quant_destroy.
 * Errors: MQ_E_NULL (d, out or a weight pointer NULL; gscale NULL for NVFP4),
 * MQ_E_ABI, MQ_E_FORMAT, MQ_E_SHAPE (a dimension outside the limits above),
 * MQ_E_ALIGN.
 */
mq_status moe_quant_init(const mq_layer_desc *d, mq_layer **out);

/*
 * Device workspace bytes that one forward call over num_tokens tokens needs
 * (256-byte aligned start required).  num_tokens >= 0.  Host only.
 */
mq_status moe_quant_workspace_size(const mq_layer *L, int64_t num_tokens, size_t *bytes);

/*
 * Enqueue one layer forward on `stream`.
 *   router_logits  [T, E] of logits_dtype, 16-byte aligned
 *   hidden_bf16    [T, H] BF16 bits, 16-byte aligned
 *   residual_bf16  NULL, or [T, H]: then out = bf16(residual + moe(hidden))
 *   out_bf16       [T, H] BF16 bits, 16-byte aligned; may alias residual_bf16
 *   workspace      >= moe_quant_workspace_size(L, T) bytes, 256-byte aligned;
 *                  its contents on entry do not matter
 *   probe          NULL, or extra outputs (see mq_probe)
 * num_tokens == 0 returns MQ_OK without enqueuing anything.  Inputs must not
 * hold NaN or Inf; results are then unspecified but every access stays in
 * bounds.  Returns MQ_E_HIP if a launch fails.
 */
mq_status moe_quant_forward(const mq_layer *L, const void *router_logits, int32_t logits_dtype,
                            const uint16_t *hidden_bf16, const uint16_t *residual_bf16,
                            int64_t num_tokens, uint16_t *out_bf16, void *workspace,
                            size_t workspace_bytes, const mq_probe *probe,
                            struct ihipStream_t *stream);

/*
 * W8A8 block FP8: moe_quant_forward for an MQ_W_FP8_B128 layer with its
 * activations quantized to FP8 as the "clef-omni-fp8" card (table "What was
 * quantized") runs them in engines, "dynamic FP8 per 1x128 group": for each
 * token (gate/up input) and each grouped row (down input) and each 128
 * consecutive input features, s = amax / 448 (FP32) and code =
 * RNE-to-E4M3(x / s) saturated to +-448; the SwiGLU intermediate is quantized
 * from its FP32 value.  Both GEMMs run on the FP8 matrix units, the
 * activation and weight scales multiplying each 128-wide k block's FP32
 * partial sum.  Same arguments, workspace size and routing as
 * moe_quant_forward (the kernels are the many-rows-per-expert ones at every
 * batch size).  The probe's h buffer (T*k*I*2 bytes) receives h as kept
 * here: the E4M3 codes uint8 [T*k, I] in grouped row order, followed by their
 * FP32 scales [T*k, I/128].  Errors: as moe_quant_forward, plus MQ_E_FORMAT
 * for another weight format.
 */
mq_status moe_quant_forward_w8a8(const mq_layer *L, const void *router_logits, int32_t logits_dtype,
                                 const uint16_t *hidden_bf16, const uint16_t *residual_bf16,
                                 int64_t num_tokens, uint16_t *out_bf16, void *workspace,
                                 size_t workspace_bytes, const mq_probe *probe,
                                 struct ihipStream_t *stream);

/*
 * Test entry: the dynamic 1x128 FP8 activation quantizer of the W8A8 path on
 * FP32 rows x [rows, K] (device), writing codes uint8 [rows, K] (E4M3FN bits)
 * and scales float [rows, K/128] (device, caller-owned), with the same group
 * arithmetic the W8A8 kernels apply to hidden rows and to the SwiGLU
 * intermediate.  K a positive multiple of 128 (at most 65536).
 * Errors: MQ_E_SHAPE, MQ_E_NULL, MQ_E_ALIGN, MQ_E_HIP.
 */
mq_status moe_quant_quantize_act(const float *x, int64_t rows, int32_t K, uint8_t *codes, float *scales,
                                 struct ihipStream_t *stream);

/*
 * NVFP4 W4A4: moe_quant_forward for an MQ_W_NVFP4_G16 layer with its
 * activations quantized to NVFP4 as well, the format the
 * "clef-flash-NVFP4-Hybrid" card (section "Quantization details") gives its
 * W4A4 layers and the "clef-omni-fp8" card (table "Which Clef-Omni quant
 * should I use?") lists for the W4A4 build: E2M1 values, one E4M3 scale per
 * 16 consecutive values, one FP32 global scale per tensor, the activation
 * global scales calibrated.  act_gscale13 is the global scale g of the
 * gate/up input (the hidden rows), act_gscale2 that of the down input (the
 * SwiGLU intermediate), one per layer, shared by its experts.  For each
 * token (gate/up) or grouped row (down) and each 16 consecutive features
 * with maximum magnitude m, in FP32:
 *   s = RNE-to-E4M3(min((m * g) / 6, 448)),
 *   code = RNE-to-E2M1((x * g) / s) saturated to +-6 (0 where s = 0),
 * and the projection sees e2m1(code) * s / g; the intermediate is quantized
 * from its FP32 value.  The GEMMs multiply the exact products e2m1 * s on the
 * FP16 matrix units and apply 1 / g to their FP32 sums.  Same arguments,
 * workspace size and routing as moe_quant_forward (the kernels are the
 * many-rows-per-expert ones at every batch size).  The probe's h buffer
 * receives the down input as kept here: FP16 values e2m1(code) * s [T*k, I]
 * in grouped row order.  Errors: as moe_quant_forward, plus MQ_E_FORMAT for
 * another weight format and MQ_E_SHAPE for a global scale that is not
 * finite and positive.
 */
mq_status moe_quant_forward_w4a4(const mq_layer *L, const void *router_logits, int32_t logits_dtype,
                                 const uint16_t *hidden_bf16, const uint16_t *residual_bf16,
                                 int64_t num_tokens, uint16_t *out_bf16, void *workspace,
                                 size_t workspace_bytes, float act_gscale13, float act_gscale2,
                                 const mq_probe *probe, struct ihipStream_t *stream);

/*
 * Test entry: the NVFP4 activation quantizer of the W4A4 path on FP32 rows
 * x [rows, K] (device) with global scale gscale, writing the E2M1 codes
 * packed two per byte, even k in the low nibble, uint8 [rows, K/2], and the
 * E4M3FN block scales uint8 [rows, K/16] (device, caller-owned): the NVFP4
 * layout of MQ_W_NVFP4_G16 weights.  K a positive multiple of 16 (at most
 * 65536); gscale finite and positive.
 * Errors: MQ_E_SHAPE, MQ_E_NULL, MQ_E_ALIGN (x 16-byte, codes 4-byte), MQ_E_HIP.
 */
mq_status moe_quant_quantize_act_nvfp4(const float *x, int64_t rows, int32_t K, float gscale,
                                       uint8_t *codes, uint8_t *scales, struct ihipStream_t *stream);

/*
 * moe_quant_forward with the router in the library: the logits of the BF16
 * gate that stays unquantized on every card ("clef-omni-int4" card, section
 * "Recipe": ignore_layers=mlp.gate; "clef-omni-NVFP4" card, section "How it
 * was made": the router is copied unchanged), read as a linear layer without
 * bias, logits[t, e] = sum_h hidden[t, h] * router[e, h], are computed and
 * selected in one kernel from 4096 tokens up: each block of 16 or 32 tokens
 * keeps its FP32 logits on chip and runs the top-k there (same order, ties
 * and weights as moe_quant_forward).  Smaller batches run the router logits
 * kernel into the workspace and then the logits-driven routing kernel, which
 * is faster there.  The rest of the path is moe_quant_forward's.
 *   hidden_bf16   [T, H] BF16 bits, 16-byte aligned
 *   router_bf16   [E, H] BF16 bits (the gate's weight), 16-byte aligned
 *   residual_bf16, num_tokens, out_bf16, workspace, workspace_bytes, probe,
 *   stream        as for moe_quant_forward (same workspace size)
 *   logits_out    NULL, or float [T, E] (4-byte aligned): receives the FP32
 *                 logits the top-k decided on (for tests)
 * Products are exact in FP32 and summed in FP32 by the matrix units in a fixed
 * order, so repeated calls are bit-identical.  E at most 256.
 * Errors: as moe_quant_forward (MQ_E_NULL when router_bf16 is NULL,
 * MQ_E_SHAPE when E > 256).
 */
mq_status moe_quant_forward_with_router(const mq_layer *L, const uint16_t *hidden_bf16,
                                        const uint16_t *router_bf16,
                                        const uint16_t *residual_bf16, int64_t num_tokens,
                                        uint16_t *out_bf16, void *workspace,
                                        size_t workspace_bytes, float *logits_out,
                                        const mq_probe *probe, struct ihipStream_t *stream);

/*
 * Synchronize `stream` and report whether the last forward that used
 * `workspace` saturated one of its FP16 intermediates (the SwiGLU output h or a
 * routing-weighted per-slot expert output; values beyond +-65504 are clamped):
 * MQ_OK if not, MQ_E_OVERFLOW if it did.  workspace as passed to forward.
 * Batches of one or two tokens keep the per-slot outputs in FP32 (the down
 * projection adds them into the output itself), so there only h can saturate.
 */
mq_status moe_quant_check(const mq_layer *L, const void *workspace, struct ihipStream_t *stream);

/*
 * Test entry: enqueue the dequantization of one expert matrix through the
 * device unpack paths the GEMMs use, writing float32 [N, K] to `out`
 * (which: 0 = W13 [2I, H], 1 = W2 [H, I]).  Each value is the format's
 * definition evaluated in FP32 with at most one rounding: INT4 (c - 8) * s is
 * exact; FP8 e4m3 * scale is one FP32 multiply; NVFP4 (e2m1 * e4m3) is exact
 * and is then divided by gscale (one IEEE FP32 division).
 * Errors: MQ_E_NULL, MQ_E_SHAPE (which or expert out of range), MQ_E_HIP.
 */
mq_status moe_quant_dequantize(const mq_layer *L, int32_t which, int32_t expert, float *out,
                               struct ihipStream_t *stream);

/*
 * Router logits of the gate that stays in BF16 ("clef-omni-fp8" card, section
 * "What was quantized"; "clef-omni-NVFP4" card, section "How it was made"),
 * read as a linear layer without bias:
 *   logits_f32[t, e] = sum_h hidden_bf16[t, h] * router_bf16[e, h]
 *   hidden_bf16  [T, H] BF16 bits, row-major, 16-byte aligned
 *   router_bf16  [E, H] BF16 bits, row-major (the gate's weight), 16-byte aligned
 *   logits_f32   [T, E] float32, row-major, 16-byte aligned; written here, and
 *                ready for moe_quant_forward with logits_dtype MQ_F32
 * All three live in device memory owned by the caller; nothing is kept after
 * the call.  Products are exact in FP32 and summed in FP32 by the matrix
 * units (an order of their own).  hidden a positive multiple of 64 (at most
 * 65536), 1 <= num_experts <= 65536, 0 <= num_tokens <= 2^22; num_tokens == 0
 * returns MQ_OK without enqueuing anything.  No layer handle is needed.
 * Errors: MQ_E_SHAPE, MQ_E_NULL, MQ_E_ALIGN, MQ_E_HIP (launch failed).
 */
mq_status moe_quant_router_logits(const uint16_t *hidden_bf16, const uint16_t *router_bf16,
                                  int64_t num_tokens, int32_t hidden, int32_t num_experts,
                                  float *logits_f32, struct ihipStream_t *stream);

/*
 * Allocation-free variant of moe_quant_forward, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  It runs the same kernels; their scratch
 * (routing tables, the FP16 intermediate and the per-slot partials) lives in
 * a static device array inside the library, MOE_QUANT_NOALLOC_SCRATCH_BYTES
 * per GPU, held by each GPU the library runs on until the process ends.  No
 * hipMalloc, hipFree or allocating library routine is called.
 *   router_logits, hidden_bf16, residual_bf16, num_tokens, out_bf16, stream:
 *                  as for moe_quant_forward
 *   overflow_flag  NULL, or a caller-owned device uint32 (4-byte aligned):
 *                  set to 0 at the start of the call and to 1 if an FP16
 *                  intermediate saturated (read it after the stream syncs)
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind: calls that overlap on one GPU (different streams, or host threads
 * without ordering between them) race on it and must not be issued.
 * Errors: as moe_quant_forward, plus MQ_E_WORKSPACE when the batch needs more
 * scratch than the array holds (moe_quant_workspace_size(L, T) above
 * MOE_QUANT_NOALLOC_SCRATCH_BYTES; about 1350 tokens at hidden 2048,
 * intermediate 768, 128 experts, top-8), checked before anything is enqueued.
 */
#define MOE_QUANT_NOALLOC_SCRATCH_BYTES (64u << 20)
mq_status moe_quant_forward_noalloc(const mq_layer *L, const void *router_logits,
                                    int32_t logits_dtype, const uint16_t *hidden_bf16,
                                    const uint16_t *residual_bf16, int64_t num_tokens,
                                    uint16_t *out_bf16, uint32_t *overflow_flag,
                                    struct ihipStream_t *stream);

/*
 * Checkpoint import: one expert's gate_proj, up_proj and down_proj, each in
 * the tensor layout of the checkpoint format the model cards name for the
 * layer's weight format, written into the packed layouts above (gate and up
 * fused into W13, gate rows first).  Source and destination tensors are
 * device memory owned by the caller.  Per projection (N = out_features, K =
 * in_features: gate and up N = I, K = H; down N = H, K = I):
 *   MQ_W_FP8_B128   FineGrainedFP8 ("clef-omni-fp8" card, section "Recipe"):
 *                   weight = E4M3 [N, K], scale = weight_scale_inv float
 *                   [N/128, K/128]; copied into place (the same bytes).
 *   MQ_W_INT4_G128  auto_gptq packing ("clef-omni-int4" card, section "What
 *                   was quantized"): weight = qweight int32 [K/8, N] (word
 *                   [i, n] holds k = 8 i + j at bits 4 j), qzeros = int32
 *                   [K/128, N/8] (word [g, c] holds column 8 c + j at bits
 *                   4 j), scale = scales fp16 [K/128, N].  The stored zero
 *                   point plus gptq_zero_offset (1 in the auto_gptq
 *                   convention) must be 8 in every group (symmetric INT4);
 *                   weights and scales are transposed into place.
 *   MQ_W_NVFP4_G16  compressed-tensors NVFP4 ("clef-omni-NVFP4" card, section
 *                   "How it was made"): weight = weight_packed uint8 [N, K/2],
 *                   scale = weight_scale E4M3 [N, K/16], global_scale =
 *                   weight_global_scale (host float); copied into place, and
 *                   the global scales into w13_gscale[expert] (gate and up
 *                   must be equal: the card's quantizer fuses them) and
 *                   w2_gscale[expert].
 * dst: a descriptor of the destination layer (the same checks as
 * moe_quant_init); its weight and scale buffers are written.
 * bad_zero_points: INT4 only, NULL or a device uint32 that is set to 1 when
 * a group's zero point is not 8 (read it after the stream syncs; the weights
 * of such a group cannot be represented and the import must be discarded).
 * Asynchronous on `stream`.  Errors: the moe_quant_init errors for dst,
 * MQ_E_NULL (a source tensor NULL), MQ_E_SHAPE (expert out of range),
 * MQ_E_ALIGN (a source tensor not 16-byte aligned), MQ_E_FORMAT (NVFP4 gate
 * and up global scales differ), MQ_E_HIP.
 */
typedef struct {
  const void *weight;  /* see above, per format                            */
  const void *scale;
  const void *qzeros;  /* INT4 only; NULL for the other formats            */
  float global_scale;  /* NVFP4 only                                        */
} mq_src_proj;

mq_status moe_quant_import_expert(const mq_layer_desc *dst, int32_t expert, const mq_src_proj *gate,
                                  const mq_src_proj *up, const mq_src_proj *down,
                                  int32_t gptq_zero_offset, uint32_t *bad_zero_points,
                                  struct ihipStream_t *stream);

void moe_quant_destroy(mq_layer *L);

/* Static strings; never NULL. */
const char *moe_quant_status_string(mq_status s);
const char *moe_quant_last_error(void);
uint32_t moe_quant_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_QUANT_H */

// Host side of the C ABI declared in include/moe_quant.h: argument checks,
// workspace carve-up and the stream-ordered launch sequence of one forward.
#include "../../include/moe_quant.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <new>

#include "internal.h"

struct mq_layer {
  mq_layer_desc d;
};

namespace {

thread_local char g_err[512] = "";

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

namespace mq {

mq_status fail(mq_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

void clear_error() { g_err[0] = 0; }

Workspace workspace_layout(int64_t T, int E, int H, int I, int k) {
  Workspace w{};
  const size_t R = (size_t)T * k;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = up256(o + bytes);
    return at;
  };
  w.flags = take(16);  // first, so its offset (0) does not depend on T
  w.topk_ids = take(R * 4);
  w.topk_w = take(R * 4);
  w.offsets = take((size_t)(E + 1) * 4);
  w.active = take((size_t)(E + 1) * 16);
  w.rowinfo = take(R * 16);
  w.mtile = take((size_t)(E + 1) * 4);
  w.rcpre = take((size_t)(E + 1) * 4);
  w.sorted_slots = take(R * 4);
  w.inv_pos = take(R * 4);
  w.chunks = take((size_t)mq::kMaxChunks * E * 4);
  w.x16 = take((size_t)T * H * 2);
  w.rowscale = take((size_t)T * 4);
  w.logits = take((size_t)T * E * 4);
  w.h = take(R * (size_t)I * 2);
  w.partial = take(R * (size_t)H * 2);
  w.total = o;
  return w;
}

size_t workspace_bytes(const mq_layer *L, int64_t T) {
  const mq_layer_desc &d = L->d;
  return workspace_layout(T, d.num_experts, d.hidden, d.intermediate, d.top_k).total;
}

}  // namespace mq

using mq::fail;
using mq::kMaxTokens;

extern "C" {

uint32_t moe_quant_abi_version(void) { return MOE_QUANT_ABI_VERSION; }

const char *moe_quant_last_error(void) { return g_err; }

const char *moe_quant_status_string(mq_status s) {
  switch (s) {
    case MQ_OK: return "MQ_OK: success";
    case MQ_E_NULL: return "MQ_E_NULL: a required pointer is NULL";
    case MQ_E_SHAPE: return "MQ_E_SHAPE: dimension out of range or not a block multiple";
    case MQ_E_ALIGN: return "MQ_E_ALIGN: pointer not aligned as required";
    case MQ_E_FORMAT: return "MQ_E_FORMAT: unknown weight format";
    case MQ_E_DTYPE: return "MQ_E_DTYPE: unknown logits dtype";
    case MQ_E_WORKSPACE: return "MQ_E_WORKSPACE: workspace missing or too small";
    case MQ_E_ABI: return "MQ_E_ABI: descriptor ABI version mismatch";
    case MQ_E_HIP: return "MQ_E_HIP: HIP runtime or launch failure";
    case MQ_E_OVERFLOW: return "MQ_E_OVERFLOW: an FP16 intermediate saturated";
  }
  return "unknown mq_status";
}

static mq_status check_desc(const mq_layer_desc *d, const char *who) {
  if (d->abi_version != MOE_QUANT_ABI_VERSION)
    return fail(MQ_E_ABI, "%s: descriptor abi_version %u, library %u", who, d->abi_version,
                MOE_QUANT_ABI_VERSION);
  if (d->format != MQ_W_INT4_G128 && d->format != MQ_W_FP8_B128 && d->format != MQ_W_NVFP4_G16)
    return fail(MQ_E_FORMAT, "%s: unknown weight format %d", who, d->format);
  const int E = d->num_experts, H = d->hidden, I = d->intermediate, k = d->top_k;
  if (E < 1 || E > mq::kMaxExperts)
    return fail(MQ_E_SHAPE, "%s: num_experts %d outside [1, %d]", who, E, mq::kMaxExperts);
  if (k < 1 || k > E || k > 64) return fail(MQ_E_SHAPE, "%s: top_k %d outside [1, min(E, 64)]", who, k);
  if (H < 128 || I < 128 || H % 128 || I % 128)
    return fail(MQ_E_SHAPE, "%s: hidden %d and intermediate %d must be positive multiples of 128 "
                "(block sizes of INT4 g128 / FP8 128x128; this version's tiles for NVFP4)", who,
                H, I);
  if (!mq::decode_fits(H) || !mq::decode_fits(I))
    return fail(MQ_E_SHAPE, "%s: hidden %d / intermediate %d above %d: the decode GEMM stages 16 whole "
                "rows of the input dimension in LDS (160 KiB per workgroup)", who,
                H, I, mq::kMaxGemmK);
  if (!d->w13 || !d->w13_scale || !d->w2 || !d->w2_scale)
    return fail(MQ_E_NULL, "%s: weight and scale pointers must be non-NULL", who);
  if (d->format == MQ_W_NVFP4_G16 && (!d->w13_gscale || !d->w2_gscale))
    return fail(MQ_E_NULL, "%s: NVFP4 needs w13_gscale and w2_gscale", who);
  if (d->format != MQ_W_NVFP4_G16 && (d->w13_gscale || d->w2_gscale))
    return fail(MQ_E_NULL, "%s: gscale pointers must be NULL for INT4 and FP8", who);
  const void *al16[4] = {d->w13, d->w13_scale, d->w2, d->w2_scale};
  for (const void *p : al16)
    if (!aligned(p, 16)) return fail(MQ_E_ALIGN, "%s: weight/scale pointer %p not 16-byte aligned", who, p);
  if ((d->w13_gscale && !aligned(d->w13_gscale, 4)) || (d->w2_gscale && !aligned(d->w2_gscale, 4)))
    return fail(MQ_E_ALIGN, "%s: gscale pointers must be 4-byte aligned", who);
  return MQ_OK;
}

mq_status moe_quant_init(const mq_layer_desc *d, mq_layer **out) {
  if (!d || !out) return fail(MQ_E_NULL, "init: desc and out must be non-NULL");
  *out = nullptr;
  const mq_status st = check_desc(d, "init");
  if (st != MQ_OK) return st;
  mq_layer *L = new (std::nothrow) mq_layer;
  if (!L) return fail(MQ_E_NULL, "init: host allocation failed");
  L->d = *d;
  *out = L;
  g_err[0] = 0;
  return MQ_OK;
}

void moe_quant_destroy(mq_layer *L) { delete L; }

mq_status moe_quant_workspace_size(const mq_layer *L, int64_t num_tokens, size_t *bytes) {
  if (!L || !bytes) return fail(MQ_E_NULL, "workspace_size: NULL argument");
  if (num_tokens < 0 || num_tokens > kMaxTokens)
    return fail(MQ_E_SHAPE, "workspace_size: num_tokens %lld outside [0, %lld]",
                (long long)num_tokens, (long long)kMaxTokens);
  *bytes = mq::workspace_bytes(L, num_tokens);
  return MQ_OK;
}

static mq::LayerDims dims_of(const mq_layer *L) {
  const mq_layer_desc &d = L->d;
  mq::LayerDims D;
  D.E = d.num_experts; D.H = d.hidden; D.I = d.intermediate; D.k = d.top_k; D.fmt = d.format;
  D.w13 = (const uint8_t *)d.w13; D.w2 = (const uint8_t *)d.w2;
  D.s13 = d.w13_scale; D.s2 = d.w2_scale;
  D.g13 = d.w13_gscale; D.g2 = d.w2_gscale;
  return D;
}

mq_status moe_quant_forward(const mq_layer *L, const void *router_logits, int32_t logits_dtype,
                            const uint16_t *hidden_bf16, const uint16_t *residual_bf16,
                            int64_t num_tokens, uint16_t *out_bf16, void *workspace,
                            size_t workspace_bytes, const mq_probe *probe,
                            struct ihipStream_t *stream) {
  return mq::forward_impl(L, router_logits, logits_dtype, hidden_bf16, residual_bf16, num_tokens,
                          out_bf16, workspace, workspace_bytes, probe, nullptr, (hipStream_t)stream);
}

}  // extern "C"

mq_status mq::forward_impl(const mq_layer *L, const void *router_logits, int32_t logits_dtype,
                           const uint16_t *hidden_bf16, const uint16_t *residual_bf16,
                           int64_t num_tokens, uint16_t *out_bf16, void *workspace,
                           size_t workspace_bytes, const mq_probe *probe, uint32_t *flags,
                           hipStream_t stream, const uint16_t *gate_w, float *logits_out,
                           int w8a8, float act_g13, float act_g2) {
  if (!L) return fail(MQ_E_NULL, "forward: NULL layer handle");
  if (num_tokens < 0 || num_tokens > kMaxTokens)
    return fail(MQ_E_SHAPE, "forward: num_tokens %lld outside [0, %lld]", (long long)num_tokens,
                (long long)kMaxTokens);
  if (!gate_w && logits_dtype != MQ_F32 && logits_dtype != MQ_BF16)
    return fail(MQ_E_DTYPE, "forward: unknown logits dtype %d", logits_dtype);
  if (gate_w && L->d.num_experts > mq::kMaxGateExperts)
    return fail(MQ_E_SHAPE, "forward_with_router: %d experts, the fused router holds at most %d",
                L->d.num_experts, mq::kMaxGateExperts);
  if (num_tokens == 0) {
    g_err[0] = 0;
    return MQ_OK;
  }
  if ((!gate_w && !router_logits) || !hidden_bf16 || !out_bf16)
    return fail(MQ_E_NULL, "forward: logits (or the router weight), hidden and out must be non-NULL");
  if ((!gate_w && !aligned(router_logits, 16)) || (gate_w && !aligned(gate_w, 16)) ||
      !aligned(hidden_bf16, 16) || !aligned(out_bf16, 16) ||
      (residual_bf16 && !aligned(residual_bf16, 16)) || (logits_out && !aligned(logits_out, 4)))
    return fail(MQ_E_ALIGN, "forward: logits/router/hidden/residual/out must be 16-byte aligned");
  const mq::LayerDims D = dims_of(L);
  const mq::Workspace W = mq::workspace_layout(num_tokens, D.E, D.H, D.I, D.k);
  if (!workspace) return fail(MQ_E_WORKSPACE, "forward: workspace is NULL");
  if (!aligned(workspace, 256)) return fail(MQ_E_ALIGN, "forward: workspace not 256-byte aligned");
  if (workspace_bytes < W.total)
    return fail(MQ_E_WORKSPACE, "forward: workspace %zu bytes, need %zu", workspace_bytes, W.total);
  if (probe) {
    const void *pp[6] = {probe->topk_ids, probe->topk_w, probe->expert_offsets,
                         probe->sorted_token_ids, probe->inv_pos, probe->h};
    for (const void *p : pp)
      if (p && !aligned(p, 4)) return fail(MQ_E_ALIGN, "forward: probe arrays must be 4-byte aligned");
  }

  mq::FwdPtrs P{};
  P.logits = router_logits;
  P.logits_bf16 = logits_dtype == MQ_BF16;
  P.gate_w = gate_w;
  P.p_logits = logits_out;
  P.w8a8 = w8a8;
  P.act_g13 = act_g13;
  P.act_g2 = act_g2;
  P.hidden = hidden_bf16;
  P.residual = residual_bf16;
  P.out = out_bf16;
  P.ws = (char *)workspace;
  P.flags = flags ? flags : (uint32_t *)(P.ws + W.flags);
  P.T = (int)num_tokens;
  if (probe) {
    P.p_ids = probe->topk_ids;
    P.p_w = probe->topk_w;
    P.p_offsets = probe->expert_offsets;
    P.p_sorted_tok = probe->sorted_token_ids;
    P.p_inv = probe->inv_pos;
    P.p_h = probe->h;
  }
  hipStream_t s = stream;
  // the W4A4 variant runs the many-rows-per-expert kernels at every batch size
  const bool decode = act_g13 == 0.f && mq::use_decode_path(num_tokens, D.E, D.k, D.H, D.I);
  auto ev = [&](int stage, int after) {
    if (probe && probe->events[2 * stage + after])
      (void)hipEventRecord((hipEvent_t)probe->events[2 * stage + after], s);
  };
  hipError_t e;
  ev(MQ_STAGE_ROUTE, 0);
  if ((e = mq::launch_route(D, P, W, decode, s)) != hipSuccess)
    return fail(MQ_E_HIP, "forward: route launch: %s", hipGetErrorString(e));
  ev(MQ_STAGE_ROUTE, 1);
  ev(MQ_STAGE_PERMUTE, 0);
  if ((e = mq::launch_permute(D, P, W, decode, s)) != hipSuccess)
    return fail(MQ_E_HIP, "forward: permute launch: %s", hipGetErrorString(e));
  ev(MQ_STAGE_PERMUTE, 1);
  // the GEMM stages' events are taken by the runtime at the start and the end
  // of the kernel itself
  auto kev = [&](int stage) {
    mq::GemmLaunch g{s, nullptr, nullptr};
    if (probe) {
      g.start = (hipEvent_t)probe->events[2 * stage];
      g.stop = (hipEvent_t)probe->events[2 * stage + 1];
    }
    return g;
  };
  e = w8a8 ? mq::launch_w8a8_gate_up(D, P, W, kev(MQ_STAGE_GATE_UP))
           : mq::launch_gate_up(D, P, W, decode, kev(MQ_STAGE_GATE_UP));
  if (e != hipSuccess) return fail(MQ_E_HIP, "forward: gate_up launch: %s", hipGetErrorString(e));
  if (P.p_h) {
    e = hipMemcpyAsync(P.p_h, P.ws + W.h, (size_t)num_tokens * D.k * D.I * 2,
                       hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return fail(MQ_E_HIP, "forward: probe copy: %s", hipGetErrorString(e));
  }
  e = w8a8 ? mq::launch_w8a8_down(D, P, W, kev(MQ_STAGE_DOWN))
           : mq::launch_down(D, P, W, decode, kev(MQ_STAGE_DOWN));
  if (e != hipSuccess) return fail(MQ_E_HIP, "forward: down launch: %s", hipGetErrorString(e));
  ev(MQ_STAGE_COMBINE, 0);
  if (!mq::down_writes_output(D, P, decode) && (e = mq::launch_combine(D, P, W, s)) != hipSuccess)
    return fail(MQ_E_HIP, "forward: combine launch: %s", hipGetErrorString(e));
  ev(MQ_STAGE_COMBINE, 1);
  g_err[0] = 0;
  return MQ_OK;
}

extern "C" {

mq_status moe_quant_forward_w8a8(const mq_layer *L, const void *router_logits, int32_t logits_dtype,
                                 const uint16_t *hidden_bf16, const uint16_t *residual_bf16,
                                 int64_t num_tokens, uint16_t *out_bf16, void *workspace,
                                 size_t workspace_bytes, const mq_probe *probe,
                                 struct ihipStream_t *stream) {
  if (!L) return fail(MQ_E_NULL, "forward_w8a8: NULL layer handle");
  if (L->d.format != MQ_W_FP8_B128)
    return fail(MQ_E_FORMAT, "forward_w8a8: W8A8 applies to MQ_W_FP8_B128 layers (format %d)", L->d.format);
  return mq::forward_impl(L, router_logits, logits_dtype, hidden_bf16, residual_bf16, num_tokens,
                          out_bf16, workspace, workspace_bytes, probe, nullptr, (hipStream_t)stream,
                          nullptr, nullptr, 1);
}

static bool valid_gscale(float g) { return std::isfinite(g) && g > 0.f; }

mq_status moe_quant_forward_w4a4(const mq_layer *L, const void *router_logits, int32_t logits_dtype,
                                 const uint16_t *hidden_bf16, const uint16_t *residual_bf16,
                                 int64_t num_tokens, uint16_t *out_bf16, void *workspace,
                                 size_t workspace_bytes, float act_gscale13, float act_gscale2,
                                 const mq_probe *probe, struct ihipStream_t *stream) {
  if (!L) return fail(MQ_E_NULL, "forward_w4a4: NULL layer handle");
  if (L->d.format != MQ_W_NVFP4_G16)
    return fail(MQ_E_FORMAT, "forward_w4a4: W4A4 applies to MQ_W_NVFP4_G16 layers (format %d)", L->d.format);
  if (!valid_gscale(act_gscale13) || !valid_gscale(act_gscale2))
    return fail(MQ_E_SHAPE, "forward_w4a4: activation global scales %g and %g must be finite and positive",
                (double)act_gscale13, (double)act_gscale2);
  return mq::forward_impl(L, router_logits, logits_dtype, hidden_bf16, residual_bf16, num_tokens,
                          out_bf16, workspace, workspace_bytes, probe, nullptr, (hipStream_t)stream,
                          nullptr, nullptr, 0, act_gscale13, act_gscale2);
}

mq_status moe_quant_quantize_act_nvfp4(const float *x, int64_t rows, int32_t K, float gscale,
                                       uint8_t *codes, uint8_t *scales, struct ihipStream_t *stream) {
  if (rows < 0 || rows > ((int64_t)1 << 30) || K <= 0 || K % 16 || K > 65536)
    return fail(MQ_E_SHAPE, "quantize_act_nvfp4: rows %lld and K %d (K a positive multiple of 16, at most 65536)",
                (long long)rows, K);
  if (!valid_gscale(gscale))
    return fail(MQ_E_SHAPE, "quantize_act_nvfp4: global scale %g must be finite and positive", (double)gscale);
  if (rows == 0) {
    g_err[0] = 0;
    return MQ_OK;
  }
  if (!x || !codes || !scales) return fail(MQ_E_NULL, "quantize_act_nvfp4: NULL argument");
  if (!aligned(x, 16) || !aligned(codes, 4))
    return fail(MQ_E_ALIGN, "quantize_act_nvfp4: x 16-byte, codes 4-byte aligned");
  const hipError_t e = mq::launch_quant_act_nvfp4(x, rows, K, gscale, codes, scales, (hipStream_t)stream);
  if (e != hipSuccess) return fail(MQ_E_HIP, "quantize_act_nvfp4: %s", hipGetErrorString(e));
  g_err[0] = 0;
  return MQ_OK;
}

mq_status moe_quant_quantize_act(const float *x, int64_t rows, int32_t K, uint8_t *codes, float *scales,
                                 struct ihipStream_t *stream) {
  if (rows < 0 || rows > ((int64_t)1 << 30) || K <= 0 || K % 128 || K > 65536)
    return fail(MQ_E_SHAPE, "quantize_act: rows %lld and K %d (K a positive multiple of 128, at most 65536)",
                (long long)rows, K);
  if (rows == 0) {
    g_err[0] = 0;
    return MQ_OK;
  }
  if (!x || !codes || !scales) return fail(MQ_E_NULL, "quantize_act: NULL argument");
  if (!aligned(x, 16) || !aligned(codes, 8) || !aligned(scales, 4))
    return fail(MQ_E_ALIGN, "quantize_act: x 16-byte, codes 8-byte, scales 4-byte aligned");
  const hipError_t e = mq::launch_quant_act(x, rows, K, codes, scales, (hipStream_t)stream);
  if (e != hipSuccess) return fail(MQ_E_HIP, "quantize_act: %s", hipGetErrorString(e));
  g_err[0] = 0;
  return MQ_OK;
}

mq_status moe_quant_forward_with_router(const mq_layer *L, const uint16_t *hidden_bf16,
                                        const uint16_t *router_bf16,
                                        const uint16_t *residual_bf16, int64_t num_tokens,
                                        uint16_t *out_bf16, void *workspace,
                                        size_t workspace_bytes, float *logits_out,
                                        const mq_probe *probe, struct ihipStream_t *stream) {
  if (!router_bf16) return fail(MQ_E_NULL, "forward_with_router: router weight is NULL");
  return mq::forward_impl(L, nullptr, MQ_F32, hidden_bf16, residual_bf16, num_tokens, out_bf16,
                          workspace, workspace_bytes, probe, nullptr, (hipStream_t)stream,
                          router_bf16, logits_out);
}

mq_status moe_quant_import_expert(const mq_layer_desc *dst, int32_t expert, const mq_src_proj *gate,
                                  const mq_src_proj *up, const mq_src_proj *down,
                                  int32_t gptq_zero_offset, uint32_t *bad_zero_points,
                                  struct ihipStream_t *stream) {
  if (!dst || !gate || !up || !down) return fail(MQ_E_NULL, "import: NULL argument");
  const mq_status st = check_desc(dst, "import");
  if (st != MQ_OK) return st;
  if (expert < 0 || expert >= dst->num_experts)
    return fail(MQ_E_SHAPE, "import: expert %d outside [0, %d)", expert, dst->num_experts);
  const bool int4 = dst->format == MQ_W_INT4_G128;
  for (const mq_src_proj *p : {gate, up, down}) {
    if (!p->weight || !p->scale || (int4 && !p->qzeros))
      return fail(MQ_E_NULL, "import: a source tensor is NULL");
    const size_t scale_align = dst->format == MQ_W_FP8_B128 ? 4 : int4 ? 2 : 1;
    if (!aligned(p->weight, 16) || !aligned(p->scale, scale_align) || (int4 && !aligned(p->qzeros, 4)))
      return fail(MQ_E_ALIGN, "import: source weights must be 16-byte aligned, scales and zeros aligned to their type");
  }
  if (bad_zero_points && !aligned(bad_zero_points, 4))
    return fail(MQ_E_ALIGN, "import: bad_zero_points must be 4-byte aligned");
  if (dst->format == MQ_W_NVFP4_G16 && gate->global_scale != up->global_scale)
    return fail(MQ_E_FORMAT, "import: NVFP4 gate and up global scales differ (%g, %g); W13 holds one",
                (double)gate->global_scale, (double)up->global_scale);
  mq_layer tmp;
  tmp.d = *dst;
  const hipError_t e = mq::launch_import_expert(dims_of(&tmp), expert, *gate, *up, *down,
                                                gptq_zero_offset, bad_zero_points, (hipStream_t)stream);
  if (e != hipSuccess) return fail(MQ_E_HIP, "import: %s", hipGetErrorString(e));
  g_err[0] = 0;
  return MQ_OK;
}

mq_status moe_quant_check(const mq_layer *L, const void *workspace, struct ihipStream_t *stream) {
  if (!L || !workspace) return fail(MQ_E_NULL, "check: NULL argument");
  // the flags word is the first field of every workspace layout (offset 0)
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return fail(MQ_E_HIP, "check: %s", hipGetErrorString(e));
  uint32_t flag = 0;
  e = hipMemcpy(&flag, workspace, sizeof(flag), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(MQ_E_HIP, "check: %s", hipGetErrorString(e));
  if (flag) return fail(MQ_E_OVERFLOW, "check: an FP16 intermediate saturated");
  g_err[0] = 0;
  return MQ_OK;
}

mq_status moe_quant_dequantize(const mq_layer *L, int32_t which, int32_t expert, float *out,
                               struct ihipStream_t *stream) {
  if (!L || !out) return fail(MQ_E_NULL, "dequantize: NULL argument");
  if (which != 0 && which != 1) return fail(MQ_E_SHAPE, "dequantize: which must be 0 or 1");
  if (expert < 0 || expert >= L->d.num_experts)
    return fail(MQ_E_SHAPE, "dequantize: expert %d outside [0, %d)", expert, L->d.num_experts);
  if (!aligned(out, 16)) return fail(MQ_E_ALIGN, "dequantize: out must be 16-byte aligned");
  hipError_t e = mq::launch_dequantize(dims_of(L), which, expert, out, (hipStream_t)stream);
  if (e != hipSuccess) return fail(MQ_E_HIP, "dequantize: %s", hipGetErrorString(e));
  g_err[0] = 0;
  return MQ_OK;
}

mq_status moe_quant_router_logits(const uint16_t *hidden_bf16, const uint16_t *router_bf16,
                                  int64_t num_tokens, int32_t hidden, int32_t num_experts,
                                  float *logits_f32, struct ihipStream_t *stream) {
  if (num_tokens < 0 || num_tokens > kMaxTokens)
    return fail(MQ_E_SHAPE, "router_logits: num_tokens %lld outside [0, %lld]", (long long)num_tokens,
                (long long)kMaxTokens);
  if (hidden <= 0 || hidden % 64 != 0 || hidden > 65536)
    return fail(MQ_E_SHAPE, "router_logits: hidden %d must be a positive multiple of 64, at most 65536",
                hidden);
  if (num_experts <= 0 || num_experts > 65536)
    return fail(MQ_E_SHAPE, "router_logits: num_experts %d outside [1, 65536]", num_experts);
  if (num_tokens == 0) {
    g_err[0] = 0;
    return MQ_OK;
  }
  if (!hidden_bf16 || !router_bf16 || !logits_f32) return fail(MQ_E_NULL, "router_logits: NULL argument");
  if (!aligned(hidden_bf16, 16) || !aligned(router_bf16, 16) || !aligned(logits_f32, 16))
    return fail(MQ_E_ALIGN, "router_logits: pointers must be 16-byte aligned");
  hipError_t e = mq::launch_router_logits(hidden_bf16, router_bf16, logits_f32, num_tokens, hidden,
                                          num_experts, (hipStream_t)stream);
  if (e != hipSuccess) return fail(MQ_E_HIP, "router_logits: %s", hipGetErrorString(e));
  g_err[0] = 0;
  return MQ_OK;
}

}  // extern "C"

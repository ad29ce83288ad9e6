// Allocation-free forward: the same launch sequence as moe_quant_forward, with
// its scratch in a static device array of this library instead of a
// caller-owned workspace (for callers that cannot allocate device memory).
//
// The array's name is only a host-side stand-in in host code; its device
// address differs per GPU and comes from hipGetSymbolAddress, taken once per
// device on the first call made with that device current, and used for every
// kernel argument afterwards.
#include <map>
#include <mutex>

#include "internal.h"

namespace {

constexpr size_t kScratchBytes = MOE_QUANT_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::map<int, void *> g_scratch_ptr;  // device -> address of that device's copy of `scratch`

hipError_t scratch_address(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it != g_scratch_ptr.end()) {
    *out = it->second;
    return hipSuccess;
  }
  void *ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (ptr == nullptr || (uintptr_t)ptr % 256 != 0) return hipErrorInvalidSymbol;
  g_scratch_ptr[dev] = ptr;
  *out = ptr;
  return hipSuccess;
}

}  // namespace

extern "C" mq_status moe_quant_forward_noalloc(const mq_layer *L, const void *router_logits,
                                               int32_t logits_dtype, const uint16_t *hidden_bf16,
                                               const uint16_t *residual_bf16, int64_t num_tokens,
                                               uint16_t *out_bf16, uint32_t *overflow_flag,
                                               struct ihipStream_t *stream) {
  if (!L) return mq::fail(MQ_E_NULL, "forward_noalloc: NULL layer handle");
  if (num_tokens < 0 || num_tokens > mq::kMaxTokens)
    return mq::fail(MQ_E_SHAPE, "forward_noalloc: num_tokens %lld outside [0, %lld]",
                    (long long)num_tokens, (long long)mq::kMaxTokens);
  if (overflow_flag && (uintptr_t)overflow_flag % 4 != 0)
    return mq::fail(MQ_E_ALIGN, "forward_noalloc: overflow_flag must be 4-byte aligned");
  if (num_tokens == 0) {
    mq::clear_error();
    return MQ_OK;
  }
  const size_t need = mq::workspace_bytes(L, num_tokens);
  if (need > kScratchBytes)
    return mq::fail(MQ_E_WORKSPACE,
                    "forward_noalloc: %lld tokens need %zu bytes of scratch, above the library's "
                    "static %zu bytes; use moe_quant_forward with a workspace",
                    (long long)num_tokens, need, kScratchBytes);
  void *ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess)
    return mq::fail(MQ_E_HIP, "forward_noalloc: scratch address: %s", hipGetErrorString(e));
  return mq::forward_impl(L, router_logits, logits_dtype, hidden_bf16, residual_bf16, num_tokens,
                          out_bf16, ws, kScratchBytes, nullptr, overflow_flag, (hipStream_t)stream);
}

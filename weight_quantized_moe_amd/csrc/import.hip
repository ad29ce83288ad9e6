// Checkpoint importers: one expert's gate_proj, up_proj and down_proj, in the
// tensor layouts the model cards' checkpoints use, placed into this library's
// packed layouts (gate and up fused into W13, gate rows first).
//
//   FineGrainedFP8 ("clef-omni-fp8" card, sections "What was quantized" and
//   "Recipe"): weight E4M3 [N, K] + weight_scale_inv FP32 [N/128, K/128] per
//   projection.  Same bytes as MQ_W_FP8_B128 row for row (I is a multiple of
//   128, so the gate and up tiles stay whole): the rows are copied into place.
//
//   auto_gptq INT4 ("clef-omni-int4" card, section "What was quantized":
//   auto_round format, auto_gptq packing, group 128, symmetric): qweight int32
//   [K/8, N], qzeros int32 [K/128, N/8], scales FP16 [K/128, N].  A qweight
//   word holds the codes of 8 consecutive k of one column, low nibble first,
//   which is byte for byte the MQ_W_INT4_G128 packing of those 8 weights
//   (codes q with zero point 8 are the library's offset-binary c = q); so the
//   weights and scales are transposed to [N, K/8] words and [N, K/128], and
//   every group's zero point is checked to be 8.
//
//   compressed-tensors NVFP4 ("clef-omni-NVFP4" card, section "How it was
//   made"): weight_packed uint8 [N, K/2] (even k in the low nibble),
//   weight_scale E4M3 [N, K/16], weight_global_scale FP32.  Same bytes as
//   MQ_W_NVFP4_G16 row for row; gate and up must carry one global scale (the
//   card's quantizer concatenates them before quantizing).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"
#include "internal.h"

namespace mq {

// dst[c][r] = src[r][c] for 32-bit words; src is [rows][cols], dst has a row
// stride of ld words.  64x64 tiles through LDS (padded rows: conflict-free
// column reads), 256 threads.
__global__ __launch_bounds__(256) void transpose_u32_kernel(const uint32_t *__restrict__ src, int rows,
                                                            int cols, uint32_t *__restrict__ dst,
                                                            int ld) {
  __shared__ uint32_t tile[64][65];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    if (r < rows && c < cols) tile[i][tx] = src[(size_t)r * cols + c];
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (c < cols && r < rows) dst[(size_t)c * ld + r] = tile[tx][i];
  }
}

// dst[n][g] = src[g][n] for 16-bit scales: src [groups][n_cols], dst [n_cols][groups].
__global__ __launch_bounds__(256) void transpose_u16_kernel(const uint16_t *__restrict__ src, int groups,
                                                            int n_cols, uint16_t *__restrict__ dst) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)groups * n_cols) return;
  const int g = (int)(idx / n_cols), n = (int)(idx % n_cols);
  dst[(size_t)n * groups + g] = src[idx];
}

// Every stored zero point + offset must be 8 (a symmetric 4-bit group); sets
// bad[0] to 1 otherwise.  qzeros [groups][n_cols / 8] words, 8 columns each.
__global__ __launch_bounds__(256) void check_zero_points_kernel(const uint32_t *__restrict__ qzeros,
                                                                int64_t words, int offset,
                                                                uint32_t *__restrict__ bad) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= words) return;
  const uint32_t w = qzeros[idx];
  bool ok = true;
#pragma unroll
  for (int j = 0; j < 8; ++j) ok &= (int)((w >> (4 * j)) & 0xFu) + offset == 8;
  if (!ok) atomicOr(bad, 1u);
}

__global__ void set_gscale_kernel(float *__restrict__ g13, float *__restrict__ g2, int e, float v13,
                                  float v2) {
  g13[e] = v13;
  g2[e] = v2;
}

static unsigned blocks(int64_t n) { return (unsigned)((n + 255) / 256); }

// One GPTQ projection (K inputs, N outputs) into N packed rows starting at w
// and their N scale rows starting at scale.
static hipError_t import_gptq(const mq_src_proj &s, int N, int K, uint8_t *w, _Float16 *scale,
                              int offset, uint32_t *bad, hipStream_t st) {
  const int KW = K / 8, G = K / 128;
  dim3 grid((unsigned)((N + 63) / 64), (unsigned)((KW + 63) / 64));
  hipLaunchKernelGGL(transpose_u32_kernel, grid, dim3(256), 0, st, (const uint32_t *)s.weight, KW, N,
                     (uint32_t *)w, KW);
  hipLaunchKernelGGL(transpose_u16_kernel, dim3(blocks((int64_t)G * N)), dim3(256), 0, st,
                     (const uint16_t *)s.scale, G, N, (uint16_t *)scale);
  if (bad)
    hipLaunchKernelGGL(check_zero_points_kernel, dim3(blocks((int64_t)G * N / 8)), dim3(256), 0, st,
                       (const uint32_t *)s.qzeros, (int64_t)G * N / 8, offset, bad);
  return hipGetLastError();
}

hipError_t launch_import_expert(const LayerDims &L, int e, const mq_src_proj &gate,
                                const mq_src_proj &up, const mq_src_proj &down, int gptq_offset,
                                uint32_t *bad, hipStream_t st) {
  const int H = L.H, I = L.I;
  uint8_t *w13 = const_cast<uint8_t *>(L.w13), *w2 = const_cast<uint8_t *>(L.w2);
  hipError_t err = hipSuccess;
  auto copy = [&](void *dst, const void *src, size_t bytes) {
    if (err == hipSuccess) err = hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, st);
  };
  if (L.fmt == FMT_FP8) {
    const size_t sg13 = (size_t)(2 * I / 128) * (H / 128), sg2 = (size_t)(H / 128) * (I / 128);
    float *s13 = (float *)const_cast<void *>(L.s13) + e * sg13;
    float *s2 = (float *)const_cast<void *>(L.s2) + e * sg2;
    uint8_t *d13 = w13 + (size_t)e * 2 * I * H;
    copy(d13, gate.weight, (size_t)I * H);
    copy(d13 + (size_t)I * H, up.weight, (size_t)I * H);
    copy(s13, gate.scale, sg13 / 2 * 4);
    copy(s13 + sg13 / 2, up.scale, sg13 / 2 * 4);
    copy(w2 + (size_t)e * H * I, down.weight, (size_t)H * I);
    copy(s2, down.scale, sg2 * 4);
    return err;
  }
  if (L.fmt == FMT_NVFP4) {
    uint8_t *d13 = w13 + (size_t)e * 2 * I * (H / 2);
    uint8_t *s13 = (uint8_t *)const_cast<void *>(L.s13) + (size_t)e * 2 * I * (H / 16);
    copy(d13, gate.weight, (size_t)I * (H / 2));
    copy(d13 + (size_t)I * (H / 2), up.weight, (size_t)I * (H / 2));
    copy(s13, gate.scale, (size_t)I * (H / 16));
    copy(s13 + (size_t)I * (H / 16), up.scale, (size_t)I * (H / 16));
    copy(w2 + (size_t)e * H * (I / 2), down.weight, (size_t)H * (I / 2));
    copy((uint8_t *)const_cast<void *>(L.s2) + (size_t)e * H * (I / 16), down.scale, (size_t)H * (I / 16));
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(set_gscale_kernel, dim3(1), dim3(1), 0, st, const_cast<float *>(L.g13),
                       const_cast<float *>(L.g2), e, gate.global_scale, down.global_scale);
    return hipGetLastError();
  }
  // INT4 from auto_gptq packing
  uint8_t *d13 = w13 + (size_t)e * 2 * I * (H / 2);
  _Float16 *s13 = (_Float16 *)const_cast<void *>(L.s13) + (size_t)e * 2 * I * (H / 128);
  if ((err = import_gptq(gate, I, H, d13, s13, gptq_offset, bad, st)) != hipSuccess) return err;
  if ((err = import_gptq(up, I, H, d13 + (size_t)I * (H / 2), s13 + (size_t)I * (H / 128), gptq_offset,
                         bad, st)) != hipSuccess)
    return err;
  return import_gptq(down, H, I, w2 + (size_t)e * H * (I / 2),
                     (_Float16 *)const_cast<void *>(L.s2) + (size_t)e * H * (I / 128), gptq_offset, bad, st);
}

}  // namespace mq

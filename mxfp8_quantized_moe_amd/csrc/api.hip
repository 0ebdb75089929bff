// C ABI entry points (include/fp8moe.h): validate on the host, then enqueue.
#include <hip/hip_runtime.h>

#include <cstring>

#include "../../include/fp8moe.h"
#include "device_common.hpp"
#include "kernels.hpp"
#include "validate.hpp"

using namespace fp8moe;

namespace fp8moe {

__global__ __launch_bounds__(256) void encode_f32_kernel(const float* __restrict__ y, int64_t n, int codec,
                                                         uint8_t* __restrict__ q) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    q[i] = (uint8_t)(codec == 0 ? enc_fp8<0>(y[i]) : enc_fp8<1>(y[i]));
}

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

hipError_t launch_encode_f32(const float* y, int64_t n, int codec, uint8_t* q, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 1 << 16);
  hipLaunchKernelGGL(encode_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, st, y, n, codec, q);
  return hipGetLastError();
}

}  // namespace fp8moe

static int launch_status(hipError_t e) { return e == hipSuccess ? FP8MOE_OK : FP8MOE_ERR_LAUNCH; }
static hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

extern "C" {

int quantize_rowwise(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x, int codec, void* q, float* scale,
                     void* stream) {
  const int st = check_quantize_rowwise(x_bf16, rows, cols, ld_x, codec, q, scale);
  if (st) return st;
  return launch_status(launch_quantize_rowwise(static_cast<const uint16_t*>(x_bf16), rows, cols, ld_x, codec,
                                               static_cast<uint8_t*>(q), scale, as_stream(stream)));
}

int swiglu_quantize_rowwise(const void* h1_bf16, int64_t rows, int64_t F, int64_t ld_h1, int codec, void* a2_bf16,
                            void* q, float* scale, void* stream) {
  const int st = check_swiglu(h1_bf16, rows, F, ld_h1, codec, a2_bf16, q, scale, nullptr, false);
  if (st) return st;
  return launch_status(launch_swiglu_quantize_rowwise(static_cast<const uint16_t*>(h1_bf16), rows, F, ld_h1, codec,
                                                      static_cast<uint16_t*>(a2_bf16), static_cast<uint8_t*>(q),
                                                      scale, as_stream(stream)));
}

int swiglu_backward_quantize_rowwise(const void* da2_bf16, const void* h1_bf16, int64_t rows, int64_t F, int64_t ld_h1,
                                     int codec, void* dh1_bf16, void* q, float* scale, void* stream) {
  const int st = check_swiglu(h1_bf16, rows, F, ld_h1, codec, dh1_bf16, q, scale, da2_bf16, true);
  if (st) return st;
  return launch_status(launch_swiglu_backward_quantize_rowwise(
      static_cast<const uint16_t*>(da2_bf16), static_cast<const uint16_t*>(h1_bf16), rows, F, ld_h1, codec,
      static_cast<uint16_t*>(dh1_bf16), static_cast<uint8_t*>(q), scale, as_stream(stream)));
}

int quantize_blockwise(const void* x_bf16, int64_t batch, int64_t rows, int64_t cols, int block_rows, int codec,
                       void* q, float* scale, void* stream) {
  const int st = check_quantize_blockwise(x_bf16, batch, rows, cols, block_rows, codec, q, scale);
  if (st) return st;
  return launch_status(launch_quantize_blockwise(static_cast<const uint16_t*>(x_bf16), batch, rows, cols, block_rows,
                                                 codec, static_cast<uint8_t*>(q), scale, as_stream(stream)));
}

int grouped_mm_blockwise(const void* a, int a_fmt, const float* a_scale, const void* b, int b_fmt,
                         const float* b_scale, const int32_t* offs, int32_t n_groups, int64_t M, int64_t N, int64_t K,
                         void* out, int out_dtype, void* stream) {
  const int st = check_grouped_mm_blockwise(a, a_fmt, a_scale, b, b_fmt, b_scale, offs, n_groups, M, N, K, out,
                                            out_dtype);
  if (st) return st;
  return launch_status(launch_grouped_mm_blockwise(static_cast<const uint8_t*>(a), a_scale,
                                                   static_cast<const uint8_t*>(b), b_scale, offs, n_groups, M, N, K,
                                                   out, out_dtype, as_stream(stream)));
}

int64_t blockwise_token_blocks_bound(int64_t tokens, int32_t n_groups) {
  return fp8moe::blockwise_token_blocks_bound(tokens, n_groups);
}

int quantize_blockwise_tokens(const void* x_bf16, int64_t tokens, int64_t cols, const int32_t* offs, int32_t n_groups,
                              int codec, void* q_t, int64_t ld_q, float* scale, void* stream) {
  const int st = check_quantize_blockwise_tokens(x_bf16, tokens, cols, offs, n_groups, codec, q_t, ld_q, scale);
  if (st) return st;
  return launch_status(launch_quantize_blockwise_tokens(static_cast<const uint16_t*>(x_bf16), tokens, cols, offs,
                                                        n_groups, codec, static_cast<uint8_t*>(q_t), ld_q, scale,
                                                        as_stream(stream)));
}

int grouped_mm_blockwise_k(const void* a_t, const float* a_scale, const void* b_t, const float* b_scale,
                           const int32_t* offs, int32_t n_groups, int64_t tokens, int64_t ld, int64_t N, int64_t K,
                           void* out, int out_dtype, void* stream) {
  const int st = check_grouped_mm_blockwise_k(a_t, a_scale, b_t, b_scale, offs, n_groups, tokens, ld, N, K, out,
                                              out_dtype);
  if (st) return st;
  return launch_status(launch_grouped_mm_blockwise_k(static_cast<const uint8_t*>(a_t), a_scale,
                                                     static_cast<const uint8_t*>(b_t), b_scale, offs, n_groups, tokens,
                                                     ld, N, K, out, out_dtype, as_stream(stream)));
}

int64_t quantize_tensorwise_workspace_bytes(void) { return kTwPartials * 4; }

int quantize_tensorwise(const void* x_bf16, int64_t batch, int64_t rows, int64_t cols, int codec, void* q, void* q_t,
                        int64_t ld_q, float* scale, int64_t n_scale, void* workspace, void* stream) {
  const int st = check_quantize_tensorwise(x_bf16, batch, rows, cols, codec, q, q_t, ld_q, scale, n_scale, workspace);
  if (st) return st;
  return launch_status(launch_quantize_tensorwise(static_cast<const uint16_t*>(x_bf16), batch, rows, cols, codec,
                                                  static_cast<uint8_t*>(q), static_cast<uint8_t*>(q_t), ld_q, scale,
                                                  n_scale, static_cast<uint32_t*>(workspace), as_stream(stream)));
}

int64_t moe_route_workspace_bytes(int64_t slots, int32_t n_experts) {
  return route_workspace_bytes(slots, n_experts);
}

int64_t moe_route_rows_bound(int64_t slots, int32_t n_experts, int32_t pad) {
  return route_rows_bound(slots, n_experts, pad);
}

int moe_route(const int32_t* expert_ids, int64_t tokens, int32_t topk, int32_t n_experts, int32_t pad,
              int32_t* counts, int32_t* offs, int32_t* dest, int32_t* src, void* workspace, void* stream) {
  const int st = check_moe_route(expert_ids, tokens, topk, n_experts, pad, counts, offs, dest, src, workspace);
  if (st) return st;
  const int64_t S = tokens * topk;
  return launch_status(launch_moe_route(expert_ids, S, n_experts, pad, counts, offs, dest, src,
                                        route_rows_bound(S, n_experts, pad), static_cast<int32_t*>(workspace),
                                        as_stream(stream)));
}

int moe_route_noalloc(const int32_t* expert_ids, int64_t tokens, int32_t topk, int32_t n_experts, int32_t pad,
                      int32_t* counts, int32_t* offs, int32_t* dest, int32_t* src, void* stream) {
  // the library's scratch stands in for the workspace (a non-null, aligned placeholder for the check)
  const int st = check_moe_route(expert_ids, tokens, topk, n_experts, pad, counts, offs, dest, src,
                                 reinterpret_cast<const void*>(uintptr_t{256}));
  if (st) return st;
  const int64_t S = tokens * topk;
  if (route_workspace_bytes(S, n_experts) > kRouteScratchBytes) return FP8MOE_ERR_SCRATCH;
  return launch_status(launch_moe_route_noalloc(expert_ids, S, n_experts, pad, counts, offs, dest, src,
                                                route_rows_bound(S, n_experts, pad), as_stream(stream)));
}

int moe_permute(const void* x_bf16, int64_t tokens, int64_t cols, int32_t topk, const int32_t* src, int64_t rows_out,
                void* xg_bf16, void* stream) {
  const int st = check_moe_permute(x_bf16, tokens, cols, topk, src, rows_out, xg_bf16);
  if (st) return st;
  return launch_status(launch_moe_permute(static_cast<const uint16_t*>(x_bf16), tokens, cols, topk, src, rows_out,
                                          static_cast<uint16_t*>(xg_bf16), as_stream(stream)));
}

int moe_permute_quantized(const void* q, const float* scale, int64_t tokens, int64_t cols, int32_t topk,
                          const int32_t* src, int64_t rows_out, int codec, void* qg, float* scale_g, void* stream) {
  const int st = check_moe_permute_quantized(q, scale, tokens, cols, topk, src, rows_out, codec, qg, scale_g);
  if (st) return st;
  return launch_status(launch_moe_permute_quantized(static_cast<const uint8_t*>(q), scale, tokens, cols, topk, src,
                                                    rows_out, codec, static_cast<uint8_t*>(qg), scale_g,
                                                    as_stream(stream)));
}

int moe_combine(const void* yg_bf16, int64_t rows_in, const int32_t* dest, const float* weights, int64_t tokens,
                int32_t topk, int64_t cols, void* y_bf16, void* stream) {
  const int st = check_moe_combine(yg_bf16, rows_in, dest, weights, tokens, topk, cols, y_bf16);
  if (st) return st;
  return launch_status(launch_moe_combine(static_cast<const uint16_t*>(yg_bf16), rows_in, dest, weights, tokens, topk,
                                          cols, static_cast<uint16_t*>(y_bf16), as_stream(stream)));
}

int moe_permute_rowwise(const void* x_bf16, int64_t tokens, int64_t cols, int32_t topk, const int32_t* src,
                        int64_t rows_out, int codec, void* xg_bf16, void* qg, float* scale_g, void* stream) {
  const int st = check_moe_permute_rowwise(x_bf16, tokens, cols, topk, src, rows_out, codec, xg_bf16, qg, scale_g);
  if (st) return st;
  return launch_status(launch_moe_permute_rowwise(static_cast<const uint16_t*>(x_bf16), tokens, cols, topk, src,
                                                  rows_out, codec, static_cast<uint16_t*>(xg_bf16),
                                                  static_cast<uint8_t*>(qg), scale_g, as_stream(stream)));
}

int moe_combine_backward(const void* dy_bf16, const void* yg_bf16, int64_t rows, const int32_t* dest,
                         const int32_t* src, const float* weights, int64_t tokens, int32_t topk, int64_t cols,
                         int codec, void* dyg_bf16, void* q, float* scale, float* dweights, void* stream) {
  const int st = check_moe_combine_backward(dy_bf16, yg_bf16, rows, dest, src, weights, tokens, topk, cols, codec,
                                            dyg_bf16, q, scale, dweights);
  if (st) return st;
  return launch_status(launch_moe_combine_backward(
      static_cast<const uint16_t*>(dy_bf16), static_cast<const uint16_t*>(yg_bf16), rows, dest, src, weights, tokens,
      topk, cols, codec, static_cast<uint16_t*>(dyg_bf16), static_cast<uint8_t*>(q), scale, dweights,
      as_stream(stream)));
}

int quantize_colwise(const void* x_bf16, int64_t batch, int64_t rows, int64_t cols, const int32_t* offs,
                     int32_t n_groups, int codec, void* q_t, int64_t ld_q, float* scale, void* stream) {
  const int st = check_quantize_colwise(x_bf16, batch, rows, cols, offs, n_groups, codec, q_t, ld_q, scale);
  if (st) return st;
  return launch_status(launch_quantize_colwise(static_cast<const uint16_t*>(x_bf16), batch, rows, cols, offs,
                                               n_groups, codec, static_cast<uint8_t*>(q_t), ld_q, scale,
                                               as_stream(stream)));
}

int moe_permute_quantize_colwise(const void* x_bf16, int64_t tokens, int64_t cols, int32_t topk, const int32_t* src,
                                 const float* weights, int64_t rows, const int32_t* offs, int32_t n_groups, int codec,
                                 void* q_t, int64_t ld_q, float* scale, void* stream) {
  const int st = check_moe_permute_colwise(x_bf16, tokens, cols, topk, src, weights, rows, offs, n_groups, codec, q_t,
                                           ld_q, scale);
  if (st) return st;
  return launch_status(launch_moe_permute_colwise(static_cast<const uint16_t*>(x_bf16), tokens, cols, topk, src,
                                                  weights, rows, offs, n_groups, codec, static_cast<uint8_t*>(q_t),
                                                  ld_q, scale, as_stream(stream)));
}

int quantize_mx(const void* x_bf16, int64_t batch, int64_t rows, int64_t cols, int axis, const int32_t* offs,
                int32_t n_groups, int rule, int scale_layout, void* q, void* scale_e8m0, int64_t rows_pad,
                int32_t* offs_pad_out, void* stream) {
  const int st = check_quantize_mx(x_bf16, batch, rows, cols, axis, offs, n_groups, rule, scale_layout, q,
                                   scale_e8m0, rows_pad, offs_pad_out);
  if (st) return st;
  return launch_status(launch_quantize_mx(static_cast<const uint16_t*>(x_bf16), batch, rows, cols, axis, offs,
                                          n_groups, rule, scale_layout, static_cast<uint8_t*>(q),
                                          static_cast<uint8_t*>(scale_e8m0), rows_pad, offs_pad_out,
                                          as_stream(stream)));
}

int quantize_mx_dual(const void* x_bf16, int64_t batch, int64_t rows, int64_t cols, const int32_t* offs,
                     int32_t n_groups, int rule, int scale_layout, void* q, void* scale_e8m0, void* q_t,
                     void* scale_t_e8m0, int64_t rows_pad, int32_t* offs_pad_out, void* stream) {
  const int st = check_quantize_mx_dual(x_bf16, batch, rows, cols, offs, n_groups, rule, scale_layout, q, scale_e8m0,
                                        q_t, scale_t_e8m0, rows_pad, offs_pad_out);
  if (st) return st;
  return launch_status(launch_quantize_mx_dual(static_cast<const uint16_t*>(x_bf16), batch, rows, cols, offs,
                                               n_groups, rule, scale_layout, static_cast<uint8_t*>(q),
                                               static_cast<uint8_t*>(scale_e8m0), static_cast<uint8_t*>(q_t),
                                               static_cast<uint8_t*>(scale_t_e8m0), rows_pad, offs_pad_out,
                                               as_stream(stream)));
}

int moe_permute_quantize_mx_dual(const void* x_bf16, int64_t tokens, int64_t cols, int32_t topk, const int32_t* src,
                                 const float* weights, int64_t rows, const int32_t* offs, int32_t n_groups, int rule,
                                 int scale_layout, void* xg_bf16, void* q, void* scale_e8m0, void* q_t,
                                 void* scale_t_e8m0, int64_t rows_pad, int32_t* offs_pad_out, void* stream) {
  const int st = check_moe_permute_mx_dual(x_bf16, tokens, cols, topk, src, weights, rows, offs, n_groups, rule,
                                           scale_layout, xg_bf16, q, scale_e8m0, q_t, scale_t_e8m0, rows_pad,
                                           offs_pad_out);
  if (st) return st;
  return launch_status(launch_moe_permute_mx_dual(
      static_cast<const uint16_t*>(x_bf16), tokens, cols, topk, src, weights, rows, offs, n_groups, rule,
      scale_layout, static_cast<uint16_t*>(xg_bf16), static_cast<uint8_t*>(q), static_cast<uint8_t*>(scale_e8m0),
      static_cast<uint8_t*>(q_t), static_cast<uint8_t*>(scale_t_e8m0), rows_pad, offs_pad_out, as_stream(stream)));
}

int swiglu_quantize_mx_dual(const void* h1_bf16, int64_t rows, int64_t F, int64_t ld_h1, const int32_t* offs,
                            int32_t n_groups, int rule, int scale_layout, void* a2_bf16, void* q, void* scale_e8m0,
                            void* q_t, void* scale_t_e8m0, int64_t rows_pad, int32_t* offs_pad_out, void* stream) {
  const int st = check_swiglu_mx_dual(h1_bf16, nullptr, false, rows, F, ld_h1, offs, n_groups, rule, scale_layout,
                                      a2_bf16, q, scale_e8m0, q_t, scale_t_e8m0, rows_pad, offs_pad_out);
  if (st) return st;
  return launch_status(launch_swiglu_mx_dual(
      static_cast<const uint16_t*>(h1_bf16), nullptr, rows, F, ld_h1, offs, n_groups, rule, scale_layout,
      static_cast<uint16_t*>(a2_bf16), static_cast<uint8_t*>(q), static_cast<uint8_t*>(scale_e8m0),
      static_cast<uint8_t*>(q_t), static_cast<uint8_t*>(scale_t_e8m0), rows_pad, offs_pad_out, as_stream(stream)));
}

int swiglu_backward_quantize_mx_dual(const void* da2_bf16, const void* h1_bf16, int64_t rows, int64_t F,
                                     int64_t ld_h1, const int32_t* offs, int32_t n_groups, int rule,
                                     int scale_layout, void* dh1_bf16, void* q, void* scale_e8m0, void* q_t,
                                     void* scale_t_e8m0, int64_t rows_pad, int32_t* offs_pad_out, void* stream) {
  const int st = check_swiglu_mx_dual(h1_bf16, da2_bf16, true, rows, F, ld_h1, offs, n_groups, rule, scale_layout,
                                      dh1_bf16, q, scale_e8m0, q_t, scale_t_e8m0, rows_pad, offs_pad_out);
  if (st) return st;
  return launch_status(launch_swiglu_mx_dual(
      static_cast<const uint16_t*>(h1_bf16), static_cast<const uint16_t*>(da2_bf16), rows, F, ld_h1, offs, n_groups,
      rule, scale_layout, static_cast<uint16_t*>(dh1_bf16), static_cast<uint8_t*>(q),
      static_cast<uint8_t*>(scale_e8m0), static_cast<uint8_t*>(q_t), static_cast<uint8_t*>(scale_t_e8m0), rows_pad,
      offs_pad_out, as_stream(stream)));
}

int64_t quantize_mx_rows_bound(int64_t rows, int32_t n_groups) { return mx_rows_bound(rows, n_groups); }

int grouped_mm_scaled(int mode, const void* a, int a_fmt, const void* a_scale, const void* b, int b_fmt,
                      const void* b_scale, int scale_kind, const int32_t* offs, int32_t n_groups, int64_t M,
                      int64_t N, int64_t K, void* out, int out_dtype, void* stream) {
  const int st = check_grouped_mm(mode, a, a_fmt, a_scale, b, b_fmt, b_scale, scale_kind, offs, n_groups, M, N,
                                  K, out, out_dtype);
  if (st) return st;
  GemmArgs g{mode, a_fmt, b_fmt, scale_kind, out_dtype, a, b, a_scale, b_scale, offs, n_groups, M, N, K, out};
  return launch_status(launch_grouped_mm(g, as_stream(stream)));
}

int fp8moe_encode_f32(const float* y, int64_t n, int codec, void* q, void* stream) {
  const int st = check_encode_f32(y, n, codec, q);
  if (st) return st;
  return launch_status(launch_encode_f32(y, n, codec, static_cast<uint8_t*>(q), as_stream(stream)));
}

const char* fp8moe_status_string(int status) {
  switch (status) {
    case FP8MOE_OK: return "ok";
    case FP8MOE_ERR_NULL: return "null pointer";
    case FP8MOE_ERR_SHAPE: return "invalid shape";
    case FP8MOE_ERR_ENUM: return "invalid enum value";
    case FP8MOE_ERR_ALIGN: return "alignment or divisibility violated";
    case FP8MOE_ERR_UNSUPPORTED: return "unsupported combination";
    case FP8MOE_ERR_LAUNCH: return "kernel launch failed";
    case FP8MOE_ERR_DEVICE: return "device query failed";
    case FP8MOE_ERR_SCRATCH: return "the call needs more scratch than the allocation-free entry point holds";
    default: return "unknown status";
  }
}

int fp8moe_default_codec(int hip_device, int* codec_out) {
  if (codec_out == nullptr) return FP8MOE_ERR_NULL;
  hipDeviceProp_t p;
  if (hipGetDeviceProperties(&p, hip_device) != hipSuccess) return FP8MOE_ERR_DEVICE;
  if (std::strncmp(p.gcnArchName, "gfx950", 6) == 0) { *codec_out = FP8MOE_E4M3FN; return FP8MOE_OK; }
  if (std::strncmp(p.gcnArchName, "gfx942", 6) == 0) { *codec_out = FP8MOE_E4M3FNUZ; return FP8MOE_OK; }
  return FP8MOE_ERR_UNSUPPORTED;
}

int fp8moe_set_colwise_poll_budget(int polls) { return set_colwise_poll_budget(polls); }

int fp8moe_set_colwise_chunk_rows(int rows) { return set_colwise_chunk_rows(rows); }

int fp8moe_version(void) { return 108; }

}  // extern "C"

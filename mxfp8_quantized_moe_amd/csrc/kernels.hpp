// Internal launchers: one per operation, called by the C ABI after validation.
// Each enqueues kernels on `st` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

namespace fp8moe {

// Compute units of the current device (queried once per device).
int device_cu_count();

hipError_t launch_quantize_rowwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int codec,
                                   uint8_t* q, float* scale, hipStream_t st);

hipError_t launch_moe_permute_colwise(const uint16_t* x, int64_t tokens, int64_t cols, int topk, const int32_t* src,
                                      const float* weights, int64_t rows, const int32_t* offs, int32_t n_groups,
                                      int codec, uint8_t* q_t, int64_t ld_q, float* scale, hipStream_t st);
hipError_t launch_quantize_colwise(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols,
                                   const int32_t* offs, int32_t n_groups, int codec, uint8_t* q_t,
                                   int64_t ld_q, float* scale, hipStream_t st);

hipError_t launch_quantize_mx(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, int axis,
                              const int32_t* offs, int32_t n_groups, int rule, int scale_layout, uint8_t* q,
                              uint8_t* sc, int64_t rows_pad, int32_t* offs_pad_out, hipStream_t st);

hipError_t launch_quantize_mx_dual(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols,
                                   const int32_t* offs, int32_t n_groups, int rule, int scale_layout, uint8_t* q,
                                   uint8_t* sc, uint8_t* q_t, uint8_t* sc_t, int64_t rows_pad,
                                   int32_t* offs_pad_out, hipStream_t st);

// SwiGLU (da2 null) or its backward (da2 given) computed on the fly and quantized into both MX forms.
hipError_t launch_moe_permute_mx_dual(const uint16_t* x, int64_t tokens, int64_t cols, int topk, const int32_t* src,
                                     const float* weights, int64_t rows, const int32_t* offs, int32_t n_groups,
                                     int rule, int scale_layout, uint16_t* xg, uint8_t* q, uint8_t* sc, uint8_t* q_t,
                                     uint8_t* sc_t, int64_t rows_pad, int32_t* offs_pad_out, hipStream_t st);
hipError_t launch_swiglu_mx_dual(const uint16_t* h1, const uint16_t* da2, int64_t rows, int64_t F, int64_t ld_h1,
                                 const int32_t* offs, int32_t n_groups, int rule, int scale_layout, uint16_t* out,
                                 uint8_t* q, uint8_t* sc, uint8_t* q_t, uint8_t* sc_t, int64_t rows_pad,
                                 int32_t* offs_pad_out, hipStream_t st);

struct GemmArgs {
  int mode, a_fmt, b_fmt, scale_kind, out_dtype;
  const void* a;
  const void* b;
  const void* sa;
  const void* sb;
  const int32_t* offs;
  int n_groups;
  int64_t M, N, K;
  void* out;
};

hipError_t launch_grouped_mm(const GemmArgs& g, hipStream_t st);

// Poll budget of the single-pass colwise exchange (negative: the default); returns the previous one.
int set_colwise_poll_budget(int polls);
// Chunk height of the single-pass colwise quantizer (128 or 512: forced; else per call); returns the previous one.
int set_colwise_chunk_rows(int rows);

hipError_t launch_encode_f32(const float* y, int64_t n, int codec, uint8_t* q, hipStream_t st);
hipError_t launch_quantize_blockwise(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, int block_rows,
                                     int codec, uint8_t* q, float* scale, hipStream_t st);
hipError_t launch_grouped_mm_blockwise(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                                       const int32_t* offs, int n_groups, int64_t M, int64_t N, int64_t K, void* out,
                                       int out_dtype, hipStream_t st);
hipError_t launch_quantize_blockwise_tokens(const uint16_t* x, int64_t M, int64_t C, const int32_t* offs, int n_groups,
                                            int codec, uint8_t* q_t, int64_t ld_q, float* scale, hipStream_t st);
hipError_t launch_grouped_mm_blockwise_k(const uint8_t* a_t, const float* sa, const uint8_t* b_t, const float* sb,
                                         const int32_t* offs, int n_groups, int64_t M, int64_t ld, int64_t N,
                                         int64_t K, void* out, int out_dtype, hipStream_t st);
hipError_t launch_quantize_tensorwise(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, int codec,
                                      uint8_t* q, uint8_t* q_t, int64_t ld_q, float* scale, int64_t n_scale,
                                      uint32_t* part, hipStream_t st);
hipError_t launch_moe_route(const int32_t* ids, int64_t S, int E, int pad, int32_t* counts, int32_t* offs,
                            int32_t* dest, int32_t* src, int64_t rows_bound, int32_t* workspace, hipStream_t st);
hipError_t launch_moe_route_noalloc(const int32_t* ids, int64_t S, int E, int pad, int32_t* counts, int32_t* offs,
                                    int32_t* dest, int32_t* src, int64_t rows_bound, hipStream_t st);
hipError_t launch_moe_permute(const uint16_t* x, int64_t tokens, int64_t cols, int topk, const int32_t* src,
                              int64_t rows_out, uint16_t* xg, hipStream_t st);
hipError_t launch_moe_permute_quantized(const uint8_t* q, const float* scale, int64_t tokens, int64_t cols, int topk,
                                        const int32_t* src, int64_t rows_out, int codec, uint8_t* qg,
                                        float* scale_g, hipStream_t st);
hipError_t launch_moe_combine(const uint16_t* yg, int64_t rows_in, const int32_t* dest, const float* w,
                              int64_t tokens, int topk, int64_t cols, uint16_t* y, hipStream_t st);
hipError_t launch_moe_permute_rowwise(const uint16_t* x, int64_t tokens, int64_t cols, int topk, const int32_t* src,
                                      int64_t rows_out, int codec, uint16_t* xg, uint8_t* qg, float* scale_g,
                                      hipStream_t st);
hipError_t launch_moe_combine_backward(const uint16_t* dy, const uint16_t* yg, int64_t rows, const int32_t* dest,
                                       const int32_t* src, const float* w, int64_t tokens, int topk, int64_t cols,
                                       int codec, uint16_t* dyg, uint8_t* q, float* scale, float* dw,
                                       hipStream_t st);
hipError_t launch_swiglu_quantize_rowwise(const uint16_t* h1, int64_t rows, int64_t F, int64_t ld_h1, int codec,
                                          uint16_t* a2, uint8_t* q, float* scale, hipStream_t st);
hipError_t launch_swiglu_backward_quantize_rowwise(const uint16_t* da2, const uint16_t* h1, int64_t rows, int64_t F,
                                                   int64_t ld_h1, int codec, uint16_t* dh1, uint8_t* q, float* scale,
                                                   hipStream_t st);

}  // namespace fp8moe

// Host-only argument validation for the C ABI.  Pure C++: no HIP header and
// no HIP call, so every rejection path runs (and is tested) without a GPU.
#pragma once

#include <stdint.h>

namespace fp8moe {

int check_quantize_rowwise(const void* x, int64_t rows, int64_t cols, int64_t ld_x, int codec, const void* q,
                           const void* scale);
int check_quantize_colwise(const void* x, int64_t batch, int64_t rows, int64_t cols, const int32_t* offs,
                           int32_t n_groups, int codec, const void* q_t, int64_t ld_q, const void* scale);
int check_quantize_mx(const void* x, int64_t batch, int64_t rows, int64_t cols, int axis, const int32_t* offs,
                      int32_t n_groups, int rule, int scale_layout, const void* q, const void* sc,
                      int64_t rows_pad, const int32_t* offs_pad_out);
int check_moe_permute_mx_dual(const void* x, int64_t tokens, int64_t cols, int32_t topk, const int32_t* src,
                              const float* weights, int64_t rows, const int32_t* offs, int32_t n_groups, int rule,
                              int scale_layout, const void* xg, const void* q, const void* sc, const void* q_t,
                              const void* sc_t, int64_t rows_pad, const int32_t* offs_pad_out);
int check_moe_permute_colwise(const void* x, int64_t tokens, int64_t cols, int32_t topk, const int32_t* src,
                              const float* weights, int64_t rows, const int32_t* offs, int32_t n_groups, int codec,
                              const void* q_t, int64_t ld_q, const void* scale);
int check_quantize_mx_dual(const void* x, int64_t batch, int64_t rows, int64_t cols, const int32_t* offs,
                           int32_t n_groups, int rule, int scale_layout, const void* q, const void* sc,
                           const void* q_t, const void* sc_t, int64_t rows_pad, const int32_t* offs_pad_out);
int check_swiglu_mx_dual(const void* h1, const void* da2, bool backward, int64_t rows, int64_t F, int64_t ld_h1,
                         const int32_t* offs, int32_t n_groups, int rule, int scale_layout, const void* out,
                         const void* q, const void* sc, const void* q_t, const void* sc_t, int64_t rows_pad,
                         const int32_t* offs_pad_out);
// Bytes of an e8m0 scale matrix of `rows` rows and `nb` 32-blocks per row in
// the K4 layout (nb rounded up to whole 128-wide stages), or -1 on overflow.
int64_t mx_k4_bytes(int64_t rows, int64_t nb);
int check_grouped_mm(int mode, const void* a, int a_fmt, const void* sa, const void* b, int b_fmt,
                     const void* sb, int scale_kind, const int32_t* offs, int32_t n_groups, int64_t M,
                     int64_t N, int64_t K, const void* out, int out_dtype);
int check_encode_f32(const void* y, int64_t n, int codec, const void* q);
int check_swiglu(const void* h1, int64_t rows, int64_t F, int64_t ld_h1, int codec, const void* out_bf16,
                 const void* q, const void* scale, const void* da2, bool backward);

int64_t mx_rows_bound(int64_t rows, int32_t n_groups);

int check_quantize_blockwise(const void* x, int64_t batch, int64_t rows, int64_t cols, int block_rows, int codec,
                             const void* q, const void* scale);
int check_grouped_mm_blockwise(const void* a, int a_fmt, const void* sa, const void* b, int b_fmt, const void* sb,
                               const int32_t* offs, int32_t n_groups, int64_t M, int64_t N, int64_t K,
                               const void* out, int out_dtype);

int64_t blockwise_token_blocks_bound(int64_t M, int32_t n_groups);
int check_quantize_blockwise_tokens(const void* x, int64_t M, int64_t C, const int32_t* offs, int32_t n_groups,
                                    int codec, const void* q_t, int64_t ld_q, const void* scale);
int check_grouped_mm_blockwise_k(const void* a_t, const void* sa, const void* b_t, const void* sb, const int32_t* offs,
                                 int32_t n_groups, int64_t M, int64_t ld, int64_t N, int64_t K, const void* out,
                                 int out_dtype);

// Tensorwise quantization: partial maxima (one u32 each) of the first pass.
constexpr int kTwPartials = 1024;
int check_quantize_tensorwise(const void* x, int64_t batch, int64_t rows, int64_t cols, int codec, const void* q,
                              const void* q_t, int64_t ld_q, const void* scale, int64_t n_scale,
                              const void* workspace);

// Routing: slots per block of the histogram and rank launches, and the most
// experts one route call takes (one workgroup scans them).
constexpr int kRouteSlots = 256;
constexpr int kRouteMaxExperts = 1024;
constexpr int64_t kRouteScratchBytes = 4 << 20;   // the fixed scratch of moe_route_noalloc
constexpr int kMaxDevices = 64;
inline int64_t route_blocks(int64_t slots) { return (slots + kRouteSlots - 1) / kRouteSlots; }
// Workspace bytes of a route call, rows of its grouped layout; -1 for invalid sizes.
int64_t route_workspace_bytes(int64_t slots, int32_t n_experts);
int64_t route_rows_bound(int64_t slots, int32_t n_experts, int32_t pad);
int check_moe_route(const int32_t* ids, int64_t tokens, int32_t topk, int32_t E, int32_t pad, const int32_t* counts,
                    const int32_t* offs, const int32_t* dest, const int32_t* src, const void* workspace);
int check_moe_permute(const void* x, int64_t tokens, int64_t cols, int32_t topk, const int32_t* src,
                      int64_t rows_out, const void* xg);
int check_moe_permute_quantized(const void* q, const float* scale, int64_t tokens, int64_t cols, int32_t topk,
                                const int32_t* src, int64_t rows_out, int codec, const void* qg,
                                const float* scale_g);
int check_moe_combine(const void* yg, int64_t rows_in, const int32_t* dest, const float* w, int64_t tokens,
                      int32_t topk, int64_t cols, const void* y);
// Rowwise quantization holds rows of up to this many columns in registers (256 threads x 8 chunks of 8);
// longer gathered rows are cast from the gathered bf16 copy, which must then be written.
constexpr int64_t kRowwiseRegCols = 16384;
int check_moe_permute_rowwise(const void* x, int64_t tokens, int64_t cols, int32_t topk, const int32_t* src,
                              int64_t rows_out, int codec, const void* xg, const void* qg, const float* scale_g);
// Combine's backward holds a token's gradient row in registers: at most this many columns.
constexpr int64_t kCombineBwdMaxCols = 16384;
int check_moe_combine_backward(const void* dy, const void* yg, int64_t rows, const int32_t* dest,
                               const int32_t* src, const float* w, int64_t tokens, int32_t topk, int64_t cols,
                               int codec, const void* dyg, const void* q, const float* scale, const float* dw);

}  // namespace fp8moe

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

}  // namespace fp8moe

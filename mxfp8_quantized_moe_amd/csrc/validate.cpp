// Host-only validation of the C ABI arguments (see include/fp8moe.h for the
// contract of each entry point).  No HIP header, no HIP call.
#include "validate.hpp"

#include <stdint.h>

#include "../../include/fp8moe.h"

namespace fp8moe {

namespace {

constexpr int64_t kI32Max = 2147483647;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool need(const void* p, int64_t elems) { return elems == 0 || p != nullptr; }

// a*b without overflow for non-negative operands; -1 if it would exceed int64.
int64_t mul(int64_t a, int64_t b) {
  if (a == 0 || b == 0) return 0;
  if (a > INT64_MAX / b) return -1;
  return a * b;
}

}  // namespace

int64_t mx_rows_bound(int64_t rows, int32_t n_groups) {
  if (rows < 0 || n_groups < 0) return -1;
  return (rows + 31LL * n_groups + 31) / 32 * 32;
}

int check_quantize_rowwise(const void* x, int64_t rows, int64_t cols, int64_t ld_x, int codec, const void* q,
                           const void* scale) {
  if (codec != FP8MOE_E4M3FN && codec != FP8MOE_E4M3FNUZ) return FP8MOE_ERR_ENUM;
  if (rows < 0 || cols < 0 || ld_x < cols || rows > kI32Max * 256LL || cols > kI32Max) return FP8MOE_ERR_SHAPE;
  const int64_t n = mul(rows, cols);
  if (n < 0 || mul(rows, ld_x) < 0) return FP8MOE_ERR_SHAPE;
  if (!need(x, n) || !need(q, n) || !need(scale, rows)) return FP8MOE_ERR_NULL;
  if (cols % 8 || ld_x % 8 || !aligned(x, 16) || !aligned(q, 16) || !aligned(scale, 4)) return FP8MOE_ERR_ALIGN;
  return FP8MOE_OK;
}

int check_quantize_colwise(const void* x, int64_t batch, int64_t rows, int64_t cols, const int32_t* offs,
                           int32_t n_groups, int codec, const void* q_t, int64_t ld_q, const void* scale) {
  if (codec != FP8MOE_E4M3FN && codec != FP8MOE_E4M3FNUZ) return FP8MOE_ERR_ENUM;
  if (batch < 1 || rows < 0 || cols < 0 || ld_q < rows) return FP8MOE_ERR_SHAPE;
  if (offs && (batch != 1 || n_groups < 1)) return FP8MOE_ERR_SHAPE;
  if (rows > kI32Max / 2 || cols > kI32Max / 2 || n_groups > (1 << 20)) return FP8MOE_ERR_SHAPE;
  const int64_t groups = offs ? n_groups : batch;
  const int64_t n_in = mul(mul(batch, rows), cols);
  const int64_t n_out = mul(mul(batch, cols), ld_q);
  if (n_in < 0 || n_out < 0 || mul(groups, cols) < 0) return FP8MOE_ERR_SHAPE;
  // grid: units x 64-column strips must fit a 1D launch
  const int64_t units = offs ? (rows + 16LL * n_groups + 511) / 512 + n_groups : batch * ((rows + 511) / 512 + 1);
  if (mul(units, (cols + 63) / 64) < 0 || mul(units, (cols + 63) / 64) > kI32Max) return FP8MOE_ERR_SHAPE;
  if (!need(x, n_in) || !need(q_t, mul(mul(batch, cols), rows)) || !need(scale, mul(groups, cols)))
    return FP8MOE_ERR_NULL;
  if (cols % 8 || ld_q % 16 || !aligned(x, 16) || !aligned(q_t, 16) || !aligned(scale, 4)) return FP8MOE_ERR_ALIGN;
  return FP8MOE_OK;
}

int check_moe_permute_colwise(const void* x, int64_t tokens, int64_t cols, int32_t topk, const int32_t* src,
                              const float* weights, int64_t rows, const int32_t* offs, int32_t n_groups, int codec,
                              const void* q_t, int64_t ld_q, const void* scale) {
  if (tokens < 0 || cols < 0 || topk < 1 || rows < 0 || cols > kI32Max) return FP8MOE_ERR_SHAPE;
  const int64_t S = mul(tokens, topk), nx = mul(tokens, cols);
  if (S < 0 || S > kI32Max || nx < 0) return FP8MOE_ERR_SHAPE;
  if (offs == nullptr) return FP8MOE_ERR_NULL;   // the grouped layout of moe_route
  // the gathered [rows][cols] tensor: q_t stands in for its pointer and alignment
  const int st = check_quantize_colwise(rows && cols ? q_t : nullptr, 1, rows, cols, offs, n_groups, codec, q_t,
                                        ld_q, scale);
  if (st) return st;
  if (!need(x, nx) || !need(src, rows)) return FP8MOE_ERR_NULL;
  if (!aligned(x, 16) || !aligned(src, 4) || !aligned(weights, 4)) return FP8MOE_ERR_ALIGN;
  return FP8MOE_OK;
}

int64_t mx_k4_bytes(int64_t rows, int64_t nb) { return mul(mul(rows, (nb + 3) / 4), 4); }

int check_quantize_mx(const void* x, int64_t batch, int64_t rows, int64_t cols, int axis, const int32_t* offs,
                      int32_t n_groups, int rule, int scale_layout, const void* q, const void* sc,
                      int64_t rows_pad, const int32_t* offs_pad_out) {
  if (rule != FP8MOE_MX_FLOOR_OCP && rule != FP8MOE_MX_CEIL) return FP8MOE_ERR_ENUM;
  if (axis != 0 && axis != 1) return FP8MOE_ERR_ENUM;
  if (scale_layout != FP8MOE_MX_LAYOUT_ROWS && scale_layout != FP8MOE_MX_LAYOUT_K4) return FP8MOE_ERR_ENUM;
  const bool k4 = scale_layout == FP8MOE_MX_LAYOUT_K4;
  if (batch < 1 || rows < 0 || cols < 0) return FP8MOE_ERR_SHAPE;
  if (rows > kI32Max / 2 || cols > kI32Max / 2) return FP8MOE_ERR_SHAPE;
  const int64_t n_in = mul(mul(batch, rows), cols);
  if (n_in < 0) return FP8MOE_ERR_SHAPE;
  if (axis == 1) {
    if (offs) return FP8MOE_ERR_UNSUPPORTED;
    const int64_t nsc = k4 ? mx_k4_bytes(mul(batch, rows), cols / 32) : n_in / 32;
    if (nsc < 0 || (k4 && nsc > kI32Max)) return FP8MOE_ERR_SHAPE;
    if (!need(x, n_in) || !need(q, n_in) || !need(sc, nsc)) return FP8MOE_ERR_NULL;
    if (cols % 32 || !aligned(x, 16) || !aligned(q, 16)) return FP8MOE_ERR_ALIGN;
    return FP8MOE_OK;
  }
  if (cols % 8 || !aligned(x, 16) || !aligned(q, 16)) return FP8MOE_ERR_ALIGN;
  if (offs == nullptr) {
    if (rows % 32) return FP8MOE_ERR_ALIGN;
    if (mul(batch * ((rows + 511) / 512), (cols + 63) / 64) > kI32Max) return FP8MOE_ERR_SHAPE;
    const int64_t nsc = k4 ? mx_k4_bytes(mul(batch, cols), rows / 32) : n_in / 32;
    if (nsc < 0 || (k4 && nsc > kI32Max)) return FP8MOE_ERR_SHAPE;
    if (!need(x, n_in) || !need(q, n_in) || !need(sc, nsc)) return FP8MOE_ERR_NULL;
    return FP8MOE_OK;
  }
  if (batch != 1 || n_groups < 1 || n_groups > (1 << 20)) return FP8MOE_ERR_SHAPE;
  if (rows_pad % 32) return FP8MOE_ERR_ALIGN;
  if (rows_pad < mx_rows_bound(rows, n_groups) || rows_pad > kI32Max / 2) return FP8MOE_ERR_SHAPE;
  const int64_t n_out = mul(cols, rows_pad);
  if (n_out < 0) return FP8MOE_ERR_SHAPE;
  const int64_t units = (rows_pad + 511) / 512 + n_groups + 1;
  if (mul(units, (cols + 63) / 64 + 1) > kI32Max) return FP8MOE_ERR_SHAPE;
  const int64_t nsc = k4 ? mx_k4_bytes(cols, rows_pad / 32) : n_out / 32;
  if (nsc < 0 || (k4 && nsc > kI32Max)) return FP8MOE_ERR_SHAPE;
  if (!need(x, n_in) || !need(q, n_out) || !need(sc, nsc)) return FP8MOE_ERR_NULL;
  return FP8MOE_OK;
}

int check_quantize_mx_dual(const void* x, int64_t batch, int64_t rows, int64_t cols, const int32_t* offs,
                           int32_t n_groups, int rule, int scale_layout, const void* q, const void* sc,
                           const void* q_t, const void* sc_t, int64_t rows_pad, const int32_t* offs_pad_out) {
  int st = check_quantize_mx(x, batch, rows, cols, 1, nullptr, 0, rule, scale_layout, q, sc, 0, nullptr);
  if (st) return st;
  st = check_quantize_mx(x, batch, rows, cols, 0, offs, n_groups, rule, scale_layout, q_t, sc_t, rows_pad,
                         offs_pad_out);
  if (st) return st;
  // one workgroup per 128 x 128 item: the grid must fit a 1D launch
  const int64_t units = offs ? (rows_pad + 127) / 128 + n_groups + 1 : mul(batch, (rows + 127) / 128);
  const int64_t grid = mul(units, (cols + 127) / 128 > 0 ? (cols + 127) / 128 : 1);
  if (units < 0 || grid < 0 || grid > kI32Max) return FP8MOE_ERR_SHAPE;
  return FP8MOE_OK;
}

int check_moe_permute_mx_dual(const void* x, int64_t tokens, int64_t cols, int32_t topk, const int32_t* src,
                              const float* weights, int64_t rows, const int32_t* offs, int32_t n_groups, int rule,
                              int scale_layout, const void* xg, const void* q, const void* sc, const void* q_t,
                              const void* sc_t, int64_t rows_pad, const int32_t* offs_pad_out) {
  if (tokens < 0 || cols < 0 || topk < 1 || rows < 0 || cols > kI32Max) return FP8MOE_ERR_SHAPE;
  const int64_t S = mul(tokens, topk), nx = mul(tokens, cols);
  if (S < 0 || S > kI32Max || nx < 0) return FP8MOE_ERR_SHAPE;
  if (offs == nullptr) return FP8MOE_ERR_NULL;   // the grouped layout of moe_route
  // the gathered [rows][cols] tensor: q stands in for its pointer and alignment
  const int st = check_quantize_mx_dual(rows && cols ? q : nullptr, 1, rows, cols, offs, n_groups, rule, scale_layout,
                                        q, sc, q_t, sc_t, rows_pad, offs_pad_out);
  if (st) return st;
  if (!need(x, nx) || !need(src, rows)) return FP8MOE_ERR_NULL;
  if (!aligned(x, 16) || !aligned(xg, 16) || !aligned(src, 4) || !aligned(weights, 4)) return FP8MOE_ERR_ALIGN;
  return FP8MOE_OK;
}

int check_swiglu_mx_dual(const void* h1, const void* da2, bool backward, int64_t rows, int64_t F, int64_t ld_h1,
                         const int32_t* offs, int32_t n_groups, int rule, int scale_layout, const void* out,
                         const void* q, const void* sc, const void* q_t, const void* sc_t, int64_t rows_pad,
                         const int32_t* offs_pad_out) {
  if (rows < 0 || F < 0 || F > kI32Max / 4 || ld_h1 < 2 * F || mul(rows, ld_h1) < 0) return FP8MOE_ERR_SHAPE;
  const int64_t cols = backward ? 2 * F : F;
  // the tensor the MX forms are taken of: its shape, pointer and alignment stand in for x
  const int st = check_quantize_mx_dual(rows && cols ? h1 : nullptr, 1, rows, cols, offs, n_groups, rule,
                                        scale_layout, q, sc, q_t, sc_t, rows_pad, offs_pad_out);
  if (st) return st;
  const int64_t n = mul(rows, F);
  if (!need(h1, n) || (backward && !need(da2, n))) return FP8MOE_ERR_NULL;
  if (F % (backward ? 128 : 32) || ld_h1 % 8 || !aligned(h1, 16) || !aligned(da2, 16) || !aligned(out, 16))
    return FP8MOE_ERR_ALIGN;
  return FP8MOE_OK;
}

int check_grouped_mm(int mode, const void* a, int a_fmt, const void* sa, const void* b, int b_fmt,
                     const void* sb, int scale_kind, const int32_t* offs, int32_t n_groups, int64_t M,
                     int64_t N, int64_t K, const void* out, int out_dtype) {
  if (mode != FP8MOE_GROUPED_M && mode != FP8MOE_GROUPED_K) return FP8MOE_ERR_ENUM;
  if (a_fmt < 0 || a_fmt > 2 || b_fmt < 0 || b_fmt > 2) return FP8MOE_ERR_ENUM;
  if (scale_kind < 0 || scale_kind > 3) return FP8MOE_ERR_ENUM;
  if (out_dtype != FP8MOE_OUT_BF16 && out_dtype != FP8MOE_OUT_F32) return FP8MOE_ERR_ENUM;
  if (M < 0 || N < 0 || K < 0 || n_groups < 1 || n_groups > (1 << 20)) return FP8MOE_ERR_SHAPE;
  if (M > kI32Max / 2 || N > kI32Max / 2 || K > kI32Max / 2) return FP8MOE_ERR_SHAPE;
  if (offs == nullptr && n_groups != 1) return FP8MOE_ERR_NULL;
  const bool a_bf16 = a_fmt == FP8MOE_OPD_BF16, b_bf16 = b_fmt == FP8MOE_OPD_BF16;
  if (a_bf16 != b_bf16) return FP8MOE_ERR_UNSUPPORTED;
  if (a_bf16 && (scale_kind != FP8MOE_SCALE_NONE || mode != FP8MOE_GROUPED_K)) return FP8MOE_ERR_UNSUPPORTED;
  if (!a_bf16 && scale_kind == FP8MOE_SCALE_NONE) return FP8MOE_ERR_UNSUPPORTED;
  const bool e8 = scale_kind == FP8MOE_SCALE_E8M0, k4 = scale_kind == FP8MOE_SCALE_E8M0_K4;
  if ((e8 || k4) && (a_fmt != FP8MOE_OPD_E4M3FN || b_fmt != FP8MOE_OPD_E4M3FN)) return FP8MOE_ERR_UNSUPPORTED;
  const int64_t E = n_groups;
  int64_t na, nb, no, nsa, nsb;
  if (mode == FP8MOE_GROUPED_M) {
    na = mul(M, K); nb = mul(mul(E, N), K); no = mul(M, N);
    nsa = e8 ? mul(M, K / 32) : k4 ? mx_k4_bytes(M, K / 32) : M;
    nsb = e8 ? mul(mul(E, N), K / 32) : k4 ? mx_k4_bytes(mul(E, N), K / 32) : mul(E, N);
  } else {
    na = mul(N, M); nb = mul(K, M); no = mul(mul(E, N), K);
    nsa = e8 ? mul(N, M / 32) : k4 ? mx_k4_bytes(N, M / 32) : mul(E, N);
    nsb = e8 ? mul(K, M / 32) : k4 ? mx_k4_bytes(K, M / 32) : mul(E, K);
  }
  if (na < 0 || nb < 0 || no < 0 || nsa < 0 || nsb < 0 || mul(no, 4) < 0) return FP8MOE_ERR_SHAPE;
  if (k4 && (nsa > kI32Max || nsb > kI32Max)) return FP8MOE_ERR_SHAPE;   // 32-bit offsets in the kernel
  if (!need(a, na) || !need(b, nb) || !need(out, no)) return FP8MOE_ERR_NULL;
  if (scale_kind != FP8MOE_SCALE_NONE && (!need(sa, nsa) || !need(sb, nsb))) return FP8MOE_ERR_NULL;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(out, 16)) return FP8MOE_ERR_ALIGN;
  if ((scale_kind == FP8MOE_SCALE_F32 || k4) && (!aligned(sa, 4) || !aligned(sb, 4))) return FP8MOE_ERR_ALIGN;
  if (a_bf16) {
    if (N % 8 || K % 8 || M % 8) return FP8MOE_ERR_ALIGN;
  } else if (mode == FP8MOE_GROUPED_M) {
    if (K > (1 << 23)) return FP8MOE_ERR_SHAPE;     // tile-row offsets are 32-bit in the kernel
    if (K % 16) return FP8MOE_ERR_ALIGN;
    if ((e8 || k4) && K % 32) return FP8MOE_ERR_ALIGN;
  } else {
    if (M > (1 << 23)) return FP8MOE_ERR_SHAPE;     // tile-row offsets are 32-bit in the kernel
    if (M % 16) return FP8MOE_ERR_ALIGN;
    if ((e8 || k4) && M % 32) return FP8MOE_ERR_ALIGN;
  }
  return FP8MOE_OK;
}

int check_swiglu(const void* h1, int64_t rows, int64_t F, int64_t ld_h1, int codec, const void* out_bf16,
                 const void* q, const void* scale, const void* da2, bool backward) {
  if (codec != FP8MOE_E4M3FN && codec != FP8MOE_E4M3FNUZ) return FP8MOE_ERR_ENUM;
  if (rows < 0 || F < 0 || rows > kI32Max * 256LL || F > kI32Max / 2 || ld_h1 < 2 * F) return FP8MOE_ERR_SHAPE;
  const int64_t n = mul(rows, 2 * F);
  if (n < 0 || mul(rows, ld_h1) < 0) return FP8MOE_ERR_SHAPE;
  if ((q == nullptr) != (scale == nullptr)) return FP8MOE_ERR_NULL;   // codes and scales come together
  if (!need(h1, n) || !need(out_bf16, n) || (backward && !need(da2, n))) return FP8MOE_ERR_NULL;
  if (F % 8 || ld_h1 % 8 || !aligned(h1, 16) || !aligned(out_bf16, 16) || !aligned(q, 16) || !aligned(scale, 4) ||
      (backward && !aligned(da2, 16)))
    return FP8MOE_ERR_ALIGN;
  return FP8MOE_OK;
}

int check_quantize_blockwise(const void* x, int64_t batch, int64_t rows, int64_t cols, int block_rows, int codec,
                             const void* q, const void* scale) {
  if (codec != FP8MOE_E4M3FN && codec != FP8MOE_E4M3FNUZ) return FP8MOE_ERR_ENUM;
  if (block_rows != 1 && block_rows != 128) return FP8MOE_ERR_ENUM;
  if (batch < 1 || rows < 0 || cols < 0 || rows > kI32Max || cols > kI32Max) return FP8MOE_ERR_SHAPE;
  const int64_t n = mul(batch, mul(rows, cols));
  const int64_t tiles = mul(batch, mul((rows + block_rows - 1) / block_rows, (cols + 127) / 128));
  if (n < 0 || tiles < 0 || tiles > (block_rows == 1 ? kI32Max * 16LL : kI32Max)) return FP8MOE_ERR_SHAPE;
  if (!need(x, n) || !need(q, n) || !need(scale, cols ? tiles : 0)) return FP8MOE_ERR_NULL;
  if (cols % 8 || !aligned(x, 16) || !aligned(q, 16) || !aligned(scale, 4)) return FP8MOE_ERR_ALIGN;
  return FP8MOE_OK;
}

int check_grouped_mm_blockwise(const void* a, int a_fmt, const void* sa, const void* b, int b_fmt, const void* sb,
                               const int32_t* offs, int32_t n_groups, int64_t M, int64_t N, int64_t K,
                               const void* out, int out_dtype) {
  if (a_fmt < FP8MOE_OPD_E4M3FN || a_fmt > FP8MOE_OPD_BF16 || b_fmt < FP8MOE_OPD_E4M3FN || b_fmt > FP8MOE_OPD_BF16 ||
      (out_dtype != FP8MOE_OUT_BF16 && out_dtype != FP8MOE_OUT_F32))
    return FP8MOE_ERR_ENUM;
  if (a_fmt != FP8MOE_OPD_E4M3FN || b_fmt != FP8MOE_OPD_E4M3FN) return FP8MOE_ERR_UNSUPPORTED;
  if (M < 0 || N < 0 || K < 0 || n_groups < 1 || M > kI32Max || N > kI32Max || K > kI32Max) return FP8MOE_ERR_SHAPE;
  const int64_t KB = (K + 127) / 128, NB = (N + 127) / 128;
  const int64_t grid = mul((M + 127) / 128 + n_groups, NB);
  const int64_t na = mul(M, K), nb = mul(mul(n_groups, N), K), no = mul(M, N);
  if (na < 0 || nb < 0 || no < 0 || grid < 0 || grid > kI32Max || mul(mul(n_groups, NB), KB) < 0) return FP8MOE_ERR_SHAPE;
  const bool work = M > 0 && N > 0;
  if (!offs || (work && (!need(a, na) || !need(b, nb) || !need(sa, mul(M, KB)) || !need(sb, mul(n_groups, NB * KB)) ||
                         !out)))
    return FP8MOE_ERR_NULL;
  if (K % 16 || !aligned(a, 16) || !aligned(b, 16) || !aligned(sa, 4) || !aligned(sb, 4) || !aligned(offs, 4) ||
      !aligned(out, out_dtype == FP8MOE_OUT_BF16 ? 2 : 4))
    return FP8MOE_ERR_ALIGN;
  return FP8MOE_OK;
}

int64_t blockwise_token_blocks_bound(int64_t M, int32_t n_groups) {
  if (M < 0 || n_groups < 1) return -1;
  return (M + 127) / 128 + n_groups;
}

int check_quantize_blockwise_tokens(const void* x, int64_t M, int64_t C, const int32_t* offs, int32_t n_groups,
                                    int codec, const void* q_t, int64_t ld_q, const void* scale) {
  if (codec != FP8MOE_E4M3FN && codec != FP8MOE_E4M3FNUZ) return FP8MOE_ERR_ENUM;
  if (M < 0 || C < 0 || n_groups < 1 || M > kI32Max || C > kI32Max || ld_q < M) return FP8MOE_ERR_SHAPE;
  const int64_t tb = blockwise_token_blocks_bound(M, n_groups);
  const int64_t grid = mul(tb, (C + 63) / 64);
  if (mul(M, C) < 0 || mul(C, ld_q) < 0 || mul(tb, C) < 0 || grid < 0 || grid > kI32Max) return FP8MOE_ERR_SHAPE;
  const bool work = M > 0 && C > 0;
  if (!offs || (work && (!x || !q_t || !scale))) return FP8MOE_ERR_NULL;
  if (C % 8 || ld_q % 16 || !aligned(x, 16) || !aligned(q_t, 16) || !aligned(scale, 4) || !aligned(offs, 4))
    return FP8MOE_ERR_ALIGN;
  return FP8MOE_OK;
}

int check_grouped_mm_blockwise_k(const void* a_t, const void* sa, const void* b_t, const void* sb, const int32_t* offs,
                                 int32_t n_groups, int64_t M, int64_t ld, int64_t N, int64_t K, const void* out,
                                 int out_dtype) {
  if (out_dtype != FP8MOE_OUT_BF16 && out_dtype != FP8MOE_OUT_F32) return FP8MOE_ERR_ENUM;
  if (M < 0 || N < 0 || K < 0 || n_groups < 1 || ld < M || M > kI32Max || N > kI32Max || K > kI32Max)
    return FP8MOE_ERR_SHAPE;
  const int64_t tb = blockwise_token_blocks_bound(M, n_groups);
  const int64_t grid = mul(n_groups, mul((N + 127) / 128, (K + 127) / 128));
  if (mul(N, ld) < 0 || mul(K, ld) < 0 || mul(mul(n_groups, N), K) < 0 || mul(tb, N + K) < 0 || grid < 0 ||
      grid > kI32Max)
    return FP8MOE_ERR_SHAPE;
  const bool work = N > 0 && K > 0;
  if (!offs || (work && (!out || (M > 0 && (!a_t || !b_t || !sa || !sb))))) return FP8MOE_ERR_NULL;
  if (ld % 16 || !aligned(a_t, 16) || !aligned(b_t, 16) || !aligned(sa, 4) || !aligned(sb, 4) || !aligned(offs, 4) ||
      !aligned(out, out_dtype == FP8MOE_OUT_BF16 ? 2 : 4))
    return FP8MOE_ERR_ALIGN;
  return FP8MOE_OK;
}

int check_quantize_tensorwise(const void* x, int64_t batch, int64_t rows, int64_t cols, int codec, const void* q,
                              const void* q_t, int64_t ld_q, const void* scale, int64_t n_scale,
                              const void* workspace) {
  if (codec != FP8MOE_E4M3FN && codec != FP8MOE_E4M3FNUZ) return FP8MOE_ERR_ENUM;
  if (batch < 1 || rows < 0 || cols < 0 || n_scale < 1 || rows > kI32Max || cols > kI32Max) return FP8MOE_ERR_SHAPE;
  const int64_t per = mul(rows, cols), n = mul(batch, per);
  if (per < 0 || n < 0) return FP8MOE_ERR_SHAPE;
  if (q_t != nullptr) {
    if (ld_q < rows) return FP8MOE_ERR_SHAPE;
    const int64_t nt = mul(mul(batch, cols), ld_q);
    const int64_t tiles = mul(batch, mul((rows + 127) / 128, (cols + 63) / 64));
    if (nt < 0 || tiles < 0 || tiles > kI32Max) return FP8MOE_ERR_SHAPE;
  }
  if (!need(x, n) || !scale || !need(workspace, n)) return FP8MOE_ERR_NULL;
  if (cols % 8 || !aligned(x, 16) || !aligned(q, 16) || !aligned(scale, 4) || !aligned(workspace, 4))
    return FP8MOE_ERR_ALIGN;
  if (q_t != nullptr && (ld_q % 16 || !aligned(q_t, 16))) return FP8MOE_ERR_ALIGN;
  return FP8MOE_OK;
}

int64_t route_rows_bound(int64_t slots, int32_t n_experts, int32_t pad) {
  if (slots < 0 || n_experts < 1 || pad < 1) return -1;
  const int64_t r = slots + (int64_t)n_experts * (pad - 1);
  return r > kI32Max ? -1 : r;
}

int64_t route_workspace_bytes(int64_t slots, int32_t n_experts) {
  if (slots < 0 || slots > kI32Max || n_experts < 1) return -1;
  return route_blocks(slots) * n_experts * 4;
}

int check_moe_route(const int32_t* ids, int64_t tokens, int32_t topk, int32_t E, int32_t pad, const int32_t* counts,
                    const int32_t* offs, const int32_t* dest, const int32_t* src, const void* workspace) {
  if (tokens < 0 || topk < 1 || E < 1 || pad < 1) return FP8MOE_ERR_SHAPE;
  const int64_t S = mul(tokens, topk);
  if (S < 0 || S > kI32Max) return FP8MOE_ERR_SHAPE;
  const int64_t rows = route_rows_bound(S, E, pad);
  if (rows < 0) return FP8MOE_ERR_SHAPE;   // grouped rows must fit int32
  if (E > kRouteMaxExperts) return FP8MOE_ERR_UNSUPPORTED;
  if (!need(ids, S) || !counts || !offs || !need(dest, S) || !need(src, rows) || !need(workspace, S))
    return FP8MOE_ERR_NULL;
  if (!aligned(ids, 4) || !aligned(counts, 4) || !aligned(offs, 4) || !aligned(dest, 4) || !aligned(src, 4) ||
      !aligned(workspace, 4))
    return FP8MOE_ERR_ALIGN;
  return FP8MOE_OK;
}

int check_moe_permute(const void* x, int64_t tokens, int64_t cols, int32_t topk, const int32_t* src,
                      int64_t rows_out, const void* xg) {
  if (tokens < 0 || cols < 0 || topk < 1 || rows_out < 0 || rows_out > kI32Max) return FP8MOE_ERR_SHAPE;
  const int64_t S = mul(tokens, topk), nx = mul(tokens, cols), ng = mul(rows_out, cols);
  if (S < 0 || S > kI32Max || nx < 0 || ng < 0) return FP8MOE_ERR_SHAPE;
  if (!need(x, nx) || !need(src, rows_out) || !need(xg, ng)) return FP8MOE_ERR_NULL;
  if (cols % 8 || !aligned(x, 16) || !aligned(xg, 16) || !aligned(src, 4)) return FP8MOE_ERR_ALIGN;
  return FP8MOE_OK;
}

int check_moe_permute_quantized(const void* q, const float* scale, int64_t tokens, int64_t cols, int32_t topk,
                                const int32_t* src, int64_t rows_out, int codec, const void* qg,
                                const float* scale_g) {
  if (codec != FP8MOE_E4M3FN && codec != FP8MOE_E4M3FNUZ) return FP8MOE_ERR_ENUM;
  if (tokens < 0 || cols < 0 || topk < 1 || rows_out < 0 || rows_out > kI32Max) return FP8MOE_ERR_SHAPE;
  const int64_t S = mul(tokens, topk), nq = mul(tokens, cols), ng = mul(rows_out, cols);
  if (S < 0 || S > kI32Max || nq < 0 || ng < 0) return FP8MOE_ERR_SHAPE;
  if (!need(q, nq) || !need(scale, tokens) || !need(src, rows_out) || !need(qg, ng) || !need(scale_g, rows_out))
    return FP8MOE_ERR_NULL;
  if (cols % 16 || !aligned(q, 16) || !aligned(qg, 16) || !aligned(src, 4) || !aligned(scale, 4) ||
      !aligned(scale_g, 4))
    return FP8MOE_ERR_ALIGN;
  return FP8MOE_OK;
}

int check_moe_combine(const void* yg, int64_t rows_in, const int32_t* dest, const float* w, int64_t tokens,
                      int32_t topk, int64_t cols, const void* y) {
  if (tokens < 0 || cols < 0 || topk < 1 || rows_in < 0 || rows_in > kI32Max) return FP8MOE_ERR_SHAPE;
  const int64_t S = mul(tokens, topk), ny = mul(tokens, cols), ng = mul(rows_in, cols);
  if (S < 0 || S > kI32Max || ny < 0 || ng < 0) return FP8MOE_ERR_SHAPE;
  const int64_t work = cols ? S : 0;   // nothing is read when there are no columns
  // w may be null: every weight 1
  if (!need(yg, cols ? ng : 0) || !need(dest, work) || !need(y, ny)) return FP8MOE_ERR_NULL;
  if (cols % 8 || !aligned(yg, 16) || !aligned(y, 16) || !aligned(dest, 4) || !aligned(w, 4)) return FP8MOE_ERR_ALIGN;
  return FP8MOE_OK;
}

int check_moe_permute_rowwise(const void* x, int64_t tokens, int64_t cols, int32_t topk, const int32_t* src,
                              int64_t rows_out, int codec, const void* xg, const void* qg, const float* scale_g) {
  if (codec != FP8MOE_E4M3FN && codec != FP8MOE_E4M3FNUZ) return FP8MOE_ERR_ENUM;
  if (tokens < 0 || cols < 0 || topk < 1 || rows_out < 0 || rows_out > kI32Max * 256LL || cols > kI32Max)
    return FP8MOE_ERR_SHAPE;
  const int64_t S = mul(tokens, topk), nx = mul(tokens, cols), ng = mul(rows_out, cols);
  if (S < 0 || S > kI32Max || nx < 0 || ng < 0) return FP8MOE_ERR_SHAPE;
  if (!need(x, nx) || !need(src, rows_out) || !need(qg, ng) || !need(scale_g, rows_out)) return FP8MOE_ERR_NULL;
  if (xg == nullptr && cols > kRowwiseRegCols && rows_out > 0) return FP8MOE_ERR_NULL;
  if (cols % 8 || !aligned(x, 16) || !aligned(xg, 16) || !aligned(qg, 16) || !aligned(src, 4) ||
      !aligned(scale_g, 4))
    return FP8MOE_ERR_ALIGN;
  return FP8MOE_OK;
}

int check_moe_combine_backward(const void* dy, const void* yg, int64_t rows, const int32_t* dest,
                               const int32_t* src, const float* w, int64_t tokens, int32_t topk, int64_t cols,
                               int codec, const void* dyg, const void* q, const float* scale, const float* dw) {
  if (codec != FP8MOE_E4M3FN && codec != FP8MOE_E4M3FNUZ) return FP8MOE_ERR_ENUM;
  if (tokens < 0 || cols < 0 || topk < 1 || rows < 0 || rows > kI32Max) return FP8MOE_ERR_SHAPE;
  if (cols > kCombineBwdMaxCols) return FP8MOE_ERR_UNSUPPORTED;
  const int64_t S = mul(tokens, topk), ny = mul(tokens, cols), ng = mul(rows, cols);
  if (S < 0 || S > kI32Max || ny < 0 || ng < 0 || tokens > kI32Max - 1024) return FP8MOE_ERR_SHAPE;
  if ((q == nullptr) != (scale == nullptr)) return FP8MOE_ERR_NULL;   // codes and scales come together
  if (!need(dy, ny) || !need(yg, ng) || !need(dest, S) || !need(src, rows) || !need(w, S) || !need(dw, S))
    return FP8MOE_ERR_NULL;
  if (cols % 8 || !aligned(dy, 16) || !aligned(yg, 16) || !aligned(dyg, 16) || !aligned(q, 16) ||
      !aligned(dest, 4) || !aligned(src, 4) || !aligned(w, 4) || !aligned(scale, 4) || !aligned(dw, 4))
    return FP8MOE_ERR_ALIGN;
  return FP8MOE_OK;
}

int check_encode_f32(const void* y, int64_t n, int codec, const void* q) {
  if (codec != FP8MOE_E4M3FN && codec != FP8MOE_E4M3FNUZ) return FP8MOE_ERR_ENUM;
  if (n < 0 || n > kI32Max * 64LL) return FP8MOE_ERR_SHAPE;
  if (!need(y, n) || !need(q, n)) return FP8MOE_ERR_NULL;
  if (!aligned(y, 4)) return FP8MOE_ERR_ALIGN;
  return FP8MOE_OK;
}

}  // namespace fp8moe

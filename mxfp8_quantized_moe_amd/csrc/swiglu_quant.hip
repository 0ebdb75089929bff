// SwiGLU between the two expert GEMMs and its backward, each fused with the
// rowwise FP8 quantization of its output.
// [P1 Details: the MoE layer's grouped GEMMs and their dynamically quantized
// operands, fused quantization kernels; P4 "MoE" (routed experts between two
// grouped GEMMs) and "Три уровня оптимизации Triton-ядер" (quantization fused
// into the kernel that produces the tensor instead of separate launches).]
//
// Forward: H1 [rows][2F] bf16 (gate columns [0, F), up columns [F, 2F)) ->
// A2 = bf16(silu(gate) * up) [rows][F], and its FP8 rowwise form.  Backward:
// dA2 [rows][F] and H1 -> dH1 = [bf16(dA2 up s (1 + g (1 - s))) |
// bf16(dA2 g s)] [rows][2F] with s = sigmoid(gate), and its FP8 rowwise form.
// Elementwise math in fp32; the bf16 result is rounded to nearest even, and
// the FP8 codes are those of the rowwise quantizer applied to that bf16 tensor.
//
// Work layout as in the rowwise quantizer: TPR threads own a row, each holding
// ITEMS 16-byte chunks (8 columns) of the result in registers between the row
// maximum and the cast; rows longer than that take a streaming variant that
// writes the bf16 result first and reads it back for the cast.  HBM sees the
// inputs read once and both outputs written once.
#include "device_common.hpp"
#include "kernels.hpp"
#include "swiglu_common.hpp"

namespace fp8moe {

__device__ __forceinline__ uint32_t sw_absmax4(uint32_t m, const u32x4& v) {
  m = pk_absmax_bf16(m, v.x);
  m = pk_absmax_bf16(m, v.y);
  m = pk_absmax_bf16(m, v.z);
  return pk_absmax_bf16(m, v.w);
}

template <int CODEC>
__device__ __forceinline__ u32x2 sw_quant_chunk(const u32x4& v, float s) {
  return u32x2{quant_bf16x4<CODEC>(v.x, v.y, s), quant_bf16x4<CODEC>(v.z, v.w, s)};
}

template <int TPR>
__device__ __forceinline__ uint32_t sw_row_max(uint32_t m, uint32_t* red) {
  if constexpr (TPR <= 64) {
#pragma unroll
    for (int off = TPR / 2; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
    return m;
  } else {
    static_assert(TPR == 256, "row group is one workgroup");
    m = wave_max_u32(m);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = m;
    __syncthreads();
    m = max(max(red[0], red[1]), max(red[2], red[3]));
    return m;
  }
}

// Forward.  F columns per output row (nc = F / 8 chunks).
template <int CODEC, int TPR, int ITEMS>
__global__ __launch_bounds__(256) void swiglu_fwd_kernel(const uint16_t* __restrict__ h1, int64_t rows, int64_t F,
                                                         int64_t ld_h1, uint16_t* __restrict__ a2,
                                                         uint8_t* __restrict__ q, float* __restrict__ scale) {
  constexpr int RPB = 256 / TPR;
  __shared__ uint32_t red[4];
  const int lt = threadIdx.x % TPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const bool valid = row < rows;
  const int64_t nc = F >> 3;
  const int64_t rr = valid ? row : 0;
  const u32x4* __restrict__ gr = reinterpret_cast<const u32x4*>(h1 + rr * ld_h1);
  const u32x4* __restrict__ ur = reinterpret_cast<const u32x4*>(h1 + rr * ld_h1 + F);
  u32x4* __restrict__ ar = reinterpret_cast<u32x4*>(a2 + rr * F);
  u32x2* __restrict__ qr = reinterpret_cast<u32x2*>(q != nullptr ? q + rr * F : nullptr);
  uint32_t m = 0;
  if constexpr (ITEMS > 0) {
    u32x4 av[ITEMS];
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int64_t c = (int64_t)i * TPR + lt;
      av[i] = u32x4{0, 0, 0, 0};
      if (valid && c < nc) {
        av[i] = sw_fwd_chunk(gr[c], ur[c]);
        ar[c] = av[i];
      }
      m = sw_absmax4(m, av[i]);
    }
    if (q == nullptr) return;   // bf16 output only (uniform over the launch)
    m = sw_row_max<TPR>(pk_fold(m), red);
    const float s = scale_from_amax(__uint_as_float(m << 16), CODEC);
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int64_t c = (int64_t)i * TPR + lt;
      if (valid && c < nc) qr[c] = sw_quant_chunk<CODEC>(av[i], s);
    }
    if (valid && lt == 0) scale[row] = s;
  } else {
    if (valid) {
      for (int64_t c = lt; c < nc; c += TPR) {
        const u32x4 a = sw_fwd_chunk(gr[c], ur[c]);
        ar[c] = a;
        m = sw_absmax4(m, a);
      }
    }
    if (q == nullptr) return;
    m = sw_row_max<TPR>(pk_fold(m), red);
    const float s = scale_from_amax(__uint_as_float(m << 16), CODEC);
    if (valid) {
      // each thread reads back only the chunks it wrote itself
      for (int64_t c = lt; c < nc; c += TPR) qr[c] = sw_quant_chunk<CODEC>(ar[c], s);
      if (lt == 0) scale[row] = s;
    }
  }
}

// Backward.  Output rows of 2F columns: gate part at chunk c, up part at nc + c.
template <int CODEC, int TPR, int ITEMS>
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const uint16_t* __restrict__ da2,
                                                         const uint16_t* __restrict__ h1, int64_t rows, int64_t F,
                                                         int64_t ld_h1, uint16_t* __restrict__ dh1,
                                                         uint8_t* __restrict__ q, float* __restrict__ scale) {
  constexpr int RPB = 256 / TPR;
  __shared__ uint32_t red[4];
  const int lt = threadIdx.x % TPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const bool valid = row < rows;
  const int64_t nc = F >> 3;
  const int64_t rr = valid ? row : 0;
  const u32x4* __restrict__ dr = reinterpret_cast<const u32x4*>(da2 + rr * F);
  const u32x4* __restrict__ gr = reinterpret_cast<const u32x4*>(h1 + rr * ld_h1);
  const u32x4* __restrict__ ur = reinterpret_cast<const u32x4*>(h1 + rr * ld_h1 + F);
  u32x4* __restrict__ orow = reinterpret_cast<u32x4*>(dh1 + rr * 2 * F);
  u32x2* __restrict__ qr = reinterpret_cast<u32x2*>(q != nullptr ? q + rr * 2 * F : nullptr);
  uint32_t m = 0;
  if constexpr (ITEMS > 0) {
    u32x4 gv[ITEMS], uv[ITEMS];
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int64_t c = (int64_t)i * TPR + lt;
      gv[i] = uv[i] = u32x4{0, 0, 0, 0};
      if (valid && c < nc) {
        sw_bwd_chunk(dr[c], gr[c], ur[c], gv[i], uv[i]);
        orow[c] = gv[i];
        orow[nc + c] = uv[i];
      }
      m = sw_absmax4(sw_absmax4(m, gv[i]), uv[i]);
    }
    if (q == nullptr) return;   // bf16 output only (uniform over the launch)
    m = sw_row_max<TPR>(pk_fold(m), red);
    const float s = scale_from_amax(__uint_as_float(m << 16), CODEC);
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int64_t c = (int64_t)i * TPR + lt;
      if (valid && c < nc) {
        qr[c] = sw_quant_chunk<CODEC>(gv[i], s);
        qr[nc + c] = sw_quant_chunk<CODEC>(uv[i], s);
      }
    }
    if (valid && lt == 0) scale[row] = s;
  } else {
    if (valid) {
      for (int64_t c = lt; c < nc; c += TPR) {
        u32x4 a, b;
        sw_bwd_chunk(dr[c], gr[c], ur[c], a, b);
        orow[c] = a;
        orow[nc + c] = b;
        m = sw_absmax4(sw_absmax4(m, a), b);
      }
    }
    if (q == nullptr) return;
    m = sw_row_max<TPR>(pk_fold(m), red);
    const float s = scale_from_amax(__uint_as_float(m << 16), CODEC);
    if (valid) {
      for (int64_t c = lt; c < nc; c += TPR) {
        qr[c] = sw_quant_chunk<CODEC>(orow[c], s);
        qr[nc + c] = sw_quant_chunk<CODEC>(orow[nc + c], s);
      }
      if (lt == 0) scale[row] = s;
    }
  }
}

// Threads per row and chunks per thread from the chunk count, as the rowwise quantizer picks them.
template <typename L>
static hipError_t sw_pick(int64_t nc, L&& launch) {
  auto items = [&](auto tpr_tag) -> hipError_t {
    constexpr int TPR = decltype(tpr_tag)::value;
    const int64_t it = (nc + TPR - 1) / TPR;
    if (it <= 1) return launch(tpr_tag, std::integral_constant<int, 1>{});
    if (it <= 2) return launch(tpr_tag, std::integral_constant<int, 2>{});
    if (it <= 4) return launch(tpr_tag, std::integral_constant<int, 4>{});
    if (it <= 8) return launch(tpr_tag, std::integral_constant<int, 8>{});
    return launch(tpr_tag, std::integral_constant<int, 0>{});
  };
  if (nc <= 64) return items(std::integral_constant<int, 16>{});
  if (nc <= 512) return items(std::integral_constant<int, 64>{});
  return items(std::integral_constant<int, 256>{});
}

template <int CODEC>
static hipError_t sw_fwd(const uint16_t* h1, int64_t rows, int64_t F, int64_t ld_h1, uint16_t* a2, uint8_t* q,
                         float* scale, hipStream_t st) {
  return sw_pick(F >> 3, [&](auto tpr_tag, auto items_tag) -> hipError_t {
    constexpr int TPR = decltype(tpr_tag)::value, ITEMS = decltype(items_tag)::value;
    const int64_t blocks = (rows + 256 / TPR - 1) / (256 / TPR);
    hipLaunchKernelGGL((swiglu_fwd_kernel<CODEC, TPR, ITEMS>), dim3((unsigned)blocks), dim3(256), 0, st, h1, rows,
                       F, ld_h1, a2, q, scale);
    return hipGetLastError();
  });
}

template <int CODEC>
static hipError_t sw_bwd(const uint16_t* da2, const uint16_t* h1, int64_t rows, int64_t F, int64_t ld_h1,
                         uint16_t* dh1, uint8_t* q, float* scale, hipStream_t st) {
  // twice the registers per chunk of the forward: chunks per thread capped one step lower
  return sw_pick((F >> 3) * 2, [&](auto tpr_tag, auto items_tag) -> hipError_t {
    constexpr int TPR = decltype(tpr_tag)::value;
    constexpr int IT2 = decltype(items_tag)::value;
    constexpr int ITEMS = IT2 == 0 ? 0 : (IT2 + 1) / 2;
    const int64_t nc = F >> 3;
    if (ITEMS > 0 && (int64_t)ITEMS * TPR < nc) return hipErrorInvalidValue;   // (cannot happen: IT2 * TPR >= 2 nc)
    const int64_t blocks = (rows + 256 / TPR - 1) / (256 / TPR);
    hipLaunchKernelGGL((swiglu_bwd_kernel<CODEC, TPR, ITEMS>), dim3((unsigned)blocks), dim3(256), 0, st, da2, h1,
                       rows, F, ld_h1, dh1, q, scale);
    return hipGetLastError();
  });
}

hipError_t launch_swiglu_quantize_rowwise(const uint16_t* h1, int64_t rows, int64_t F, int64_t ld_h1, int codec,
                                          uint16_t* a2, uint8_t* q, float* scale, hipStream_t st) {
  if (rows == 0 || F == 0) return hipSuccess;
  return codec == 0 ? sw_fwd<0>(h1, rows, F, ld_h1, a2, q, scale, st)
                    : sw_fwd<1>(h1, rows, F, ld_h1, a2, q, scale, st);
}

hipError_t launch_swiglu_backward_quantize_rowwise(const uint16_t* da2, const uint16_t* h1, int64_t rows, int64_t F,
                                                   int64_t ld_h1, int codec, uint16_t* dh1, uint8_t* q, float* scale,
                                                   hipStream_t st) {
  if (rows == 0 || F == 0) return hipSuccess;
  return codec == 0 ? sw_bwd<0>(da2, h1, rows, F, ld_h1, dh1, q, scale, st)
                    : sw_bwd<1>(da2, h1, rows, F, ld_h1, dh1, q, scale, st);
}

}  // namespace fp8moe

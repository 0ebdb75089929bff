// Rowwise dynamic FP8 quantization: one fp32 scale per row over the last dim,
// in one fused pass (absolute max -> scale -> multiply -> clamp -> encode).
// [P4 "Три уровня оптимизации Triton-ядер": a single kernel replaces the chain
// of separate absmax/scale/clip/cast launches; expert weights are quantized by
// one launch parallel over experts and output-dimension blocks, which here is
// the [E*N, K] row view.  P1 Details: fused quantization, rowwise recipe.]
//
// Work layout: TPR threads own one row (TPR = 16, 64 or 256); each thread
// loads ITEMS 16-byte chunks (8 bf16) at stride TPR chunks, so a wave's loads
// are contiguous.  The row stays in registers between the max and the cast:
// HBM sees 2 bytes read + 1 byte written per element.  Rows longer than
// TPR*ITEMS*8 take the streaming variant (ITEMS == 0), which reads the row a
// second time for the cast.
#include "device_common.hpp"
#include "kernels.hpp"

namespace fp8moe {

template <int TPR>
__device__ __forceinline__ uint32_t row_group_max(uint32_t m, uint32_t* red) {
  if constexpr (TPR <= 64) {
    return group_max_u32<TPR>(m);
  } else {
    static_assert(TPR == 256, "row group is one workgroup");
    m = group_max_u32<64>(m);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = m;
    __syncthreads();
    m = max(max(red[0], red[1]), max(red[2], red[3]));
    return m;
  }
}

template <int CODEC>
__device__ __forceinline__ u32x2 quant_chunk(const u32x4& v, float s) {
  return u32x2{quant_bf16x4<CODEC>(v.x, v.y, s), quant_bf16x4<CODEC>(v.z, v.w, s)};
}

template <int CODEC, int TPR, int ITEMS>
__global__ __launch_bounds__(256) void rowwise_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                      int64_t cols, int64_t ld_x,
                                                      uint8_t* __restrict__ q,
                                                      float* __restrict__ scale) {
  constexpr int RPB = 256 / TPR;
  __shared__ uint32_t red[4];
  const int lt = threadIdx.x % TPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const bool valid = row < rows;
  const int64_t nchunk = cols >> 3;
  const u32x4* __restrict__ xr = reinterpret_cast<const u32x4*>(x + (valid ? row : 0) * ld_x);
  u32x2* __restrict__ qr = reinterpret_cast<u32x2*>(q + (valid ? row : 0) * cols);

  if constexpr (ITEMS > 0) {
    u32x4 v[ITEMS];
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int64_t c = (int64_t)i * TPR + lt;
      if (valid && c < nchunk) {
        v[i] = xr[c];
      } else {
        v[i] = u32x4{0, 0, 0, 0};
      }
      m = pk_absmax_bf16(m, v[i].x);
      m = pk_absmax_bf16(m, v[i].y);
      m = pk_absmax_bf16(m, v[i].z);
      m = pk_absmax_bf16(m, v[i].w);
    }
    m = row_group_max<TPR>(pk_fold(m), red);
    const float s = scale_from_amax(__uint_as_float(m << 16), CODEC);
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int64_t c = (int64_t)i * TPR + lt;
      if (valid && c < nchunk) qr[c] = quant_chunk<CODEC>(v[i], s);
    }
    if (valid && lt == 0) scale[row] = s;
  } else {
    uint32_t m = 0;
    for (int64_t c = lt; c < nchunk; c += TPR) {
      const u32x4 v = valid ? xr[c] : u32x4{0, 0, 0, 0};
      m = pk_absmax_bf16(m, v.x);
      m = pk_absmax_bf16(m, v.y);
      m = pk_absmax_bf16(m, v.z);
      m = pk_absmax_bf16(m, v.w);
    }
    m = row_group_max<TPR>(pk_fold(m), red);
    const float s = scale_from_amax(__uint_as_float(m << 16), CODEC);
    if (valid) {
      for (int64_t c = lt; c < nchunk; c += TPR) qr[c] = quant_chunk<CODEC>(xr[c], s);
      if (lt == 0) scale[row] = s;
    }
  }
}

template <int CODEC, int TPR, int ITEMS>
static hipError_t launch_rw(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q,
                            float* scale, hipStream_t st) {
  constexpr int RPB = 256 / TPR;
  const int64_t blocks = (rows + RPB - 1) / RPB;
  hipLaunchKernelGGL((rowwise_kernel<CODEC, TPR, ITEMS>), dim3((unsigned)blocks), dim3(256), 0, st, x,
                     rows, cols, ld_x, q, scale);
  return hipGetLastError();
}

template <int CODEC>
static hipError_t dispatch_rw(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q,
                              float* scale, hipStream_t st) {
  const int64_t nchunk = cols >> 3;
  auto pick = [&](auto tpr_tag) -> hipError_t {
    constexpr int TPR = decltype(tpr_tag)::value;
    const int64_t items = (nchunk + TPR - 1) / TPR;
    if (items <= 1) return launch_rw<CODEC, TPR, 1>(x, rows, cols, ld_x, q, scale, st);
    if (items <= 2) return launch_rw<CODEC, TPR, 2>(x, rows, cols, ld_x, q, scale, st);
    if (items <= 4) return launch_rw<CODEC, TPR, 4>(x, rows, cols, ld_x, q, scale, st);
    if (items <= 8) return launch_rw<CODEC, TPR, 8>(x, rows, cols, ld_x, q, scale, st);
    return launch_rw<CODEC, TPR, 0>(x, rows, cols, ld_x, q, scale, st);
  };
  if (nchunk <= 64) return pick(std::integral_constant<int, 16>{});
  if (nchunk <= 512) return pick(std::integral_constant<int, 64>{});
  return pick(std::integral_constant<int, 256>{});
}

hipError_t launch_quantize_rowwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int codec,
                                   uint8_t* q, float* scale, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  return codec == 0 ? dispatch_rw<0>(x, rows, cols, ld_x, q, scale, st)
                    : dispatch_rw<1>(x, rows, cols, ld_x, q, scale, st);
}

}  // namespace fp8moe

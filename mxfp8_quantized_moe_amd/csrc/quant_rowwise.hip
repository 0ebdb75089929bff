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
//
// The gather form (GATHER) quantizes rows gathered into the MoE grouped
// layout: output row r reads token src[r] / topk (a zero row where src[r]
// names no slot), optionally writes the gathered bf16 row too, and quantizes
// it in the same pass [P1 Details, MoE paragraph: the routed rows quantized
// by a fused kernel ahead of the grouped GEMM].  The streaming variant reads
// the gathered row back for the cast, so it needs that bf16 copy.
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

// Row gather of the grouped layout (unused without GATHER).
struct RowGather {
  const int32_t* src;   // [rows] slot of each output row
  int topk;
  int64_t slots;        // tokens * topk
  uint16_t* xg;         // [rows][cols] gathered bf16 copy, or null
};

template <int CODEC, int TPR, int ITEMS, bool GATHER>
__global__ __launch_bounds__(256) void rowwise_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                      int64_t cols, int64_t ld_x,
                                                      uint8_t* __restrict__ q,
                                                      float* __restrict__ scale, RowGather gt) {
  constexpr int RPB = 256 / TPR;
  __shared__ uint32_t red[4];
  const int lt = threadIdx.x % TPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const bool valid = row < rows;
  const int64_t nchunk = cols >> 3;
  int64_t in_row = valid ? row : 0;
  bool has = valid;   // the row has input (a gathered padding row is zeros)
  if constexpr (GATHER) {
    const int sl = valid ? gt.src[row] : -1;
    has = sl >= 0 && (int64_t)sl < gt.slots;
    in_row = has ? sl / gt.topk : 0;
  }
  const u32x4* __restrict__ xr = reinterpret_cast<const u32x4*>(x + in_row * ld_x);
  u32x2* __restrict__ qr = reinterpret_cast<u32x2*>(q + (valid ? row : 0) * cols);
  u32x4* __restrict__ gr = nullptr;
  if constexpr (GATHER) {
    if (gt.xg != nullptr) gr = reinterpret_cast<u32x4*>(gt.xg + (valid ? row : 0) * cols);
  }

  if constexpr (ITEMS > 0) {
    u32x4 v[ITEMS];
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int64_t c = (int64_t)i * TPR + lt;
      if (has && c < nchunk) {
        v[i] = xr[c];
      } else {
        v[i] = u32x4{0, 0, 0, 0};
      }
      if constexpr (GATHER) {
        if (gr != nullptr && valid && c < nchunk) gr[c] = v[i];
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
      const u32x4 v = has ? xr[c] : u32x4{0, 0, 0, 0};
      if constexpr (GATHER) {
        if (valid) gr[c] = v;   // the launcher requires the copy here
      }
      m = pk_absmax_bf16(m, v.x);
      m = pk_absmax_bf16(m, v.y);
      m = pk_absmax_bf16(m, v.z);
      m = pk_absmax_bf16(m, v.w);
    }
    m = row_group_max<TPR>(pk_fold(m), red);
    const float s = scale_from_amax(__uint_as_float(m << 16), CODEC);
    if (valid) {
      // the gathered form reads back the chunks this thread wrote itself
      const u32x4* __restrict__ rd = GATHER ? gr : xr;
      for (int64_t c = lt; c < nchunk; c += TPR) qr[c] = quant_chunk<CODEC>(rd[c], s);
      if (lt == 0) scale[row] = s;
    }
  }
}

template <int CODEC, int TPR, int ITEMS, bool GATHER>
static hipError_t launch_rw(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q,
                            float* scale, const RowGather& gt, hipStream_t st) {
  constexpr int RPB = 256 / TPR;
  const int64_t blocks = (rows + RPB - 1) / RPB;
  hipLaunchKernelGGL((rowwise_kernel<CODEC, TPR, ITEMS, GATHER>), dim3((unsigned)blocks), dim3(256), 0, st, x,
                     rows, cols, ld_x, q, scale, gt);
  return hipGetLastError();
}

template <int CODEC, bool GATHER>
static hipError_t dispatch_rw(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q,
                              float* scale, const RowGather& gt, hipStream_t st) {
  const int64_t nchunk = cols >> 3;
  auto pick = [&](auto tpr_tag) -> hipError_t {
    constexpr int TPR = decltype(tpr_tag)::value;
    const int64_t items = (nchunk + TPR - 1) / TPR;
    if (items <= 1) return launch_rw<CODEC, TPR, 1, GATHER>(x, rows, cols, ld_x, q, scale, gt, st);
    if (items <= 2) return launch_rw<CODEC, TPR, 2, GATHER>(x, rows, cols, ld_x, q, scale, gt, st);
    if (items <= 4) return launch_rw<CODEC, TPR, 4, GATHER>(x, rows, cols, ld_x, q, scale, gt, st);
    if (items <= 8) return launch_rw<CODEC, TPR, 8, GATHER>(x, rows, cols, ld_x, q, scale, gt, st);
    // the streaming cast re-reads the gathered copy (rows over kRowwiseRegCols columns; the ABI checks it)
    if (GATHER && gt.xg == nullptr) return hipErrorInvalidValue;
    return launch_rw<CODEC, TPR, 0, GATHER>(x, rows, cols, ld_x, q, scale, gt, st);
  };
  if (nchunk <= 64) return pick(std::integral_constant<int, 16>{});
  if (nchunk <= 512) return pick(std::integral_constant<int, 64>{});
  return pick(std::integral_constant<int, 256>{});
}

hipError_t launch_quantize_rowwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int codec,
                                   uint8_t* q, float* scale, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const RowGather none{nullptr, 1, 0, nullptr};
  return codec == 0 ? dispatch_rw<0, false>(x, rows, cols, ld_x, q, scale, none, st)
                    : dispatch_rw<1, false>(x, rows, cols, ld_x, q, scale, none, st);
}

hipError_t launch_moe_permute_rowwise(const uint16_t* x, int64_t tokens, int64_t cols, int topk, const int32_t* src,
                                      int64_t rows_out, int codec, uint16_t* xg, uint8_t* qg, float* scale_g,
                                      hipStream_t st) {
  if (rows_out == 0) return hipSuccess;
  const RowGather gt{src, topk, tokens * topk, xg};
  return codec == 0 ? dispatch_rw<0, true>(x, rows_out, cols, cols, qg, scale_g, gt, st)
                    : dispatch_rw<1, true>(x, rows_out, cols, cols, qg, scale_g, gt, st);
}

}  // namespace fp8moe

// Tensorwise FP8 quantization: one scale for the whole tensor, the coarsest
// of the scaling granularities.  [P4 "Скейлы: от тензора до микроблока" (one
// scale per tensor); P4 FAQ (tensorwise faster and coarser than rowwise); P3,
// the four scaling strategies.]
//
// The scale and cast follow the rowwise recipe with every element as the one
// reduction set: s = fmax / max(amax, 1e-12f), y = clamp(fp32(x * s)), encode.
// The grouped GEMM takes s as its fp32 per-row / per-column scales, every
// entry equal (the call broadcasts s into a vector of the caller's length).
//
// Launches: partial |x| maxima (one per block, grid-strided over 16-byte
// chunks) into the caller's workspace; then the row-major cast (or, with a
// transposed copy asked for, only the broadcast of s) and the transposed cast,
// which writes the row-major codes from the same tile; each block folds the
// partials into s itself.
#include "device_common.hpp"
#include "kernels.hpp"
#include "validate.hpp"

namespace fp8moe {

namespace {

constexpr int kTwRows = 128;   // transposed tile: rows (output bytes per column segment)
constexpr int kTwCols = 64;    // transposed tile: columns

__device__ __forceinline__ uint32_t chunk_absmax(uint32_t m, const u32x4& v) {
  m = pk_absmax_bf16(m, v.x);
  m = pk_absmax_bf16(m, v.y);
  m = pk_absmax_bf16(m, v.z);
  return pk_absmax_bf16(m, v.w);
}

// Max over the 256 threads of a workgroup, returned to every thread.
__device__ __forceinline__ uint32_t block_max_u32(uint32_t m, uint32_t* red) {
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = max(max(red[0], red[1]), max(red[2], red[3]));
  __syncthreads();
  return m;
}

// The tensor's scale from the np partial maxima (bf16 |x| bit patterns).
__device__ __forceinline__ float tw_scale(const uint32_t* __restrict__ part, int np, int codec, uint32_t* red) {
  uint32_t m = 0;
  for (int i = threadIdx.x; i < np; i += 256) m = max(m, part[i]);
  m = block_max_u32(m, red);
  return scale_from_amax(__uint_as_float(m << 16), codec);
}

}  // namespace

__global__ __launch_bounds__(256) void tw_amax_kernel(const u32x4* __restrict__ x, int64_t nchunk,
                                                      uint32_t* __restrict__ part) {
  __shared__ uint32_t red[4];
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t m0 = 0, m1 = 0;
  for (; i + 3 * stride < nchunk; i += 4 * stride) {   // four loads in flight
    const u32x4 a = x[i], b = x[i + stride], c = x[i + 2 * stride], d = x[i + 3 * stride];
    m0 = chunk_absmax(chunk_absmax(m0, a), b);
    m1 = chunk_absmax(chunk_absmax(m1, c), d);
  }
  for (; i < nchunk; i += stride) m0 = chunk_absmax(m0, x[i]);
  const uint32_t m = block_max_u32(max(pk_fold(m0), pk_fold(m1)), red);
  if (threadIdx.x == 0) part[blockIdx.x] = m;
}

// Row-major cast (when q is given) and the broadcast of s into scale[0, n_scale).
template <int CODEC>
__global__ __launch_bounds__(256) void tw_cast_kernel(const u32x4* __restrict__ x, int64_t nchunk,
                                                      const uint32_t* __restrict__ part, int np,
                                                      u32x2* __restrict__ q, float* __restrict__ scale,
                                                      int64_t n_scale) {
  __shared__ uint32_t red[4];
  const float s = tw_scale(part, np, CODEC, red);
  const int64_t stride = (int64_t)gridDim.x * 256;
  const int64_t t0 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q != nullptr) {
    int64_t i = t0;
    for (; i + stride < nchunk; i += 2 * stride) {
      const u32x4 a = x[i], b = x[i + stride];
      q[i] = u32x2{quant_bf16x4<CODEC>(a.x, a.y, s), quant_bf16x4<CODEC>(a.z, a.w, s)};
      q[i + stride] = u32x2{quant_bf16x4<CODEC>(b.x, b.y, s), quant_bf16x4<CODEC>(b.z, b.w, s)};
    }
    for (; i < nchunk; i += stride) {
      const u32x4 a = x[i];
      q[i] = u32x2{quant_bf16x4<CODEC>(a.x, a.y, s), quant_bf16x4<CODEC>(a.z, a.w, s)};
    }
  }
  for (int64_t i = t0; i < n_scale; i += stride) scale[i] = s;
}

// Transposed cast: tile of 128 rows x 64 columns of batch item b; thread
// (rq, cc) casts rows 4rq..4rq+3 x columns 8cc..8cc+7, stores them row-major
// when q is given (one read of x serves both layouts), and writes, per column,
// the four codes as one word of the [column][row] LDS tile; then each thread
// stores two 16-row segments of output rows (columns).
template <int CODEC>
__global__ __launch_bounds__(256) void tw_cast_t_kernel(const uint16_t* __restrict__ x, int rows, int cols,
                                                        const uint32_t* __restrict__ part, int np,
                                                        uint8_t* __restrict__ q, uint8_t* __restrict__ q_t,
                                                        int64_t ld_q, int tiles_r, int tiles_c) {
  __shared__ uint32_t red[4];
  __shared__ uint32_t T[kTwCols][kTwRows / 4 + 2];   // [column][row/4], rows padded by 8 bytes
  const float s = tw_scale(part, np, CODEC, red);
  const int tile = blockIdx.x;
  const int64_t b = tile / (tiles_r * tiles_c);
  const int tr = (tile / tiles_c) % tiles_r, tc = tile % tiles_c;
  const int r0 = tr * kTwRows, c0 = tc * kTwCols;
  const int t = threadIdx.x, cc = t & 7, rq = t >> 3;
  const uint16_t* __restrict__ xb = x + b * rows * (int64_t)cols;
  uint32_t lo[4], hi[4];   // codes of columns 8cc..8cc+3 / 8cc+4..8cc+7, one word per row
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = r0 + 4 * rq + i, c = c0 + 8 * cc;
    const bool in = r < rows && c < cols;
    u32x4 v = u32x4{0, 0, 0, 0};
    if (in) v = *reinterpret_cast<const u32x4*>(xb + (int64_t)r * cols + c);
    lo[i] = quant_bf16x4<CODEC>(v.x, v.y, s);
    hi[i] = quant_bf16x4<CODEC>(v.z, v.w, s);
    if (q != nullptr && in) *reinterpret_cast<u32x2*>(q + (b * rows + r) * (int64_t)cols + c) = u32x2{lo[i], hi[i]};
  }
  // column j's bytes over the four rows -> one word (row 4rq in the low byte)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int sh = 8 * j;
    T[8 * cc + j][rq] = ((lo[0] >> sh) & 0xFFu) | (((lo[1] >> sh) & 0xFFu) << 8) | (((lo[2] >> sh) & 0xFFu) << 16) |
                        (((lo[3] >> sh) & 0xFFu) << 24);
    T[8 * cc + 4 + j][rq] = ((hi[0] >> sh) & 0xFFu) | (((hi[1] >> sh) & 0xFFu) << 8) |
                            (((hi[2] >> sh) & 0xFFu) << 16) | (((hi[3] >> sh) & 0xFFu) << 24);
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int seg = t + 256 * k, col = seg >> 3, rc = seg & 7;
    const int c = c0 + col, r = r0 + 16 * rc;
    if (c >= cols || r >= rows) continue;
    const uint32_t* w = &T[col][4 * rc];
    uint8_t* dst = q_t + (b * cols + c) * ld_q + r;
    if (rows - r >= 16) {
      *reinterpret_cast<u32x4*>(dst) = u32x4{w[0], w[1], w[2], w[3]};
    } else {
      for (int e = 0; e < rows - r; ++e) dst[e] = (uint8_t)(w[e >> 2] >> (8 * (e & 3)));
    }
  }
}

hipError_t launch_quantize_tensorwise(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, int codec,
                                      uint8_t* q, uint8_t* q_t, int64_t ld_q, float* scale, int64_t n_scale,
                                      uint32_t* part, hipStream_t st) {
  const int64_t nchunk = batch * rows * cols / 8;
  // partials: about four chunks per thread, at most kTwPartials blocks
  const int np = (int)std::min<int64_t>(kTwPartials, (nchunk + 1023) / 1024);
  if (np > 0)
    hipLaunchKernelGGL(tw_amax_kernel, dim3((unsigned)np), dim3(256), 0, st, reinterpret_cast<const u32x4*>(x),
                       nchunk, part);
  // with q_t, the transposed kernel also writes q; the plain cast then only broadcasts s
  const bool fused = q_t != nullptr && rows > 0 && cols > 0;
  uint8_t* q_rm = fused ? nullptr : q;
  const int64_t work = std::max<int64_t>(q_rm ? nchunk : 0, n_scale);
  const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>(4096, (work + 511) / 512));
  if (codec == 0)
    hipLaunchKernelGGL(tw_cast_kernel<0>, dim3(grid), dim3(256), 0, st, reinterpret_cast<const u32x4*>(x), nchunk,
                       part, np, reinterpret_cast<u32x2*>(q_rm), scale, n_scale);
  else
    hipLaunchKernelGGL(tw_cast_kernel<1>, dim3(grid), dim3(256), 0, st, reinterpret_cast<const u32x4*>(x), nchunk,
                       part, np, reinterpret_cast<u32x2*>(q_rm), scale, n_scale);
  if (fused) {
    const int tiles_r = (int)((rows + kTwRows - 1) / kTwRows), tiles_c = (int)((cols + kTwCols - 1) / kTwCols);
    const int64_t tiles = batch * tiles_r * tiles_c;
    if (codec == 0)
      hipLaunchKernelGGL(tw_cast_t_kernel<0>, dim3((unsigned)tiles), dim3(256), 0, st, x, (int)rows, (int)cols, part,
                         np, q, q_t, ld_q, tiles_r, tiles_c);
    else
      hipLaunchKernelGGL(tw_cast_t_kernel<1>, dim3((unsigned)tiles), dim3(256), 0, st, x, (int)rows, (int)cols, part,
                         np, q, q_t, ld_q, tiles_r, tiles_c);
  }
  return hipGetLastError();
}

}  // namespace fp8moe

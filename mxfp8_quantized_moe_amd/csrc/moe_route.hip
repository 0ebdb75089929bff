// MoE routing around the grouped GEMMs: token slots grouped by expert into
// (optionally padded) offsets with a stable destination row per slot, rows
// gathered into that grouped layout, and expert outputs combined per token.
// [P1 Details (the grouped GEMM over an offsets tensor); P4 "MoE" (tokens
// routed to experts, grouped GEMMs over the routed rows); P2 Details (groups
// padded to the MX block size).]
//
// Slot i = t * topk + j is token t's j-th expert choice; within an expert the
// slots keep their order; each group may be padded to a multiple of `pad`
// rows (zeros); an id outside [0, E) drops its slot (destination -1).
// The combine sums the topk weighted rows of a token in slot order, each
// product and sum one fp32 operation rounded to nearest, then rounds to bf16.
//
// route: three launches on the caller's workspace (one int per block of
// kRouteSlots slots and expert): per-block expert histograms (LDS atomics);
// one workgroup turns them into running counts over blocks (the rows of each
// expert in earlier blocks), the counts, the padded inclusive scan over
// experts (offs), and sets every source entry to -1; one wave per block then
// ranks its slots stably (lanes by shuffles, earlier passes by a per-expert
// running count in LDS) and writes destinations and sources, a slot's row
// being its group's start + the earlier blocks' rows + its rank in the block.
#include "device_common.hpp"
#include "kernels.hpp"
#include "validate.hpp"

namespace fp8moe {

static_assert(kRouteSlots % 64 == 0, "the rank kernel walks a block in whole waves");

__global__ __launch_bounds__(256) void route_hist_kernel(const int32_t* __restrict__ ids, int64_t S, int E,
                                                         int32_t* __restrict__ hist) {
  __shared__ int h[kRouteMaxExperts];
  const int t = threadIdx.x;
  for (int e = t; e < E; e += 256) h[e] = 0;
  __syncthreads();
  const int64_t s0 = (int64_t)blockIdx.x * kRouteSlots;
  for (int i = t; i < kRouteSlots; i += 256) {
    const int64_t s = s0 + i;
    if (s < S) {
      const int e = ids[s];
      if (e >= 0 && e < E) atomicAdd(&h[e], 1);
    }
  }
  __syncthreads();
  for (int e = t; e < E; e += 256) hist[(int64_t)blockIdx.x * E + e] = h[e];
}

__global__ __launch_bounds__(1024) void route_scan_kernel(int32_t* __restrict__ hist, int nb, int E, int pad,
                                                          int32_t* __restrict__ counts, int32_t* __restrict__ offs,
                                                          int32_t* __restrict__ src, int64_t rows_bound) {
  __shared__ int sc[kRouteMaxExperts];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    int b = 0;
    for (; b + 4 <= nb; b += 4) {   // four independent loads in flight
      int c[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) c[u] = hist[(int64_t)(b + u) * E + e];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        hist[(int64_t)(b + u) * E + e] = run;   // rows of e in blocks before b + u
        run += c[u];
      }
    }
    for (; b < nb; ++b) {
      const int c = hist[(int64_t)b * E + e];
      hist[(int64_t)b * E + e] = run;
      run += c;
    }
  }
  const int padded = e < E ? (run + pad - 1) / pad * pad : 0;
  sc[e] = padded;
  __syncthreads();
  for (int off = 1; off < kRouteMaxExperts; off <<= 1) {   // inclusive scan over experts
    const int v = e >= off ? sc[e - off] : 0;
    __syncthreads();
    sc[e] += v;
    __syncthreads();
  }
  if (e < E) {
    counts[e] = run;
    offs[e] = sc[e];
  }
  for (int64_t r = e; r < rows_bound; r += kRouteMaxExperts) src[r] = -1;
}

// One wave per block of kRouteSlots slots.
__global__ __launch_bounds__(64) void route_rank_kernel(const int32_t* __restrict__ ids, int64_t S, int E, int pad,
                                                        const int32_t* __restrict__ base,
                                                        const int32_t* __restrict__ counts,
                                                        const int32_t* __restrict__ offs,
                                                        int32_t* __restrict__ dest, int32_t* __restrict__ src,
                                                        int64_t rows_bound) {
  __shared__ int run[kRouteMaxExperts];   // group start + earlier blocks' rows + this block's earlier passes
  const int lane = threadIdx.x;
  const int32_t* __restrict__ bb = base + (int64_t)blockIdx.x * E;
  for (int e = lane; e < E; e += 64) run[e] = offs[e] - (counts[e] + pad - 1) / pad * pad + bb[e];
  __syncthreads();
  const int64_t s0 = (int64_t)blockIdx.x * kRouteSlots;
  for (int p = 0; p < kRouteSlots / 64; ++p) {
    const int64_t s = s0 + p * 64 + lane;
    const int e = s < S ? ids[s] : -1;
    const bool valid = e >= 0 && e < E;
    // earlier and later lanes of this pass with the same expert
    int before = 0, after = 0;
    for (int j = 0; j < 64; ++j) {
      const int ej = __shfl(e, j, 64);
      before += (j < lane && ej == e) ? 1 : 0;
      after += (j > lane && ej == e) ? 1 : 0;
    }
    int d = -1;
    if (valid) d = run[e] + before;   // every lane reads run[] before any lane updates it
    __syncthreads();
    if (valid && after == 0) run[e] += before + 1;
    if (s < S) dest[s] = d;
    if (valid && d < rows_bound) src[d] = (int32_t)s;   // always true when ids do not change under the call
    __syncthreads();
  }
}

// One workgroup per grouped row: row r of xg is row src[r] / topk of x, zeros
// where src[r] is -1 (or names no slot).
__global__ __launch_bounds__(256) void permute_kernel(const uint16_t* __restrict__ x, int64_t tokens, int64_t cols,
                                                      int topk, const int32_t* __restrict__ src,
                                                      uint16_t* __restrict__ xg) {
  const int64_t r = blockIdx.x;
  const int s = src[r];
  u32x4* __restrict__ out = reinterpret_cast<u32x4*>(xg + r * cols);
  if (s >= 0 && (int64_t)s < tokens * topk) {
    const u32x4* __restrict__ in = reinterpret_cast<const u32x4*>(x + (int64_t)(s / topk) * cols);
    for (int64_t c = threadIdx.x; c < (cols >> 3); c += 256) out[c] = in[c];
  } else {
    for (int64_t c = threadIdx.x; c < (cols >> 3); c += 256) out[c] = u32x4{0, 0, 0, 0};
  }
}

typedef float rt_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 rt_bf16x2 __attribute__((ext_vector_type(2)));

// One workgroup per token: y[t] = sum_j w[t, j] * yg[dest[t, j]] in slot order.
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ yg, int64_t rows_in,
                                                      const int32_t* __restrict__ dest,
                                                      const float* __restrict__ w, int topk, int64_t cols,
                                                      uint16_t* __restrict__ y) {
#pragma clang fp contract(off)   // a product and the sum it enters round separately (no FMA)
  const int64_t t = blockIdx.x;
  const int32_t* __restrict__ dt = dest + t * topk;
  const float* __restrict__ wt = w + t * topk;
  for (int64_t c = threadIdx.x; c < (cols >> 3); c += 256) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < topk; ++j) {
      const int d = dt[j];
      if (d < 0 || (int64_t)d >= rows_in) continue;   // a dropped slot
      const float wj = wt[j];
      const u32x4 v = reinterpret_cast<const u32x4*>(yg + (int64_t)d * cols)[c];
      const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc[2 * k] = acc[2 * k] + wj * bf16_lo(vw[k]);
        acc[2 * k + 1] = acc[2 * k + 1] + wj * bf16_hi(vw[k]);
      }
    }
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      o[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(rt_f32x2{acc[2 * k], acc[2 * k + 1]}, rt_bf16x2));
    reinterpret_cast<u32x4*>(y + t * cols)[c] = u32x4{o[0], o[1], o[2], o[3]};
  }
}

hipError_t launch_moe_route(const int32_t* ids, int64_t S, int E, int pad, int32_t* counts, int32_t* offs,
                            int32_t* dest, int32_t* src, int64_t rows_bound, int32_t* workspace, hipStream_t st) {
  const int64_t nb = route_blocks(S);
  if (nb > 0)
    hipLaunchKernelGGL(route_hist_kernel, dim3((unsigned)nb), dim3(256), 0, st, ids, S, E, workspace);
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(kRouteMaxExperts), 0, st, workspace, (int)nb, E, pad, counts,
                     offs, src, rows_bound);
  if (nb > 0)
    hipLaunchKernelGGL(route_rank_kernel, dim3((unsigned)nb), dim3(64), 0, st, ids, S, E, pad, workspace, counts,
                       offs, dest, src, rows_bound);
  return hipGetLastError();
}

hipError_t launch_moe_permute(const uint16_t* x, int64_t tokens, int64_t cols, int topk, const int32_t* src,
                              int64_t rows_out, uint16_t* xg, hipStream_t st) {
  if (rows_out == 0 || cols == 0) return hipSuccess;
  hipLaunchKernelGGL(permute_kernel, dim3((unsigned)rows_out), dim3(256), 0, st, x, tokens, cols, topk, src, xg);
  return hipGetLastError();
}

hipError_t launch_moe_combine(const uint16_t* yg, int64_t rows_in, const int32_t* dest, const float* w,
                              int64_t tokens, int topk, int64_t cols, uint16_t* y, hipStream_t st) {
  if (tokens == 0 || cols == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)tokens), dim3(256), 0, st, yg, rows_in, dest, w, topk, cols, y);
  return hipGetLastError();
}

}  // namespace fp8moe

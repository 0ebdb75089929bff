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
// kRouteSlots slots and expert): per-block expert histograms (LDS atomics;
// the same grid sets every source entry to -1); one workgroup turns them into
// running counts over blocks (the rows of each expert in earlier blocks), the
// counts and the padded inclusive scan over experts (offs); one wave per block
// then ranks its slots stably (same-expert lanes found by ballots over the
// id's bits, earlier passes by a per-expert running row in LDS) and writes
// destinations and sources, a slot's row being its group's start + the
// earlier blocks' rows + its rank in the block.
#include "device_common.hpp"
#include "kernels.hpp"
#include "validate.hpp"

#include <mutex>

namespace fp8moe {

static_assert(kRouteSlots % 64 == 0, "the rank kernel walks a block in whole waves");
static_assert(kRouteMaxExperts == 1024, "the scan kernel runs one thread per (expert, range) in 1024");

// Per-block histograms; the grid also sets every source entry to -1.
__global__ __launch_bounds__(256) void route_hist_kernel(const int32_t* __restrict__ ids, int64_t S, int E,
                                                         int32_t* __restrict__ hist, int32_t* __restrict__ src,
                                                         int64_t rows_bound) {
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
  for (int64_t r = (int64_t)blockIdx.x * 256 + t; r < rows_bound; r += (int64_t)gridDim.x * 256) src[r] = -1;
  __syncthreads();
  for (int e = t; e < E; e += 256) hist[(int64_t)blockIdx.x * E + e] = h[e];
}

// Inclusive sum over the lanes of each aligned segment of `seg` lanes (seg a
// power of two <= 64) of a wave.
__device__ __forceinline__ int seg_scan(int v, int seg) {
  const int q = (threadIdx.x & 63) & (seg - 1);
  for (int off = 1; off < seg; off <<= 1) {
    const int u = __shfl_up(v, off, 64);
    if (q >= off) v += u;
  }
  return v;
}

// One workgroup: P threads per expert (P a power of two, P * E <= 1024) each
// take a range of blocks; hist[b][e] becomes the rows of e in blocks before b.
// Then counts, and offs = the inclusive scan of the padded counts.  With no
// slots (nb == 0) the histogram launch did not run and src is filled here.
// A thread keeps up to kKeep of its blocks' counts in registers (one pass over
// hist); the scans run on wave shuffles with one LDS exchange each.
__global__ __launch_bounds__(1024) void route_scan_kernel(int32_t* __restrict__ hist, int nb, int E, int P, int pad,
                                                          int32_t* __restrict__ counts, int32_t* __restrict__ offs,
                                                          int32_t* __restrict__ src, int64_t rows_bound) {
  constexpr int kKeep = 16;
  __shared__ int part[kRouteMaxExperts];   // P > 64 only: per-thread sums
  __shared__ int tot[kRouteMaxExperts];    // per-expert totals
  __shared__ int wsum[16];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int e = t / P, q = t % P;
  const bool mine = e < E;
  const int chunk = (nb + P - 1) / P;
  const int b0 = min(q * chunk, nb), b1 = min(b0 + chunk, nb);
  const bool keep = chunk <= kKeep;
  int c[kKeep];
  int sum = 0;
  if (mine) {
    if (keep) {
#pragma unroll
      for (int u = 0; u < kKeep; ++u) {
        c[u] = b0 + u < b1 ? hist[(int64_t)(b0 + u) * E + e] : 0;
        sum += c[u];
      }
    } else {
      for (int b = b0; b < b1; ++b) sum += hist[(int64_t)b * E + e];
    }
  }
  int incl;   // inclusive sum over this expert's ranges up to q
  if (P <= 64) {
    incl = seg_scan(sum, P);
  } else {    // an expert spans several waves (E <= 8)
    part[t] = sum;
    __syncthreads();
    for (int off = 1; off < P; off <<= 1) {
      const int v = q >= off ? part[t - off] : 0;
      __syncthreads();
      part[t] += v;
      __syncthreads();
    }
    incl = part[t];
  }
  if (mine) {
    int run = incl - sum;   // rows of e in blocks before b0
    if (keep) {
#pragma unroll
      for (int u = 0; u < kKeep; ++u)
        if (b0 + u < b1) {
          hist[(int64_t)(b0 + u) * E + e] = run;
          run += c[u];
        }
    } else {
      for (int b = b0; b < b1; ++b) {
        const int cb = hist[(int64_t)b * E + e];
        hist[(int64_t)b * E + e] = run;
        run += cb;
      }
    }
    if (q == P - 1) tot[e] = incl;
  }
  __syncthreads();
  const int total = t < E ? tot[t] : 0;
  const int padded = (total + pad - 1) / pad * pad;
  int x = seg_scan(padded, 64);   // inclusive scan over experts: within the wave, then across waves
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  for (int w = 0; w < wave; ++w) x += wsum[w];
  if (t < E) {
    counts[t] = total;
    offs[t] = x;
  }
  if (nb == 0)
    for (int64_t r = t; r < rows_bound; r += kRouteMaxExperts) src[r] = -1;
}

// One wave per block of kRouteSlots slots, in passes of 64.  In a pass, the
// lanes holding the same expert are found from `nbits` ballots over the bits
// of the id; a slot's rank is the number of such lanes below it, and the last
// of them advances the expert's running row in LDS.
__global__ __launch_bounds__(64) void route_rank_kernel(const int32_t* __restrict__ ids, int64_t S, int E, int nbits,
                                                        int pad, const int32_t* __restrict__ base,
                                                        const int32_t* __restrict__ counts,
                                                        const int32_t* __restrict__ offs,
                                                        int32_t* __restrict__ dest, int32_t* __restrict__ src,
                                                        int64_t rows_bound) {
  constexpr int NP = kRouteSlots / 64;
  __shared__ int run[kRouteMaxExperts];   // group start + earlier blocks' rows + this block's earlier passes
  const int lane = threadIdx.x;
  const int64_t s0 = (int64_t)blockIdx.x * kRouteSlots;
  int ev[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int64_t s = s0 + p * 64 + lane;
    ev[p] = s < S ? ids[s] : -1;
  }
  const int32_t* __restrict__ bb = base + (int64_t)blockIdx.x * E;
  for (int e = lane; e < E; e += 64) run[e] = offs[e] - (counts[e] + pad - 1) / pad * pad + bb[e];
  __syncthreads();
  const uint64_t below = (1ull << lane) - 1;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int e = ev[p];
    const bool valid = e >= 0 && e < E;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const int before = __popcll(peers & below);
    const bool last = ((peers >> lane) >> 1) == 0;
    const int d = valid ? run[e] + before : -1;   // every lane reads run[] before any lane updates it
    __syncthreads();
    if (valid && last) run[e] = d + 1;
    const int64_t s = s0 + p * 64 + lane;
    if (s < S) dest[s] = d;
    if (valid && d < rows_bound) src[d] = (int32_t)s;   // always true when ids do not change under the call
    __syncthreads();
  }
}

// Gather into the grouped layout: row r of xg is row src[r] / topk of x (rb
// bytes per row, a multiple of 16), zeros where src[r] is -1 (or names no
// slot).  With row scales (sg non-null), sg[r] is the token's scale, and a
// padding row takes the scale the rowwise recipe gives an all-zero row.
// RPB rows per workgroup (256 / RPB threads each), more when rows are short.
template <int RPB>
__global__ __launch_bounds__(256) void permute_kernel(const uint8_t* __restrict__ x, int64_t tokens, int64_t rb,
                                                      int topk, const int32_t* __restrict__ src, int64_t rows_out,
                                                      uint8_t* __restrict__ xg, const float* __restrict__ s_in,
                                                      float* __restrict__ sg, int codec) {
  constexpr int TPR = 256 / RPB;
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  if (r >= rows_out) return;   // no barrier in this kernel
  const int tid = threadIdx.x % TPR;
  const int64_t nc = rb >> 4;
  const int s = src[r];
  const bool ok = s >= 0 && (int64_t)s < tokens * topk;
  u32x4* __restrict__ out = reinterpret_cast<u32x4*>(xg + r * rb);
  if (ok) {
    const u32x4* __restrict__ in = reinterpret_cast<const u32x4*>(x + (int64_t)(s / topk) * rb);
    int64_t c = tid;
    for (; c + 3 * TPR < nc; c += 4 * TPR) {   // four 16-byte loads in flight per thread on long rows
      const u32x4 v0 = in[c], v1 = in[c + TPR], v2 = in[c + 2 * TPR], v3 = in[c + 3 * TPR];
      out[c] = v0;
      out[c + TPR] = v1;
      out[c + 2 * TPR] = v2;
      out[c + 3 * TPR] = v3;
    }
    for (; c < nc; c += TPR) out[c] = in[c];
  } else {
    for (int64_t c = tid; c < nc; c += TPR) out[c] = u32x4{0, 0, 0, 0};
  }
  if (sg != nullptr && tid == 0) sg[r] = ok ? s_in[s / topk] : scale_from_amax(0.0f, codec);
}

typedef float rt_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 rt_bf16x2 __attribute__((ext_vector_type(2)));

// One workgroup per token: y[t] = sum_j w[t, j] * yg[dest[t, j]] in slot
// order (w null: every weight 1).  A thread loads its chunk of up to eight
// rows before summing (a dropped slot loads row 0 and its result is not taken).
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ yg, int64_t rows_in,
                                                      const int32_t* __restrict__ dest,
                                                      const float* __restrict__ w, int topk, int64_t cols,
                                                      uint16_t* __restrict__ y) {
#pragma clang fp contract(off)   // a product and the sum it enters round separately (no FMA)
  constexpr int KB = 8;          // slots per batch of loads
  const int64_t t = blockIdx.x;
  const int64_t nc = cols >> 3;
  const int32_t* __restrict__ dt = dest + t * topk;
  const float* __restrict__ wt = w != nullptr ? w + t * topk : nullptr;
  u32x4* __restrict__ out = reinterpret_cast<u32x4*>(y + t * cols);
  for (int64_t c = threadIdx.x; c < nc; c += 256) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < topk; j0 += KB) {
      u32x4 v[KB];
      bool ok[KB];
#pragma unroll
      for (int u = 0; u < KB; ++u) {   // the guards are uniform over the wave
        const int j = j0 + u;
        ok[u] = false;
        v[u] = u32x4{0, 0, 0, 0};
        if (j < topk) {
          const int d = dt[j];
          ok[u] = d >= 0 && (int64_t)d < rows_in;
          if (rows_in > 0) v[u] = reinterpret_cast<const u32x4*>(yg + (int64_t)(ok[u] ? d : 0) * cols)[c];
        }
      }
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        if (j0 + u >= topk) break;
        const float wj = wt != nullptr ? wt[j0 + u] : 1.0f;
        const uint32_t vw[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float s0 = acc[2 * k] + wj * bf16_lo(vw[k]);
          const float s1 = acc[2 * k + 1] + wj * bf16_hi(vw[k]);
          acc[2 * k] = ok[u] ? s0 : acc[2 * k];
          acc[2 * k + 1] = ok[u] ? s1 : acc[2 * k + 1];
        }
      }
    }
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      o[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(rt_f32x2{acc[2 * k], acc[2 * k + 1]}, rt_bf16x2));
    // streamed (non-temporal): the layer's output is not read again by the layer's own launches, and its
    // dirty lines otherwise drain during the next launch (Llama4-Scout: the router weights' gradient that
    // follows took 80 us instead of 54 us alone)
    typedef unsigned int nt_v4u __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(nt_v4u{o[0], o[1], o[2], o[3]}, reinterpret_cast<nt_v4u*>(out + c));
  }
}

// Backward of the combine.  Workgroups [0, tokens) take one token each: the
// token's gradient row dy[t] stays in registers (ITEMS 16-byte chunks per
// thread, 256 threads), and for each of its slots s = t*topk + j, in order,
// the workgroup forms the routed row's gradient dyg[dest[s]] = bf16(w[s] *
// dy[t]) (one fp32 product, rounded to nearest even; written unless dyg is
// null), reduces the router weight's gradient dw[s] = <dy[t], yg[dest[s]]>
// (exact bf16 products, fp32 sums), and, with codes requested, quantizes the
// routed row rowwise from those bf16 values.  A dropped slot gets dw = 0.
// Workgroups from `tokens` on clear the grouped rows that hold no slot
// (padding): zeros, zero codes and the all-zero row's scale.
template <int CODEC, int ITEMS, bool QUANT>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const uint16_t* __restrict__ dy,
                                                          const uint16_t* __restrict__ yg, int64_t rows,
                                                          const int32_t* __restrict__ dest,
                                                          const int32_t* __restrict__ src,
                                                          const float* __restrict__ w, int64_t tokens, int topk,
                                                          int64_t cols, uint16_t* __restrict__ dyg,
                                                          uint8_t* __restrict__ q, float* __restrict__ scale,
                                                          float* __restrict__ dw, int zero_blocks) {
  __shared__ float red_sum[2][4];
  __shared__ uint32_t red_max[2][4];
  const int tid = threadIdx.x;
  const int64_t nc = cols >> 3;
  const int64_t S = tokens * topk;
  if ((int64_t)blockIdx.x >= tokens) {   // padding rows (no barrier on this side)
    const float s0 = scale_from_amax(0.0f, CODEC);
    for (int64_t r = (int64_t)blockIdx.x - tokens; r < rows; r += zero_blocks) {
      const int sl = src[r];
      if (sl >= 0 && (int64_t)sl < S) continue;
      if (dyg != nullptr) {
        u32x4* __restrict__ o = reinterpret_cast<u32x4*>(dyg + r * cols);
        for (int64_t c = tid; c < nc; c += 256) o[c] = u32x4{0, 0, 0, 0};
      }
      if constexpr (QUANT) {
        u32x2* __restrict__ qo = reinterpret_cast<u32x2*>(q + r * cols);
        for (int64_t c = tid; c < nc; c += 256) qo[c] = u32x2{0, 0};
        if (tid == 0) scale[r] = s0;
      }
    }
    return;
  }
  const int64_t t = blockIdx.x;
  const u32x4* __restrict__ dr = reinterpret_cast<const u32x4*>(dy + t * cols);
  u32x4 dv[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int64_t c = (int64_t)i * 256 + tid;
    dv[i] = c < nc ? dr[c] : u32x4{0, 0, 0, 0};
  }
  int b = 0;   // reduction buffer of the next slot that reduces
  for (int j = 0; j < topk; ++j) {   // uniform over the workgroup
    const int64_t sl = t * topk + j;
    const int d = dest[sl];
    if (d < 0 || (int64_t)d >= rows) {
      if (tid == 0) dw[sl] = 0.0f;
      continue;
    }
    const float wj = w[sl];
    const u32x4* __restrict__ yr = reinterpret_cast<const u32x4*>(yg + (int64_t)d * cols);
    u32x4* __restrict__ gr = dyg != nullptr ? reinterpret_cast<u32x4*>(dyg + (int64_t)d * cols) : nullptr;
    u32x4 gv[ITEMS];
    float acc = 0.0f;
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int64_t c = (int64_t)i * 256 + tid;
      gv[i] = u32x4{0, 0, 0, 0};
      if (c < nc) {
        const u32x4 yv = yr[c];
        const uint32_t dw4[4] = {dv[i].x, dv[i].y, dv[i].z, dv[i].w};
        const uint32_t yw4[4] = {yv.x, yv.y, yv.z, yv.w};
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float d0 = bf16_lo(dw4[k]), d1 = bf16_hi(dw4[k]);
          acc = fmaf(d0, bf16_lo(yw4[k]), acc);
          acc = fmaf(d1, bf16_hi(yw4[k]), acc);
          const float p0 = wj * d0, p1 = wj * d1;   // fp32 products, each rounded once
          o[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(rt_f32x2{p0, p1}, rt_bf16x2));
        }
        gv[i] = u32x4{o[0], o[1], o[2], o[3]};
        if (gr != nullptr) gr[c] = gv[i];
      }
      if constexpr (QUANT) {
        m = pk_absmax_bf16(m, gv[i].x);
        m = pk_absmax_bf16(m, gv[i].y);
        m = pk_absmax_bf16(m, gv[i].z);
        m = pk_absmax_bf16(m, gv[i].w);
      }
    }
    // workgroup reductions: the buffers alternate between reducing slots, so one barrier per slot
    // suffices (a buffer is rewritten only after the next slot's barrier, which every read precedes)
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if constexpr (QUANT) m = wave_max_u32(pk_fold(m));
    if ((tid & 63) == 0) {
      red_sum[b][tid >> 6] = acc;
      if constexpr (QUANT) red_max[b][tid >> 6] = m;
    }
    __syncthreads();
    if (tid == 0) dw[sl] = (red_sum[b][0] + red_sum[b][1]) + (red_sum[b][2] + red_sum[b][3]);
    if constexpr (QUANT) {
      m = max(max(red_max[b][0], red_max[b][1]), max(red_max[b][2], red_max[b][3]));
      const float s = scale_from_amax(__uint_as_float(m << 16), CODEC);
      u32x2* __restrict__ qr = reinterpret_cast<u32x2*>(q + (int64_t)d * cols);
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        const int64_t c = (int64_t)i * 256 + tid;
        if (c < nc)
          qr[c] = u32x2{quant_bf16x4<CODEC>(gv[i].x, gv[i].y, s), quant_bf16x4<CODEC>(gv[i].z, gv[i].w, s)};
      }
      if (tid == 0) scale[d] = s;
    }
    b ^= 1;
  }
}

hipError_t launch_moe_route(const int32_t* ids, int64_t S, int E, int pad, int32_t* counts, int32_t* offs,
                            int32_t* dest, int32_t* src, int64_t rows_bound, int32_t* workspace, hipStream_t st) {
  const int64_t nb = route_blocks(S);
  int P = 1;
  while (P * 2 * E <= kRouteMaxExperts) P *= 2;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  if (nb > 0)
    hipLaunchKernelGGL(route_hist_kernel, dim3((unsigned)nb), dim3(256), 0, st, ids, S, E, workspace, src,
                       rows_bound);
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(kRouteMaxExperts), 0, st, workspace, (int)nb, E, P, pad, counts,
                     offs, src, rows_bound);
  if (nb > 0)
    hipLaunchKernelGGL(route_rank_kernel, dim3((unsigned)nb), dim3(64), 0, st, ids, S, E, nbits, pad, workspace,
                       counts, offs, dest, src, rows_bound);
  return hipGetLastError();
}

// ------------------------------------------------------------ allocation-free routing
//
// The block histograms of moe_route_noalloc live in a fixed file-scope device
// array owned by the library: each GPU the library runs on holds its own copy
// until the process ends.  In host code the array's name is only a stand-in,
// so its device address is taken once per device with hipGetSymbolAddress
// (with that device current, at the entry point's first call on it) and only
// that address is ever passed to kernels.  Every call on a GPU shares that
// GPU's array (the histogram kernel rewrites all of it that a call uses, so
// nothing needs clearing); calls that overlap on one GPU race.
static __device__ __align__(256) int32_t scratch[kRouteScratchBytes / 4];

static int32_t* route_scratch(hipError_t* err) {
  static std::mutex mu;
  static int32_t* ptr[kMaxDevices] = {};
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (ptr[dev] == nullptr) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    ptr[dev] = static_cast<int32_t*>(p);
  }
  return ptr[dev];
}

hipError_t launch_moe_route_noalloc(const int32_t* ids, int64_t S, int E, int pad, int32_t* counts, int32_t* offs,
                                    int32_t* dest, int32_t* src, int64_t rows_bound, hipStream_t st) {
  hipError_t err = hipSuccess;
  int32_t* ws = route_scratch(&err);
  if (ws == nullptr) return err == hipSuccess ? hipErrorInvalidSymbol : err;
  return launch_moe_route(ids, S, E, pad, counts, offs, dest, src, rows_bound, ws, st);
}

// Rows per workgroup: enough that most of the 256 threads have a 16-byte chunk.
static hipError_t launch_permute(const uint8_t* x, int64_t tokens, int64_t rb, int topk, const int32_t* src,
                                 int64_t rows_out, uint8_t* xg, const float* s_in, float* sg, int codec,
                                 hipStream_t st) {
  const int64_t nc = rb >> 4;
  if (nc <= 128) {
    hipLaunchKernelGGL(permute_kernel<4>, dim3((unsigned)((rows_out + 3) / 4)), dim3(256), 0, st, x, tokens, rb, topk,
                       src, rows_out, xg, s_in, sg, codec);
  } else if (nc <= 256) {
    hipLaunchKernelGGL(permute_kernel<2>, dim3((unsigned)((rows_out + 1) / 2)), dim3(256), 0, st, x, tokens, rb, topk,
                       src, rows_out, xg, s_in, sg, codec);
  } else {
    hipLaunchKernelGGL(permute_kernel<1>, dim3((unsigned)rows_out), dim3(256), 0, st, x, tokens, rb, topk, src,
                       rows_out, xg, s_in, sg, codec);
  }
  return hipGetLastError();
}

hipError_t launch_moe_permute(const uint16_t* x, int64_t tokens, int64_t cols, int topk, const int32_t* src,
                              int64_t rows_out, uint16_t* xg, hipStream_t st) {
  if (rows_out == 0 || cols == 0) return hipSuccess;
  return launch_permute(reinterpret_cast<const uint8_t*>(x), tokens, 2 * cols, topk, src, rows_out,
                        reinterpret_cast<uint8_t*>(xg), nullptr, nullptr, 0, st);
}

hipError_t launch_moe_permute_quantized(const uint8_t* q, const float* scale, int64_t tokens, int64_t cols, int topk,
                                        const int32_t* src, int64_t rows_out, int codec, uint8_t* qg,
                                        float* scale_g, hipStream_t st) {
  if (rows_out == 0) return hipSuccess;
  return launch_permute(q, tokens, cols, topk, src, rows_out, qg, scale, scale_g, codec, st);
}

template <int CODEC, bool QUANT>
static hipError_t combine_bwd_items(const uint16_t* dy, const uint16_t* yg, int64_t rows, const int32_t* dest,
                                    const int32_t* src, const float* w, int64_t tokens, int topk, int64_t cols,
                                    uint16_t* dyg, uint8_t* q, float* scale, float* dw, hipStream_t st) {
  const int64_t items = ((cols >> 3) + 255) / 256;
  // padding rows are cleared by workgroups past `tokens`: none when nothing is written for them
  const int zero_blocks = dyg == nullptr && !QUANT ? 0 : (int)std::min<int64_t>(rows, 1024);
  if (tokens + zero_blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)(tokens + zero_blocks));
  auto go = [&](auto it_tag) -> hipError_t {
    constexpr int IT = decltype(it_tag)::value;
    hipLaunchKernelGGL((combine_bwd_kernel<CODEC, IT, QUANT>), grid, dim3(256), 0, st, dy, yg, rows, dest, src, w,
                       tokens, topk, cols, dyg, q, scale, dw, zero_blocks);
    return hipGetLastError();
  };
  if (items <= 1) return go(std::integral_constant<int, 1>{});
  if (items <= 2) return go(std::integral_constant<int, 2>{});
  if (items <= 4) return go(std::integral_constant<int, 4>{});
  if (items <= 8) return go(std::integral_constant<int, 8>{});
  return hipErrorInvalidValue;   // beyond the columns the ABI accepts
}

hipError_t launch_moe_combine_backward(const uint16_t* dy, const uint16_t* yg, int64_t rows, const int32_t* dest,
                                       const int32_t* src, const float* w, int64_t tokens, int topk, int64_t cols,
                                       int codec, uint16_t* dyg, uint8_t* q, float* scale, float* dw,
                                       hipStream_t st) {
  if (tokens == 0 && rows == 0) return hipSuccess;   // (no columns: the kernel reads nothing, dw is 0)
  const bool quant = q != nullptr;
  if (codec == 0)
    return quant ? combine_bwd_items<0, true>(dy, yg, rows, dest, src, w, tokens, topk, cols, dyg, q, scale, dw, st)
                 : combine_bwd_items<0, false>(dy, yg, rows, dest, src, w, tokens, topk, cols, dyg, q, scale, dw,
                                               st);
  return quant ? combine_bwd_items<1, true>(dy, yg, rows, dest, src, w, tokens, topk, cols, dyg, q, scale, dw, st)
               : combine_bwd_items<1, false>(dy, yg, rows, dest, src, w, tokens, topk, cols, dyg, q, scale, dw, st);
}

hipError_t launch_moe_combine(const uint16_t* yg, int64_t rows_in, const int32_t* dest, const float* w,
                              int64_t tokens, int topk, int64_t cols, uint16_t* y, hipStream_t st) {
  if (tokens == 0 || cols == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)tokens), dim3(256), 0, st, yg, rows_in, dest, w, topk, cols, y);
  return hipGetLastError();
}

}  // namespace fp8moe

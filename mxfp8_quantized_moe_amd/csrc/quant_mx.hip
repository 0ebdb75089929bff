// MXFP8 dynamic quantization: e4m3fn codes with one e8m0 scale per 1x32 block.
// [P2 Details: MXFP8 data/scale layout diagram (e4m3 data, e8m0 scale per 1x32
// block); activations and weights quantized on the fly before the scaled
// grouped GEMM; wgrad blocks run along the contracting (token) dimension.
// P4 "Скейлы: от тензора до микроблока".]
//
// The scale factor 2^-X is a power of two, so x * 2^-X is exact in fp32 (bf16
// inputs); the clamp to +-448 and the round-to-nearest-even encode follow.
// The cast runs on gfx950's scaled converter, which takes the block's e8m0
// code as its scale (mx_cvt4 in device_common.hpp states why it is exact).
//
// Two layouts:
//  * blocks along the last dim (fwd/dgrad operands, K-contiguous): 4 lanes per
//    block, 16 bytes each, a 2-step shuffle reduction.
//  * blocks along rows (wgrad operands; weights for dgrad): a 64-column tile
//    with the output transposed through LDS.  A
//    32-row block is exactly the 8 row-slots of one wave in one iteration, so
//    its reduction is three lane shuffles.  With group offsets, blocks restart
//    at every group, each group is padded to a multiple of 32 rows with +0,
//    groups sit back to back at padded offsets, and the columns past the last
//    padded group are written with zero codes and zero scales.
//
// The dual form reads each tile once and writes both: the row-block output and
// the last-dim blocks of the same rows (a weight's forward and dgrad operands,
// or an activation's dgrad and wgrad operands, from one read).
//
// Scales go out row-major ([R][NB], NB blocks per row) or in the K4 layout
// the GEMM reads one 128-wide stage at a time from: byte (r, b) at
// ((b / 4) R + r) 4 + b % 4, with the bytes past the last block of a row
// (up to the next multiple of four) written as 0.
#include "device_common.hpp"
#include "kernels.hpp"
#include "swiglu_common.hpp"
#include "tile_lds.hpp"

namespace fp8moe {

// Division of 32-bit unsigned values by a fixed divisor d >= 1 with a
// multiply-high and a shift (the round-up multiplier method): with
// l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1, the quotient is
// (mulhi(n, m) + n) >> l for every n < 2^32.
struct DivU32 {
  uint32_t m;
  int l;
  uint32_t d;
};
static DivU32 make_div(uint32_t d) {
  int l = 0;
  while (l < 32 && (1ull << l) < d) ++l;
  const uint64_t m = ((1ull << 32) * ((1ull << l) - d)) / d + 1;
  return DivU32{(uint32_t)m, l, d};
}
__device__ __forceinline__ uint32_t div_u32(uint32_t n, const DivU32& q) {
  return (uint32_t)(((uint64_t)__umulhi(n, q.m) + n) >> q.l);
}

// Byte offset of scale (row r, block b) in the K4 layout with R rows.
__device__ __forceinline__ int64_t k4_index(int64_t r, int b, int64_t R) {
  return ((int64_t)(b >> 2) * R + r) * 4 + (b & 3);
}

// ------------------------------------------------------------ last-dim blocks

template <int RULE, bool K4>
__global__ __launch_bounds__(256) void mx_lastdim_kernel(const uint16_t* __restrict__ x, int64_t n_chunks,
                                                         uint8_t* __restrict__ q, uint8_t* __restrict__ sc,
                                                         DivU32 nb, int64_t n_rows) {
  // chunk = 8 consecutive elements; 4 chunks = one block; rows are multiples of 32
  for (int64_t ci = (int64_t)blockIdx.x * 256 + threadIdx.x; ci < n_chunks; ci += (int64_t)gridDim.x * 256) {
    const u32x4 v = reinterpret_cast<const u32x4*>(x)[ci];
    uint32_t m = pk_absmax_bf16(pk_absmax_bf16(0u, v.x), v.y);
    m = pk_fold(pk_absmax_bf16(pk_absmax_bf16(m, v.z), v.w));
    m = lane_max_xor<2, false>(lane_max_xor<1, false>(m));
    const int X = mx_exponent_bf16(m, RULE);
    const float s = mx_scale_operand(X + 127);
    reinterpret_cast<u32x2*>(q)[ci] = u32x2{mx_cvt4<RULE == 0>(v.x, v.y, s), mx_cvt4<RULE == 0>(v.z, v.w, s)};
    if constexpr (K4) {
      // 16 lanes hold one stage's four blocks of one row when rows have whole
      // stages (chunks start at multiples of 256, rows at multiples of 16):
      // their first lane writes the four codes as one word.  Otherwise a
      // block's first lane writes its byte (and the row's padding).
      const uint32_t blk = (uint32_t)(ci >> 2);          // < 2^31: the K4 tensor is bounded by the host
      if ((nb.d & 3) == 0) {
        const int lane = threadIdx.x & 63;
        const uint32_t e = (uint32_t)(X + 127);
        const uint32_t w = e | ((uint32_t)__shfl((int)e, lane + 4, 64) << 8) |
                           ((uint32_t)__shfl((int)e, lane + 8, 64) << 16) |
                           ((uint32_t)__shfl((int)e, lane + 12, 64) << 24);
        if ((ci & 15) == 0) {
          const uint32_t r = div_u32(blk, nb);
          *reinterpret_cast<uint32_t*>(sc + k4_index(r, (int)(blk - r * nb.d), n_rows)) = w;
        }
      } else if ((ci & 3) == 0) {
        const uint32_t r = div_u32(blk, nb);
        const int b = (int)(blk - r * nb.d);
        uint8_t* d = sc + k4_index(r, b, n_rows);
        d[0] = (uint8_t)(X + 127);
        if (b == (int)nb.d - 1)
          for (int e = 1; (b + e) & 3; ++e) d[e] = 0;   // pad to the stage's four blocks
      }
    } else if ((ci & 3) == 0) {
      sc[ci >> 2] = (uint8_t)(X + 127);
    }
  }
}

// ------------------------------------------------------------ row blocks

// Row-block work items are 64 columns x kMxRows rows: a 16 KiB LDS tile and 32
// data registers per thread, so several workgroups share a CU and hide each
// other's load latency.
constexpr int kMxRows = 256;
constexpr int kMxIters = kMxRows / 128;
constexpr int kMxTileBytes = kTileCols * kMxRows;

// Column c, row r of the codes tile (the colwise tile's swizzle over 16 segments).
__device__ __forceinline__ int mx_tile_off(int c, int r) {
  return c * kMxRows + ((((r >> 4) ^ (2 * (c >> 3))) & (kMxRows / 16 - 1)) << 4) + (r & 15);
}

__device__ __forceinline__ int mx_chunks(int lo, int hi) {
  const int mp = (hi - lo + 31) & ~31;
  return (mp + kMxRows - 1) / kMxRows;   // an empty group owns no unit
}
struct MxChunks {
  __device__ int operator()(int lo, int hi) const { return mx_chunks(lo, hi); }
};
struct MxPad {
  __device__ int operator()(int lo, int hi) const { return (hi - lo + 31) & ~31; }
};

// Padded offsets of a grouped row-block call: inclusive cumulative sum of
// ceil32 of each group's rows (one workgroup, 256 threads).
__device__ __noinline__ void mx_write_offs_pad(const int32_t* __restrict__ offs, int n_groups, int rows,
                                               int32_t* __restrict__ offs_pad_out) {
  __shared__ int tmp[4];
  __shared__ int s_hi[256];
  __shared__ int s_tot[2];
  const int t = threadIdx.x;
  int carry = 0, pbase = 0;
  for (int g0 = 0; g0 < n_groups; g0 += 256) {
    const int e = g0 + t;
    const int vv = e < n_groups ? clamp_off(offs[e], rows) : 0;
    const int h = max(block_scan_max<256>(vv, tmp), carry);
    s_hi[t] = h;
    __syncthreads();
    const int l = t == 0 ? carry : s_hi[t - 1];
    const int pd = e < n_groups ? ((h - l + 31) & ~31) : 0;
    const int pincl = block_scan_sum<256>(pd, tmp) + pbase;
    if (e < n_groups) offs_pad_out[e] = pincl;
    if (t == 255) { s_tot[0] = pincl; s_tot[1] = h; }
    __syncthreads();
    pbase = s_tot[0];
    carry = s_tot[1];
    __syncthreads();
  }
}

template <int RULE, bool GROUPED, bool K4>
__global__ __launch_bounds__(256) void mx_rows_kernel(const uint16_t* __restrict__ x, int64_t batch, int rows,
                                                      int cols, const int32_t* __restrict__ offs, int n_groups,
                                                      uint8_t* __restrict__ q, uint8_t* __restrict__ sc,
                                                      int64_t rows_pad, int32_t* __restrict__ offs_pad_out,
                                                      int n_strips) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kMxTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_x[64 * (kMxRows / 32)];   // e8m0 codes: [column][block of the tile]

  const int strip = blockIdx.x % n_strips;
  const int u = blockIdx.x / n_strips;
  const int t = threadIdx.x, cc = t & 7, rs = t >> 3, lane = t & 63, w = t >> 6;

  // geometry: input rows [lo, hi) -> padded output rows [plo, phi) of the output space
  int lo, hi, plo, phi, j;
  int64_t ld_q;
  uint8_t* qb;
  int64_t srow0, s_rows;   // scale row of column 0 and scale rows in all
  int s_nb;                // blocks per scale row
  if constexpr (GROUPED) {
    if (blockIdx.x == 0 && offs_pad_out != nullptr) mx_write_offs_pad(offs, n_groups, rows, offs_pad_out);
    const Unit un = find_unit_quant<256>(offs, n_groups, rows, u, MxChunks{}, MxPad{});
    if (un.e >= 0) {
      lo = un.lo; hi = un.hi; plo = un.pbase; phi = plo + ((hi - lo + 31) & ~31); j = un.j;
    } else {
      // tail: columns [padded total, rows_pad) get zero codes and zero scales
      lo = hi = 0; plo = un.pbase; phi = (int)rows_pad; j = un.j;
      if (plo + j * kMxRows >= phi) return;
    }
    ld_q = rows_pad; qb = q;
    srow0 = 0; s_rows = cols; s_nb = (int)(rows_pad / 32);
  } else {
    const int upb = mx_chunks(0, rows);
    const int64_t b = upb ? u / upb : batch;
    if (b >= batch) return;
    j = u % upb;
    lo = (int)0; hi = rows; plo = 0; phi = rows;
    ld_q = rows;
    qb = q + b * cols * (int64_t)rows;
    srow0 = b * cols; s_rows = batch * cols; s_nb = rows / 32;
    x += b * (int64_t)rows * cols;
  }

  const int A = plo + j * kMxRows;                 // output row of tile row 0 (multiple of 32)
  const int r_end = min(A + kMxRows, phi);         // output rows of this unit: [A, r_end)
  const int c0 = strip * kTileCols;
  const int col = c0 + cc * 8;
  const bool col_ok = col < cols;
  // an interior tile (all 512 rows and 64 columns are input data) loads without checks
  const bool full = c0 + kTileCols <= cols && A + kMxRows <= r_end && lo + (A + kMxRows - plo) <= hi;
  u32x4 v[kMxIters][4];
  if (full) {
    const uint16_t* xr = x + (int64_t)(lo + A - plo + 4 * rs) * cols + col;   // this thread's first row
#pragma unroll
    for (int i = 0; i < kMxIters; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) v[i][k] = *reinterpret_cast<const u32x4*>(xr + (int64_t)(128 * i + k) * cols);
  } else {
#pragma unroll
    for (int i = 0; i < kMxIters; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int r = A + 128 * i + 4 * rs + k;       // output row
        const int in = lo + (r - plo);                 // input row (pad rows: in >= hi)
        const bool ok = col_ok && r < r_end && in < hi;
        v[i][k] = ok ? *reinterpret_cast<const u32x4*>(x + (int64_t)in * cols + col) : u32x4{0, 0, 0, 0};
      }
  }

#pragma unroll
  for (int i = 0; i < kMxIters; ++i) {
    uint32_t m[4] = {0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      m[0] = pk_absmax_bf16(m[0], v[i][k].x);
      m[1] = pk_absmax_bf16(m[1], v[i][k].y);
      m[2] = pk_absmax_bf16(m[2], v[i][k].z);
      m[3] = pk_absmax_bf16(m[3], v[i][k].w);
    }
    // the 32-row block of this wave: reduce over the 8 row slots (lanes 8 apart)
#pragma unroll
    for (int p = 0; p < 4; ++p)
      m[p] = lane_max_xor<32, true>(lane_max_xor<16, true>(lane_max_xor<8, true>(m[p])));
    float s[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t a16 = (m[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
      const int X = mx_exponent_bf16(a16, RULE);
      s[k] = mx_scale_operand(X + 127);
      if (lane < 8) s_x[(cc * 8 + k) * (kMxRows / 32) + 4 * i + w] = (uint8_t)(X + 127);
    }
    // column k of rows 0..3: the bf16 pairs (row 0, row 1) and (row 2, row 3) of that column, built
    // with byte permutes, give the column's four codes in row order, one word for the tile
    const uint32_t r0[4] = {v[i][0].x, v[i][0].y, v[i][0].z, v[i][0].w};
    const uint32_t r1[4] = {v[i][1].x, v[i][1].y, v[i][1].z, v[i][1].w};
    const uint32_t r2[4] = {v[i][2].x, v[i][2].y, v[i][2].z, v[i][2].w};
    const uint32_t r3[4] = {v[i][3].x, v[i][3].y, v[i][3].z, v[i][3].w};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t sel = (k & 1) ? 0x07060302u : 0x05040100u;   // high or low bf16 of each word
      const uint32_t p01 = __builtin_amdgcn_perm(r1[k >> 1], r0[k >> 1], sel);
      const uint32_t p23 = __builtin_amdgcn_perm(r3[k >> 1], r2[k >> 1], sel);
      const uint32_t word = mx_cvt4<RULE == 0>(p01, p23, s[k]);
      *reinterpret_cast<uint32_t*>(tile + mx_tile_off(cc * 8 + k, 128 * i + 4 * rs)) = word;
    }
  }
  __syncthreads();

  // transposed store: each pass writes 16 columns x 16 segments of 16 rows
  constexpr int kSeg = kMxRows / 16, kColsPerPass = 256 / kSeg, kPasses = kTileCols / kColsPerPass;
  if (full) {
    uint8_t* qo = qb + (int64_t)(c0 + t / kSeg) * ld_q + A + 16 * (t % kSeg);
#pragma unroll
    for (int p = 0; p < kPasses; ++p)
      *reinterpret_cast<u32x4*>(qo + (int64_t)(kColsPerPass * p) * ld_q) =
          *reinterpret_cast<const u32x4*>(tile + mx_tile_off(p * kColsPerPass + t / kSeg, 16 * (t % kSeg)));
  } else {
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int ci = p * kColsPerPass + t / kSeg, sg = t % kSeg;
      const int c = c0 + ci, R0 = A + 16 * sg;
      if (c < cols && R0 < r_end)
        *reinterpret_cast<u32x4*>(qb + (int64_t)c * ld_q + R0) = *reinterpret_cast<const u32x4*>(tile + mx_tile_off(ci, 16 * sg));
    }
  }
  // scales: column t/4, blocks 4*(t%4) .. +3 of this tile
  {
    constexpr int kBlk = kMxRows / 32, kThrPerCol = kBlk / 4;   // block quads per column
    const int ci = t / kThrPerCol, c = c0 + ci;
    const int nb = (r_end - A) >> 5;
    if (ci < kTileCols && c < cols) {
      const int64_t srow = srow0 + c;
      const int b0 = 4 * (t % kThrPerCol), blk0 = (A >> 5) + b0;
      if (b0 + 4 <= nb && (blk0 & 3) == 0 && (K4 || (s_nb & 3) == 0)) {
        // four whole blocks starting at a multiple of four: one aligned word
        const uint32_t wv = *reinterpret_cast<const uint32_t*>(s_x + ci * kBlk + b0);
        *reinterpret_cast<uint32_t*>(sc + (K4 ? k4_index(srow, blk0, s_rows) : srow * s_nb + blk0)) = wv;
      } else {
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) {
          const int b = b0 + b4;
          if (b < nb) {
            const int blk = (A >> 5) + b;
            if constexpr (K4) {
              uint8_t* d = sc + k4_index(srow, blk, s_rows);
              d[0] = s_x[ci * kBlk + b];
              if (blk == s_nb - 1)
                for (int e = 1; (blk + e) & 3; ++e) d[e] = 0;   // pad to the stage's four blocks
            } else {
              sc[srow * s_nb + blk] = s_x[ci * kBlk + b];
            }
          }
        }
      }
    }
  }
}

int64_t mx_rows_units_bound(int64_t batch, int64_t rows, const int32_t* offs, int32_t n_groups, int64_t rows_pad) {
  if (offs) return (rows_pad + kMxRows - 1) / kMxRows + n_groups + 1;
  return batch * ((rows + kMxRows - 1) / kMxRows);
}

template <int RULE>
static hipError_t launch_rows(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, const int32_t* offs,
                              int32_t n_groups, bool k4, uint8_t* q, uint8_t* sc, int64_t rows_pad,
                              int32_t* offs_pad_out, dim3 grid, int n_strips, hipStream_t st) {
  if (offs) {
    auto k = k4 ? mx_rows_kernel<RULE, true, true> : mx_rows_kernel<RULE, true, false>;
    hipLaunchKernelGGL(k, grid, dim3(256), 0, st, x, (int64_t)1, (int)rows, (int)cols, offs, n_groups, q, sc,
                       rows_pad, offs_pad_out, n_strips);
  } else {
    auto k = k4 ? mx_rows_kernel<RULE, false, true> : mx_rows_kernel<RULE, false, false>;
    hipLaunchKernelGGL(k, grid, dim3(256), 0, st, x, batch, (int)rows, (int)cols, nullptr, 0, q, sc, rows,
                       nullptr, n_strips);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_mx(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, int axis,
                              const int32_t* offs, int32_t n_groups, int rule, int scale_layout, uint8_t* q,
                              uint8_t* sc, int64_t rows_pad, int32_t* offs_pad_out, hipStream_t st) {
  const bool k4 = scale_layout == 1;
  if (axis == 1) {
    const int64_t n_chunks = batch * rows * cols / 8;
    if (n_chunks == 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n_chunks + 255) / 256, 1 << 20);
    const DivU32 nb = make_div((uint32_t)(cols / 32));
    const int64_t n_rows = batch * rows;
    auto k = rule == 0 ? (k4 ? mx_lastdim_kernel<0, true> : mx_lastdim_kernel<0, false>)
                       : (k4 ? mx_lastdim_kernel<1, true> : mx_lastdim_kernel<1, false>);
    hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(256), 0, st, x, n_chunks, q, sc, nb, n_rows);
    return hipGetLastError();
  }
  if (cols == 0) {
    if (offs == nullptr || offs_pad_out == nullptr) return hipSuccess;
  }
  const int n_strips = (int)std::max<int64_t>((cols + kTileCols - 1) / kTileCols, 1);
  const int64_t units = mx_rows_units_bound(batch, rows, offs, n_groups, rows_pad);
  if (units == 0) return hipSuccess;
  const dim3 grid((unsigned)(units * n_strips));
  return rule == 0 ? launch_rows<0>(x, batch, rows, cols, offs, n_groups, k4, q, sc, rows_pad, offs_pad_out, grid,
                                    n_strips, st)
                   : launch_rows<1>(x, batch, rows, cols, offs, n_groups, k4, q, sc, rows_pad, offs_pad_out, grid,
                                    n_strips, st);
}

// ------------------------------------------------------------ both forms from one read
//
// Work items are 128 columns x 128 rows.  Thread t holds the 16-column slice
// cc = t & 7 of rows 4 rs .. 4 rs + 3 (rs = t >> 3), so a wave's 8 row slots
// are one 32-row block (three lane exchanges give a column's block maximum)
// and a 32-column last-dim block is the slices of two adjacent lanes (one
// exchange).  Every row's 128 last-dim codes leave as one whole cache line
// (eight 16-byte stores) and its four e8m0 bytes as one word; the row-block
// codes are transposed through a 16 KiB LDS tile and leave as 128-byte column
// segments.  Narrower items than the row-block kernel's 64 x 256: with 64
// columns, each workgroup wrote half of every row's line and the two halves
// met only in memory.
constexpr int kDualRows = 128, kDualCols = 128;

// Where the dual kernel's tensor comes from.  PROD 0: read as is.  PROD 1: the
// SwiGLU output bf16(silu(gate) * up) computed from W1's output h1 (gate in
// columns [0, F), up in [F, 2F)).  PROD 2: SwiGLU's input gradient [d gate |
// d up] (2F columns) computed from dA2 and h1.  The tensor then never exists
// in memory unless `out` asks for a bf16 copy.  Columns of a 16-column slice
// never straddle F (F % 16 == 0).
struct DualSrc {
  const uint16_t* x;      // PROD 0: [rows][cols]; PROD 3: token rows [tokens][cols]
  const uint16_t* h1;     // PROD 1, 2: [rows][ld_h1]
  const uint16_t* da2;    // PROD 2: [rows][F]
  int64_t ld_h1;
  int F;
  uint16_t* out;          // optional bf16 copy of the tensor, [rows][cols]
  const int32_t* src;     // PROD 3: [rows] routing slot of each grouped row
  const float* gw;        // PROD 3: [slots] router weights, or null
  int topk;               // PROD 3: slots per token
  int64_t slots;          // PROD 3: tokens * topk
};


// The 16 columns [col, col + 16) of tensor row `row` (cols columns) as two 8-column chunks.
template <int PROD>
__device__ __forceinline__ void dual_load(const DualSrc& sr, int64_t row, int col, int cols, u32x4& v0, u32x4& v1) {
  if constexpr (PROD == 0) {
    const uint16_t* p = sr.x + row * cols + col;
    v0 = *reinterpret_cast<const u32x4*>(p);
    v1 = *reinterpret_cast<const u32x4*>(p + 8);
  } else if constexpr (PROD == 3) {
    // grouped row `row` holds routing slot s = src[row] of token s / topk (a zero row for no slot),
    // times the slot's router weight when weights are given
    const int sl = sr.src[row];
    if (sl < 0 || (int64_t)sl >= sr.slots) {
      v0 = v1 = u32x4{0, 0, 0, 0};
      return;
    }
    const uint16_t* p = sr.x + (int64_t)(sl / sr.topk) * cols + col;
    v0 = *reinterpret_cast<const u32x4*>(p);
    v1 = *reinterpret_cast<const u32x4*>(p + 8);
    if (sr.gw != nullptr) {
      const float wj = sr.gw[sl];
      v0 = bf16x8_times(v0, wj);
      v1 = bf16x8_times(v1, wj);
    }
  } else if constexpr (PROD == 1) {
    const uint16_t* g = sr.h1 + row * sr.ld_h1 + col;
    const u32x4 g0 = *reinterpret_cast<const u32x4*>(g), g1 = *reinterpret_cast<const u32x4*>(g + 8);
    const u32x4 u0 = *reinterpret_cast<const u32x4*>(g + sr.F), u1 = *reinterpret_cast<const u32x4*>(g + sr.F + 8);
    v0 = sw_fwd_chunk(g0, u0);
    v1 = sw_fwd_chunk(g1, u1);
  } else {
    const bool up = col >= sr.F;
    const int cf = up ? col - sr.F : col;
    const uint16_t* d = sr.da2 + row * sr.F + cf;
    const uint16_t* g = sr.h1 + row * sr.ld_h1 + cf;
    const u32x4 d0 = *reinterpret_cast<const u32x4*>(d), d1 = *reinterpret_cast<const u32x4*>(d + 8);
    const u32x4 g0 = *reinterpret_cast<const u32x4*>(g), g1 = *reinterpret_cast<const u32x4*>(g + 8);
    const u32x4 u0 = *reinterpret_cast<const u32x4*>(g + sr.F), u1 = *reinterpret_cast<const u32x4*>(g + sr.F + 8);
    u32x4 dg, du;
    sw_bwd_chunk(d0, g0, u0, dg, du);
    v0 = up ? du : dg;
    sw_bwd_chunk(d1, g1, u1, dg, du);
    v1 = up ? du : dg;
  }
}

// Column c, row r of the codes tile: 8 segments of 16 rows per column, the
// segment index XOR-ed with the 16-column slice so a wave's 4-row writes of
// one slice column spread over 32 banks.
__device__ __forceinline__ int mx_dual_off(int c, int r) {
  return c * kDualRows + ((((r >> 4) ^ (c >> 4)) & 7) << 4) + (r & 15);
}

__device__ __forceinline__ int mx_dual_chunks(int lo, int hi) {
  return (((hi - lo + 31) & ~31) + kDualRows - 1) / kDualRows;
}
struct MxDualChunks {
  __device__ int operator()(int lo, int hi) const { return mx_dual_chunks(lo, hi); }
};

template <int RULE, bool GROUPED, bool K4, int PROD>
__global__ __launch_bounds__(256) void mx_dual_kernel(DualSrc sr, int64_t batch, int rows,
                                                      int cols, const int32_t* __restrict__ offs, int n_groups,
                                                      uint8_t* __restrict__ ql, uint8_t* __restrict__ scl,
                                                      int64_t l_rows, uint8_t* __restrict__ q,
                                                      uint8_t* __restrict__ sc, int64_t rows_pad,
                                                      int32_t* __restrict__ offs_pad_out, int n_strips) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kDualCols * kDualRows];
  __shared__ __attribute__((aligned(16))) uint8_t s_x[kDualCols * (kDualRows / 32)];   // [column][block]

  int strip = blockIdx.x % n_strips;
  int u = blockIdx.x / n_strips;
  if constexpr (!GROUPED) {
    // Weights: items in bands of 8 row blocks, row blocks fastest within a
    // band, so items issued together write adjacent 128-byte pieces of the same
    // transposed output rows (1 KiB runs) while still reading whole 256-byte
    // row segments (Llama4-Scout W1 1082 -> 1047 us; bands of 4, 16, 32 and
    // row blocks fastest over the whole tensor measured slower).
    const int units = (int)(gridDim.x / n_strips);
    const int band = blockIdx.x / (8 * n_strips), rem = blockIdx.x % (8 * n_strips);
    const int rows_in = min(8, units - 8 * band);
    u = 8 * band + rem % rows_in;
    strip = rem / rows_in;
  }
  const int t = threadIdx.x, cc = t & 7, rs = t >> 3, lane = t & 63, w = t >> 6;

  // geometry, as the row-block kernel: input rows [lo, hi) -> padded output rows [plo, phi)
  int lo, hi, plo, phi, j;
  int64_t ld_q;
  uint8_t* qb;
  int64_t srow0, s_rows;   // row-block scales: row of column 0, rows in all
  int s_nb;                // row-block scales: blocks per row
  int64_t lrow0 = 0;       // last-dim output row of input row 0
  if constexpr (GROUPED) {
    if (blockIdx.x == 0 && offs_pad_out != nullptr) mx_write_offs_pad(offs, n_groups, rows, offs_pad_out);
    const Unit un = find_unit_quant<256>(offs, n_groups, rows, u, MxDualChunks{}, MxPad{});
    if (un.e >= 0) {
      lo = un.lo; hi = un.hi; plo = un.pbase; phi = plo + ((hi - lo + 31) & ~31); j = un.j;
    } else {
      lo = hi = 0; plo = un.pbase; phi = (int)rows_pad; j = un.j;
      if (plo + j * kDualRows >= phi) return;
    }
    ld_q = rows_pad; qb = q;
    srow0 = 0; s_rows = cols; s_nb = (int)(rows_pad / 32);
  } else {
    const int upb = mx_dual_chunks(0, rows);
    const int64_t b = upb ? u / upb : batch;
    if (b >= batch) return;
    j = u % upb;
    lo = 0; hi = rows; plo = 0; phi = rows;
    ld_q = rows;
    qb = q + b * cols * (int64_t)rows;
    srow0 = b * cols; s_rows = batch * cols; s_nb = rows / 32;
    lrow0 = b * (int64_t)rows;                     // tensor rows of batch item b start here
  }

  const int A = plo + j * kDualRows;               // output row of tile row 0 (multiple of 32)
  const int r_end = min(A + kDualRows, phi);
  // Items stride over the columns of the tensor, except for SwiGLU's backward, whose items stride
  // over F and emit both the d gate tile (columns c0 ..) and the d up tile (F + c0 ..) of dH1 from one
  // evaluation of the product rule (F % 128 == 0, so those tiles are whole).
  const int cols_i = PROD == 2 ? sr.F : cols;
  const int c0 = strip * kDualCols;
  const int col = c0 + cc * 16;
  const bool col_ok = col < cols_i;                // cols % 32 == 0: a slice is wholly in or out
  const bool full = c0 + kDualCols <= cols_i && A + kDualRows <= r_end && lo + (A + kDualRows - plo) <= hi;
  u32x4 v[4][2], vu[PROD == 2 ? 4 : 1][2];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = A + 4 * rs + k, in = lo + (r - plo);
    v[k][0] = v[k][1] = u32x4{0, 0, 0, 0};
    if constexpr (PROD == 2) vu[k][0] = vu[k][1] = u32x4{0, 0, 0, 0};
    if (full || (col_ok && r < r_end && in < hi)) {
      if constexpr (PROD == 2) {
        const int64_t row = lrow0 + in;
        const uint16_t* d = sr.da2 + row * sr.F + col;
        const uint16_t* g = sr.h1 + row * sr.ld_h1 + col;
        const u32x4 d0 = *reinterpret_cast<const u32x4*>(d), d1 = *reinterpret_cast<const u32x4*>(d + 8);
        const u32x4 g0 = *reinterpret_cast<const u32x4*>(g), g1 = *reinterpret_cast<const u32x4*>(g + 8);
        const u32x4 u0 = *reinterpret_cast<const u32x4*>(g + sr.F), u1 = *reinterpret_cast<const u32x4*>(g + sr.F + 8);
        sw_bwd_chunk(d0, g0, u0, v[k][0], vu[k][0]);
        sw_bwd_chunk(d1, g1, u1, v[k][1], vu[k][1]);
        if (sr.out != nullptr) {
          uint16_t* o = sr.out + row * cols + col;
          *reinterpret_cast<u32x4*>(o) = v[k][0];
          *reinterpret_cast<u32x4*>(o + 8) = v[k][1];
          *reinterpret_cast<u32x4*>(o + sr.F) = vu[k][0];
          *reinterpret_cast<u32x4*>(o + sr.F + 8) = vu[k][1];
        }
      } else {
        dual_load<PROD>(sr, lrow0 + in, col, cols, v[k][0], v[k][1]);
        if (sr.out != nullptr) {
          uint16_t* o = sr.out + (lrow0 + in) * cols + col;
          *reinterpret_cast<u32x4*>(o) = v[k][0];
          *reinterpret_cast<u32x4*>(o + 8) = v[k][1];
        }
      }
    }
  }

  // Both MX forms of the 128 x 128 register tile `v`, whose column 0 is tensor column c0o.
  auto emit = [&](const u32x4 (&v)[4][2], const int c0o) {
  const int col = c0o + cc * 16;
  // last-dim blocks: per row, the 32 columns of lanes cc and cc ^ 1
  {
    const int nb = cols >> 5, b0 = c0o >> 5;             // b0 % 4 == 0: a tile row is one K4 word
    const int nvalid = min(4, nb - b0);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t m = 0;
      m = pk_absmax_bf16(m, v[k][0].x); m = pk_absmax_bf16(m, v[k][0].y);
      m = pk_absmax_bf16(m, v[k][0].z); m = pk_absmax_bf16(m, v[k][0].w);
      m = pk_absmax_bf16(m, v[k][1].x); m = pk_absmax_bf16(m, v[k][1].y);
      m = pk_absmax_bf16(m, v[k][1].z); m = pk_absmax_bf16(m, v[k][1].w);
      m = lane_max_xor<1, false>(pk_fold(m));
      const int X = mx_exponent_bf16(m, RULE);
      const float so = mx_scale_operand(X + 127);
      const uint32_t e = (uint32_t)(X + 127);
      const uint32_t e1 = (uint32_t)__shfl((int)e, lane + 2, 64);   // blocks 1..3 of the row (lanes cc 2, 4, 6)
      const uint32_t e2 = (uint32_t)__shfl((int)e, lane + 4, 64);
      const uint32_t e3 = (uint32_t)__shfl((int)e, lane + 6, 64);
      const int r = A + 4 * rs + k, in = lo + (r - plo);
      if (full || (r < r_end && in < hi)) {
        const int64_t grow = lrow0 + in;
        if (col_ok)
          *reinterpret_cast<u32x4*>(ql + grow * cols + col) =
              u32x4{mx_cvt4<RULE == 0>(v[k][0].x, v[k][0].y, so), mx_cvt4<RULE == 0>(v[k][0].z, v[k][0].w, so),
                    mx_cvt4<RULE == 0>(v[k][1].x, v[k][1].y, so), mx_cvt4<RULE == 0>(v[k][1].z, v[k][1].w, so)};
        if (cc == 0) {
          // the blocks past the row's last (K4: up to the stage's four) are zero
          const uint32_t word = (e | (e1 << 8) | (e2 << 16) | (e3 << 24)) &
                                (nvalid >= 4 ? 0xFFFFFFFFu : ((1u << (8 * nvalid)) - 1u));
          if constexpr (K4) {
            *reinterpret_cast<uint32_t*>(scl + k4_index(grow, b0, l_rows)) = word;
          } else if (nvalid == 4 && ((grow * nb + b0) & 3) == 0) {
            *reinterpret_cast<uint32_t*>(scl + grow * nb + b0) = word;
          } else {
            for (int i = 0; i < nvalid; ++i) scl[grow * nb + b0 + i] = (uint8_t)(word >> (8 * i));
          }
        }
      }
    }
  }

  // row blocks: the wave's 32 rows of each of the thread's 16 columns
  {
    uint32_t m[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      m[4 * h + 0] = m[4 * h + 1] = m[4 * h + 2] = m[4 * h + 3] = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        m[4 * h + 0] = pk_absmax_bf16(m[4 * h + 0], v[k][h].x);
        m[4 * h + 1] = pk_absmax_bf16(m[4 * h + 1], v[k][h].y);
        m[4 * h + 2] = pk_absmax_bf16(m[4 * h + 2], v[k][h].z);
        m[4 * h + 3] = pk_absmax_bf16(m[4 * h + 3], v[k][h].w);
      }
    }
#pragma unroll
    for (int p = 0; p < 8; ++p) m[p] = lane_max_xor<32, true>(lane_max_xor<16, true>(lane_max_xor<8, true>(m[p])));
#pragma unroll
    for (int jc = 0; jc < 16; ++jc) {
      const uint32_t a16 = (m[jc >> 1] >> (16 * (jc & 1))) & 0xFFFFu;
      const int X = mx_exponent_bf16(a16, RULE);
      if (lane < 8) s_x[(cc * 16 + jc) * (kDualRows / 32) + w] = (uint8_t)(X + 127);
      const int h = jc >> 3, wi = (jc >> 1) & 3;
      auto word_of = [&](int k) {
        const u32x4& q4 = v[k][h];
        return wi == 0 ? q4.x : wi == 1 ? q4.y : wi == 2 ? q4.z : q4.w;
      };
      const uint32_t sel = (jc & 1) ? 0x07060302u : 0x05040100u;   // high or low bf16 of each word
      const uint32_t p01 = __builtin_amdgcn_perm(word_of(1), word_of(0), sel);
      const uint32_t p23 = __builtin_amdgcn_perm(word_of(3), word_of(2), sel);
      *reinterpret_cast<uint32_t*>(tile + mx_dual_off(cc * 16 + jc, 4 * rs)) =
          mx_cvt4<RULE == 0>(p01, p23, mx_scale_operand(X + 127));
    }
  }
  __syncthreads();

  // transposed codes: 4 passes of 32 columns x 8 segments of 16 rows
#pragma unroll
  for (int p = 0; p < kDualCols / 32; ++p) {
    const int ci = p * 32 + (t >> 3), sg = t & 7;
    const int c = c0o + ci, R0 = A + 16 * sg;
    const u32x4 d = *reinterpret_cast<const u32x4*>(tile + mx_dual_off(ci, 16 * sg));
    if (full || (c < cols && R0 < r_end)) *reinterpret_cast<u32x4*>(qb + (int64_t)c * ld_q + R0) = d;
  }
  // row-block scales: column t's (up to) four blocks of this item
  if (t < kDualCols) {
    const int ci = t, c = c0o + ci;
    const int nbt = (r_end - A) >> 5;
    if (c < cols) {
      const int64_t srow = srow0 + c;
      const int blk0 = A >> 5;
      if (nbt == 4 && (blk0 & 3) == 0 && (K4 || (s_nb & 3) == 0)) {
        const uint32_t wv = *reinterpret_cast<const uint32_t*>(s_x + ci * 4);
        *reinterpret_cast<uint32_t*>(sc + (K4 ? k4_index(srow, blk0, s_rows) : srow * s_nb + blk0)) = wv;
      } else {
        for (int b = 0; b < nbt; ++b) {
          const int blk = blk0 + b;
          if constexpr (K4) {
            uint8_t* d = sc + k4_index(srow, blk, s_rows);
            d[0] = s_x[ci * 4 + b];
            if (blk == s_nb - 1)
              for (int e = 1; (blk + e) & 3; ++e) d[e] = 0;   // pad to the stage's four blocks
          } else {
            sc[srow * s_nb + blk] = s_x[ci * 4 + b];
          }
        }
      }
    }
  }
  };

  emit(v, c0);
  if constexpr (PROD == 2) {
    __syncthreads();   // the codes tile and the block exponents are reused
    emit(vu, sr.F + c0);
  }
}

template <int RULE, int PROD>
static hipError_t launch_dual(const DualSrc& sr, int64_t batch, int64_t rows, int64_t cols, const int32_t* offs,
                              int32_t n_groups, bool k4, uint8_t* ql, uint8_t* scl, uint8_t* q, uint8_t* sc,
                              int64_t rows_pad, int32_t* offs_pad_out, dim3 grid, int n_strips, hipStream_t st) {
  const int64_t l_rows = batch * rows;
  if (offs) {
    auto k = k4 ? mx_dual_kernel<RULE, true, true, PROD> : mx_dual_kernel<RULE, true, false, PROD>;
    hipLaunchKernelGGL(k, grid, dim3(256), 0, st, sr, (int64_t)1, (int)rows, (int)cols, offs, n_groups, ql, scl,
                       l_rows, q, sc, rows_pad, offs_pad_out, n_strips);
  } else {
    auto k = k4 ? mx_dual_kernel<RULE, false, true, PROD> : mx_dual_kernel<RULE, false, false, PROD>;
    hipLaunchKernelGGL(k, grid, dim3(256), 0, st, sr, batch, (int)rows, (int)cols, nullptr, 0, ql, scl, l_rows, q,
                       sc, rows, nullptr, n_strips);
  }
  return hipGetLastError();
}

int64_t mx_dual_grid_bound(int64_t batch, int64_t rows, int64_t cols, bool grouped, int32_t n_groups,
                           int64_t rows_pad) {
  const int64_t units = grouped ? (rows_pad + kDualRows - 1) / kDualRows + n_groups + 1
                                : batch * ((rows + kDualRows - 1) / kDualRows);
  return units * std::max<int64_t>((cols + kDualCols - 1) / kDualCols, 1);
}

hipError_t launch_quantize_mx_dual(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols,
                                   const int32_t* offs, int32_t n_groups, int rule, int scale_layout, uint8_t* q,
                                   uint8_t* sc, uint8_t* q_t, uint8_t* sc_t, int64_t rows_pad,
                                   int32_t* offs_pad_out, hipStream_t st) {
  const bool k4 = scale_layout == 1;
  if (cols == 0) {
    if (offs == nullptr || offs_pad_out == nullptr) return hipSuccess;
  }
  const int n_strips = (int)std::max<int64_t>((cols + kDualCols - 1) / kDualCols, 1);
  const int64_t blocks = mx_dual_grid_bound(batch, rows, cols, offs != nullptr, n_groups, rows_pad);
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks);
  const DualSrc sr{x, nullptr, nullptr, 0, 0, nullptr};
  return rule == 0 ? launch_dual<0, 0>(sr, batch, rows, cols, offs, n_groups, k4, q, sc, q_t, sc_t, rows_pad,
                                       offs_pad_out, grid, n_strips, st)
                   : launch_dual<1, 0>(sr, batch, rows, cols, offs, n_groups, k4, q, sc, q_t, sc_t, rows_pad,
                                       offs_pad_out, grid, n_strips, st);
}

hipError_t launch_swiglu_mx_dual(const uint16_t* h1, const uint16_t* da2, int64_t rows, int64_t F, int64_t ld_h1,
                                 const int32_t* offs, int32_t n_groups, int rule, int scale_layout, uint16_t* out,
                                 uint8_t* q, uint8_t* sc, uint8_t* q_t, uint8_t* sc_t, int64_t rows_pad,
                                 int32_t* offs_pad_out, hipStream_t st) {
  const bool k4 = scale_layout == 1, bwd = da2 != nullptr;
  const int64_t cols = bwd ? 2 * F : F;
  if (cols == 0 && offs_pad_out == nullptr) return hipSuccess;
  const int64_t cols_i = bwd ? F : cols;   // the backward's items stride over F (two output tiles each)
  const int n_strips = (int)std::max<int64_t>((cols_i + kDualCols - 1) / kDualCols, 1);
  const int64_t blocks = mx_dual_grid_bound(1, rows, cols_i, offs != nullptr, n_groups, rows_pad);
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks);
  const DualSrc sr{nullptr, h1, da2, ld_h1, (int)F, out};
  if (bwd)
    return rule == 0 ? launch_dual<0, 2>(sr, 1, rows, cols, offs, n_groups, k4, q, sc, q_t, sc_t, rows_pad,
                                         offs_pad_out, grid, n_strips, st)
                     : launch_dual<1, 2>(sr, 1, rows, cols, offs, n_groups, k4, q, sc, q_t, sc_t, rows_pad,
                                         offs_pad_out, grid, n_strips, st);
  return rule == 0 ? launch_dual<0, 1>(sr, 1, rows, cols, offs, n_groups, k4, q, sc, q_t, sc_t, rows_pad,
                                       offs_pad_out, grid, n_strips, st)
                   : launch_dual<1, 1>(sr, 1, rows, cols, offs, n_groups, k4, q, sc, q_t, sc_t, rows_pad,
                                       offs_pad_out, grid, n_strips, st);
}

hipError_t launch_moe_permute_mx_dual(const uint16_t* x, int64_t tokens, int64_t cols, int topk, const int32_t* src,
                                     const float* weights, int64_t rows, const int32_t* offs, int32_t n_groups,
                                     int rule, int scale_layout, uint16_t* xg, uint8_t* q, uint8_t* sc, uint8_t* q_t,
                                     uint8_t* sc_t, int64_t rows_pad, int32_t* offs_pad_out, hipStream_t st) {
  const bool k4 = scale_layout == 1;
  if (cols == 0 && offs_pad_out == nullptr) return hipSuccess;
  const int n_strips = (int)std::max<int64_t>((cols + kDualCols - 1) / kDualCols, 1);
  const int64_t blocks = mx_dual_grid_bound(1, rows, cols, true, n_groups, rows_pad);
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks);
  const DualSrc sr{x, nullptr, nullptr, 0, 0, xg, src, weights, topk, tokens * topk};
  auto kern = rule == 0 ? (k4 ? mx_dual_kernel<0, true, true, 3> : mx_dual_kernel<0, true, false, 3>)
                        : (k4 ? mx_dual_kernel<1, true, true, 3> : mx_dual_kernel<1, true, false, 3>);
  hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, sr, (int64_t)1, (int)rows, (int)cols, offs, n_groups, q, sc, rows,
                     q_t, sc_t, rows_pad, offs_pad_out, n_strips);
  return hipGetLastError();
}

}  // namespace fp8moe

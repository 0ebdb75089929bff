// Blockwise FP8 scaling: one fp32 scale per fixed tile (1 x 128 along the
// contraction for activations, 128 x 128 for weights), and the grouped GEMM
// over blockwise-scaled operands.  [P4 "Скейлы: от тензора до микроблока" (a
// scale per fixed-size tile, between rowwise and MXFP8; blockwise kernels for
// MI300 and MI350); P3, the four scaling strategies.]
//
// Each tile follows the rowwise recipe: s = fmax / max(amax, 1e-12f),
// codes = enc(clamp(fp32(x * s))).  The GEMM (GROUPED_M) sums, per 128-wide
// contraction block kb, the exact FP8 products of the block in fp32 (MFMA) and
// adds that partial sum times 1 / (sa[m][kb] * sb[e][n / 128][kb]) to the
// running fp32 result: the scale changes every block, so it cannot wait for
// the epilogue as the rowwise scales do.
//
// GEMM tile 128 x 128 per workgroup, four waves of 64 x 64 (2 x 2 MFMA blocks
// of 32 x 32), 64 running + 64 partial accumulator registers per lane.  Each
// 128-wide block is staged through LDS (global -> registers -> LDS) between
// two barriers, the next block's loads in flight during the current block's
// MFMAs; registers capped for two workgroups per CU.
#include "device_common.hpp"
#include "kernels.hpp"
#include "validate.hpp"

namespace fp8moe {

namespace {

typedef int bw_v8i __attribute__((ext_vector_type(8)));
typedef float bw_v16f __attribute__((ext_vector_type(16)));

constexpr int kBwTile = 128;               // GEMM tile rows / columns and contraction block
constexpr int kBwStride = kBwTile + 16;    // LDS row stride in bytes (16-byte aligned, spreads banks)

__device__ __forceinline__ uint32_t chunk_absmax(const u32x4& v) {
  uint32_t m = pk_absmax_bf16(0u, v.x);
  m = pk_absmax_bf16(m, v.y);
  m = pk_absmax_bf16(m, v.z);
  return pk_fold(pk_absmax_bf16(m, v.w));
}

template <int CODEC>
__device__ __forceinline__ u32x2 cast_chunk(const u32x4& v, float s) {
  return u32x2{quant_bf16x4<CODEC>(v.x, v.y, s), quant_bf16x4<CODEC>(v.z, v.w, s)};
}

__device__ __forceinline__ uint16_t bw_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

}  // namespace

// 1 x 128 tiles: 16 tiles per workgroup, 16 threads per tile, one 16-byte
// chunk each.  x is [R][C] (all batch rows stacked); scale is [R][nc].
template <int CODEC>
__global__ __launch_bounds__(256) void bw_quant_rows_kernel(const uint16_t* __restrict__ x, int64_t R, int cols,
                                                            int nc, uint8_t* __restrict__ q,
                                                            float* __restrict__ scale) {
  const int t = threadIdx.x;
  const int64_t tile = (int64_t)blockIdx.x * 16 + (t >> 4);
  const bool tv = tile < R * nc;
  const int64_t row = tv ? tile / nc : 0;
  const int cb = tv ? (int)(tile % nc) : 0;
  const int c = cb * kBwTile + (t & 15) * 8;
  const bool valid = tv && c < cols;
  u32x4 v = u32x4{0, 0, 0, 0};
  if (valid) v = *reinterpret_cast<const u32x4*>(x + row * cols + c);
  uint32_t m = chunk_absmax(v);
  m = group_max_u32<16>(m);   // within 16 lanes
  const float s = scale_from_amax(__uint_as_float(m << 16), CODEC);
  if (valid) *reinterpret_cast<u32x2*>(q + row * cols + c) = cast_chunk<CODEC>(v, s);
  if (tv && (t & 15) == 0) scale[row * nc + cb] = s;
}

// 128 x 128 tiles: one tile per workgroup; thread t takes chunk column t % 16
// of rows t / 16 + 16 i (i < 8).  x is [B][R][C]; scale is [B][nr][nc].
template <int CODEC>
__global__ __launch_bounds__(256) void bw_quant_tiles_kernel(const uint16_t* __restrict__ x, int rows, int cols,
                                                             int nr, int nc, uint8_t* __restrict__ q,
                                                             float* __restrict__ scale) {
  __shared__ uint32_t red[4];
  const int t = threadIdx.x;
  const int64_t b = blockIdx.x / (nr * nc);
  const int rb = (blockIdx.x / nc) % nr, cb = blockIdx.x % nc;
  const int c = cb * kBwTile + (t & 15) * 8;
  const int64_t base = b * rows * (int64_t)cols;
  u32x4 v[8];
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = rb * kBwTile + (t >> 4) + 16 * i;
    v[i] = u32x4{0, 0, 0, 0};
    if (r < rows && c < cols) v[i] = *reinterpret_cast<const u32x4*>(x + base + (int64_t)r * cols + c);
    m = max(m, chunk_absmax(v[i]));
  }
  m = wave_max_u32(m);
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  m = max(max(red[0], red[1]), max(red[2], red[3]));
  const float s = scale_from_amax(__uint_as_float(m << 16), CODEC);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = rb * kBwTile + (t >> 4) + 16 * i;
    if (r < rows && c < cols) *reinterpret_cast<u32x2*>(q + base + (int64_t)r * cols + c) = cast_chunk<CODEC>(v[i], s);
  }
  if (t == 0) scale[blockIdx.x] = s;
}

struct BwGemm {
  const uint8_t* a;      // [M][K] e4m3fn codes
  const float* sa;       // [M][KB]
  const uint8_t* b;      // [E][N][K]
  const float* sb;       // [E][NB][KB]
  const int32_t* offs;   // [E]
  void* out;             // [M][N] bf16 or f32
  int E, M, N, K, KB, NB, col_tiles;
};

template <int OUT>
__global__ __launch_bounds__(256, 2) void bw_gemm_kernel(BwGemm p) {   // two workgroups per CU
  __shared__ __attribute__((aligned(16))) uint8_t As[kBwTile * kBwStride];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[kBwTile * kBwStride];
  __shared__ float inv_a[kBwTile];
  __shared__ float inv_b;
  struct Ch {
    __device__ int operator()(int lo, int hi) const { return (hi - lo + kBwTile - 1) / kBwTile; }
  };
  struct NoPad {
    __device__ int operator()(int, int) const { return 0; }
  };
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1, g = lane >> 5, lrow = lane & 31;
  const int ru = blockIdx.x / p.col_tiles, ct = blockIdx.x % p.col_tiles;
  const Unit un = find_unit<256>(p.offs, p.E, p.M, ru, Ch{}, NoPad{});   // every thread: it synchronizes
  if (un.e < 0) return;   // uniform
  const int e = un.e;
  const int m0 = un.lo + un.j * kBwTile, n0 = ct * kBwTile;
  const int pv = min(kBwTile, un.hi - m0), qv = min(kBwTile, p.N - n0);
  const int nb = n0 / kBwTile;

  bw_v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // Block kb + 1's operands and scales load into registers while block kb's
  // MFMAs run; they go to LDS after the barrier that ends block kb.
  u32x4 va[4], vb[4];
  float ra = 0.0f, rb = 0.0f;
  auto load_block = [&](int kb) {
    const int k0 = kb * kBwTile;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = t + 256 * u, row = idx >> 3, ch = idx & 7;
      const int k = k0 + ch * 16;
      va[u] = u32x4{0, 0, 0, 0};
      vb[u] = u32x4{0, 0, 0, 0};
      if (row < pv && k < p.K) va[u] = *reinterpret_cast<const u32x4*>(p.a + (int64_t)(m0 + row) * p.K + k);
      if (row < qv && k < p.K)
        vb[u] = *reinterpret_cast<const u32x4*>(p.b + ((int64_t)e * p.N + n0 + row) * p.K + k);
    }
    if (t < pv) ra = p.sa[(int64_t)(m0 + t) * p.KB + kb];
    if (t == kBwTile) rb = p.sb[((int64_t)e * p.NB + nb) * p.KB + kb];
  };
  if (p.KB > 0) load_block(0);
  for (int kb = 0; kb < p.KB; ++kb) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = t + 256 * u, row = idx >> 3, ch = idx & 7;
      *reinterpret_cast<u32x4*>(As + row * kBwStride + ch * 16) = va[u];
      *reinterpret_cast<u32x4*>(Bs + row * kBwStride + ch * 16) = vb[u];
    }
    if (t < kBwTile) inv_a[t] = t < pv ? __frcp_rn(ra) : 0.0f;
    if (t == kBwTile) inv_b = __frcp_rn(rb);
    __syncthreads();
    if (kb + 1 < p.KB) load_block(kb + 1);

    bw_v16f part[2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {   // two 64-wide MFMA steps; lane half g holds 32 contiguous bytes
      bw_v8i fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint8_t* pa = As + (wm * 64 + 32 * i + lrow) * kBwStride + ks * 64 + 32 * g;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(pa), hi = *reinterpret_cast<const u32x4*>(pa + 16);
        fa[i] = bw_v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        const uint8_t* pb = Bs + (wn * 64 + 32 * i + lrow) * kBwStride + ks * 64 + 32 * g;
        const u32x4 lb = *reinterpret_cast<const u32x4*>(pb), hb = *reinterpret_cast<const u32x4*>(pb + 16);
        fb[i] = bw_v8i{(int)lb.x, (int)lb.y, (int)lb.z, (int)lb.w, (int)hb.x, (int)hb.y, (int)hb.z, (int)hb.w};
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if (ks == 0) {
            bw_v16f z;
#pragma unroll
            for (int v = 0; v < 16; ++v) z[v] = 0.0f;
            part[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], z, 0, 0, 0, 0, 0, 0);
          } else {
            part[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], part[i][j], 0, 0, 0, 0, 0, 0);
          }
        }
    }
    // running result += partial / (sa * sb): element v of block (i, j) is row
    // 32 i + 8 (v / 4) + 4 g + v % 4 and column 32 j + lrow of the wave's 64 x 64
    const float ib = inv_b;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float f = inv_a[wm * 64 + 32 * i + 8 * (v >> 2) + 4 * g + (v & 3)] * ib;
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j][v] += part[i][j][v] * f;
      }
    __syncthreads();   // the next block's staging overwrites As, Bs and the scales
  }

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = wm * 64 + 32 * i + 8 * (v >> 2) + 4 * g + (v & 3);
      if (r >= pv) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = wn * 64 + 32 * j + lrow;
        if (c >= qv) continue;
        const int64_t o = (int64_t)(m0 + r) * p.N + n0 + c;
        if constexpr (OUT == 0)
          static_cast<uint16_t*>(p.out)[o] = bw_bf16_rne(acc[i][j][v]);
        else
          static_cast<float*>(p.out)[o] = acc[i][j][v];
      }
    }
}

// ---------------------------------------------------------------- weight gradient
//
// Token-major operands in 128-token blocks that restart at every group start
// (unit u = the u-th block in group order, as the scheduler enumerates them),
// one scale per column and block.  Group starts are arbitrary, so a block's
// bytes in the transposed layout are 16-byte aligned only when its first token
// is: aligned blocks move 16 bytes at a time, others byte by byte.

struct Blocks128 {
  __device__ int operator()(int lo, int hi) const { return (hi - lo + kBwTile - 1) / kBwTile; }
};
struct OnePerGroup {
  __device__ int operator()(int, int) const { return 1; }
};
struct NoPad2 {
  __device__ int operator()(int, int) const { return 0; }
};

// Unit (block, 64-column strip): thread (rq, cc) holds tokens 4rq..4rq+3 x
// columns 8cc..8cc+7; column maxima over the block by shuffles and LDS, then
// the codes go through a [column][token] LDS tile to the transposed output.
template <int CODEC>
__global__ __launch_bounds__(256) void bw_quant_tokens_kernel(const uint16_t* __restrict__ x, int M, int C,
                                                              const int32_t* __restrict__ offs, int E,
                                                              uint8_t* __restrict__ q_t, int64_t ld_q,
                                                              float* __restrict__ scale, int n_strips) {
  __shared__ uint32_t cm[4][64];
  __shared__ float s_col[64];
  __shared__ uint32_t T[64][kBwTile / 4 + 2];
  const int strip = blockIdx.x % n_strips, u = blockIdx.x / n_strips;
  const Unit un = find_unit<256>(offs, E, M, u, Blocks128{}, NoPad2{});   // every thread: it synchronizes
  if (un.e < 0) return;   // uniform
  const int t0 = un.lo + kBwTile * un.j, tl = min(kBwTile, un.hi - t0), c0 = strip * 64;
  const int t = threadIdx.x, cc = t & 7, rq = t >> 3, lane = t & 63, wave = t >> 6;
  u32x4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * rq + i, c = c0 + 8 * cc;
    v[i] = u32x4{0, 0, 0, 0};
    if (r < tl && c < C) v[i] = *reinterpret_cast<const u32x4*>(x + (int64_t)(t0 + r) * C + c);
  }
  uint32_t m[8];
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    m[jj] = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = jj < 2 ? v[i].x : jj < 4 ? v[i].y : jj < 6 ? v[i].z : v[i].w;
      m[jj] = max(m[jj], ((jj & 1) ? (w >> 16) : w) & 0x7FFFu);
    }
    m[jj] = lane_max_xor<32, false>(lane_max_xor<16, false>(lane_max_xor<8, false>(m[jj])));
  }
  if (lane < 8) {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) cm[wave][8 * lane + jj] = m[jj];
  }
  __syncthreads();
  if (t < 64) {
    const uint32_t mm = max(max(cm[0][t], cm[1][t]), max(cm[2][t], cm[3][t]));
    s_col[t] = scale_from_amax(__uint_as_float(mm << 16), CODEC);
    if (c0 + t < C) scale[(int64_t)u * C + c0 + t] = s_col[t];
  }
  __syncthreads();
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const float sc = s_col[8 * cc + jj];
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = jj < 2 ? v[i].x : jj < 4 ? v[i].y : jj < 6 ? v[i].z : v[i].w;
      const float val = (jj & 1) ? bf16_hi(w) : bf16_lo(w);
      word |= enc_fp8<CODEC>(scale_clamp<CODEC>(val, sc)) << (8 * i);
    }
    T[8 * cc + jj][rq] = word;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int seg = t + 256 * k, col = seg >> 3, rc = seg & 7;
    const int c = c0 + col, r = 16 * rc;
    if (c >= C || r >= tl) continue;
    const uint32_t* w = &T[col][4 * rc];
    uint8_t* dst = q_t + (int64_t)c * ld_q + t0 + r;
    if (tl - r >= 16 && ((t0 + r) & 15) == 0) {
      *reinterpret_cast<u32x4*>(dst) = u32x4{w[0], w[1], w[2], w[3]};
    } else {
      const int n = min(16, tl - r);
      for (int b = 0; b < n; ++b) dst[b] = (uint8_t)(w[b >> 2] >> (8 * (b & 3)));
    }
  }
}

struct BwGemmK {
  const uint8_t* a;      // phys [N][ld] codes of dY (token-contiguous)
  const float* sa;       // [TB][N]
  const uint8_t* b;      // phys [K][ld] codes of X
  const float* sb;       // [TB][K]
  const int32_t* offs;   // [E]
  void* out;             // [E][N][K]
  int E, M, N, K, NT, KT;
  int64_t ld;
};

// 16 token bytes [t0 + 16 ch, +16) of a row, bytes at or past tl zero.
__device__ __forceinline__ u32x4 bw_load_tokens(const uint8_t* __restrict__ row, int t0, int ch, int tl) {
  const int o = 16 * ch;
  if (o >= tl) return u32x4{0, 0, 0, 0};
  if ((t0 & 15) == 0 && tl - o >= 16) return *reinterpret_cast<const u32x4*>(row + t0 + o);
  uint32_t w[4] = {0, 0, 0, 0};
  const int n = min(16, tl - o);
  for (int b = 0; b < n; ++b) w[b >> 2] |= (uint32_t)row[t0 + o + b] << (8 * (b & 3));
  return u32x4{w[0], w[1], w[2], w[3]};
}

// Tile (expert e, 128 rows of N, 128 columns of K): the sum over e's token
// blocks of the block's MFMA product times 1 / (sa[tb][n] * sb[tb][k]); the
// next block's loads in flight during the current block's MFMAs.
template <int OUT>
__global__ __launch_bounds__(256, 2) void bw_gemm_k_kernel(BwGemmK p) {
  __shared__ __attribute__((aligned(16))) uint8_t As[kBwTile * kBwStride];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[kBwTile * kBwStride];
  __shared__ float inv_a[kBwTile], inv_b[kBwTile];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1, g = lane >> 5, lrow = lane & 31;
  const int e = blockIdx.x / (p.NT * p.KT), nt = (blockIdx.x / p.KT) % p.NT, kt = blockIdx.x % p.KT;
  // one unit per group: unit e is group e; pbase counts the 128-token blocks of the groups before it
  const Unit un = find_unit<256>(p.offs, p.E, p.M, e, OnePerGroup{}, Blocks128{});
  const int n0 = nt * kBwTile, k0 = kt * kBwTile;
  const int nv = min(kBwTile, p.N - n0), kv = min(kBwTile, p.K - k0);
  const int lo = un.lo, hi = max(un.hi, un.lo), tb0 = un.pbase;
  const int nblk = (hi - lo + kBwTile - 1) / kBwTile;

  bw_v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // Block jb + 1's operands and scale load into registers while block jb's MFMAs run.
  u32x4 va[4], vb[4];
  float rs = 0.0f;
  auto load_block = [&](int jb) {
    const int t0 = lo + kBwTile * jb, tl = min(kBwTile, hi - t0), tb = tb0 + jb;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = t + 256 * u, row = idx >> 3, ch = idx & 7;
      va[u] = row < nv ? bw_load_tokens(p.a + (int64_t)(n0 + row) * p.ld, t0, ch, tl) : u32x4{0, 0, 0, 0};
      vb[u] = row < kv ? bw_load_tokens(p.b + (int64_t)(k0 + row) * p.ld, t0, ch, tl) : u32x4{0, 0, 0, 0};
    }
    if (t < kBwTile) rs = t < nv ? p.sa[(int64_t)tb * p.N + n0 + t] : 1.0f;
    else rs = t - kBwTile < kv ? p.sb[(int64_t)tb * p.K + k0 + t - kBwTile] : 1.0f;
  };
  if (nblk > 0) load_block(0);
  for (int jb = 0; jb < nblk; ++jb) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = t + 256 * u, row = idx >> 3, ch = idx & 7;
      *reinterpret_cast<u32x4*>(As + row * kBwStride + ch * 16) = va[u];
      *reinterpret_cast<u32x4*>(Bs + row * kBwStride + ch * 16) = vb[u];
    }
    if (t < kBwTile) inv_a[t] = t < nv ? __frcp_rn(rs) : 0.0f;
    else inv_b[t - kBwTile] = t - kBwTile < kv ? __frcp_rn(rs) : 0.0f;
    __syncthreads();
    if (jb + 1 < nblk) load_block(jb + 1);
    bw_v16f part[2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bw_v8i fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint8_t* pa = As + (wm * 64 + 32 * i + lrow) * kBwStride + ks * 64 + 32 * g;
        const u32x4 l0 = *reinterpret_cast<const u32x4*>(pa), h0 = *reinterpret_cast<const u32x4*>(pa + 16);
        fa[i] = bw_v8i{(int)l0.x, (int)l0.y, (int)l0.z, (int)l0.w, (int)h0.x, (int)h0.y, (int)h0.z, (int)h0.w};
        const uint8_t* pb = Bs + (wn * 64 + 32 * i + lrow) * kBwStride + ks * 64 + 32 * g;
        const u32x4 l1 = *reinterpret_cast<const u32x4*>(pb), h1 = *reinterpret_cast<const u32x4*>(pb + 16);
        fb[i] = bw_v8i{(int)l1.x, (int)l1.y, (int)l1.z, (int)l1.w, (int)h1.x, (int)h1.y, (int)h1.z, (int)h1.w};
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if (ks == 0) {
            bw_v16f z;
#pragma unroll
            for (int v = 0; v < 16; ++v) z[v] = 0.0f;
            part[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], z, 0, 0, 0, 0, 0, 0);
          } else {
            part[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], part[i][j], 0, 0, 0, 0, 0, 0);
          }
        }
    }
    float ib[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) ib[j] = inv_b[wn * 64 + 32 * j + lrow];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float fa_ = inv_a[wm * 64 + 32 * i + 8 * (v >> 2) + 4 * g + (v & 3)];
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j][v] += part[i][j][v] * (fa_ * ib[j]);
      }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = wm * 64 + 32 * i + 8 * (v >> 2) + 4 * g + (v & 3);
      if (r >= nv) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = wn * 64 + 32 * j + lrow;
        if (c >= kv) continue;
        const int64_t o = ((int64_t)e * p.N + n0 + r) * p.K + k0 + c;
        if constexpr (OUT == 0)
          static_cast<uint16_t*>(p.out)[o] = bw_bf16_rne(acc[i][j][v]);
        else
          static_cast<float*>(p.out)[o] = acc[i][j][v];
      }
    }
}

hipError_t launch_quantize_blockwise_tokens(const uint16_t* x, int64_t M, int64_t C, const int32_t* offs, int n_groups,
                                            int codec, uint8_t* q_t, int64_t ld_q, float* scale, hipStream_t st) {
  if (M == 0 || C == 0) return hipSuccess;
  const int n_strips = (int)((C + 63) / 64);
  const int64_t units = (M + kBwTile - 1) / kBwTile + n_groups;   // bound on the blocks
  const unsigned grid = (unsigned)(units * n_strips);
  if (codec == 0)
    hipLaunchKernelGGL(bw_quant_tokens_kernel<0>, dim3(grid), dim3(256), 0, st, x, (int)M, (int)C, offs, n_groups,
                       q_t, ld_q, scale, n_strips);
  else
    hipLaunchKernelGGL(bw_quant_tokens_kernel<1>, dim3(grid), dim3(256), 0, st, x, (int)M, (int)C, offs, n_groups,
                       q_t, ld_q, scale, n_strips);
  return hipGetLastError();
}

hipError_t launch_grouped_mm_blockwise_k(const uint8_t* a_t, const float* sa, const uint8_t* b_t, const float* sb,
                                         const int32_t* offs, int n_groups, int64_t M, int64_t ld, int64_t N,
                                         int64_t K, void* out, int out_dtype, hipStream_t st) {
  if (N == 0 || K == 0) return hipSuccess;
  BwGemmK p;
  p.a = a_t; p.sa = sa; p.b = b_t; p.sb = sb; p.offs = offs; p.out = out;
  p.E = n_groups; p.M = (int)M; p.N = (int)N; p.K = (int)K; p.ld = ld;
  p.NT = (int)((N + kBwTile - 1) / kBwTile);
  p.KT = (int)((K + kBwTile - 1) / kBwTile);
  const unsigned grid = (unsigned)((int64_t)n_groups * p.NT * p.KT);
  if (out_dtype == 0)
    hipLaunchKernelGGL(bw_gemm_k_kernel<0>, dim3(grid), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL(bw_gemm_k_kernel<1>, dim3(grid), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_quantize_blockwise(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, int block_rows,
                                     int codec, uint8_t* q, float* scale, hipStream_t st) {
  if (batch * rows == 0 || cols == 0) return hipSuccess;
  const int nc = (int)((cols + kBwTile - 1) / kBwTile);
  if (block_rows == 1) {
    const int64_t R = batch * rows;
    const unsigned grid = (unsigned)((R * nc + 15) / 16);
    if (codec == 0)
      hipLaunchKernelGGL(bw_quant_rows_kernel<0>, dim3(grid), dim3(256), 0, st, x, R, (int)cols, nc, q, scale);
    else
      hipLaunchKernelGGL(bw_quant_rows_kernel<1>, dim3(grid), dim3(256), 0, st, x, R, (int)cols, nc, q, scale);
  } else {
    const int nr = (int)((rows + kBwTile - 1) / kBwTile);
    const unsigned grid = (unsigned)(batch * nr * nc);
    if (codec == 0)
      hipLaunchKernelGGL(bw_quant_tiles_kernel<0>, dim3(grid), dim3(256), 0, st, x, (int)rows, (int)cols, nr, nc, q,
                         scale);
    else
      hipLaunchKernelGGL(bw_quant_tiles_kernel<1>, dim3(grid), dim3(256), 0, st, x, (int)rows, (int)cols, nr, nc, q,
                         scale);
  }
  return hipGetLastError();
}

hipError_t launch_grouped_mm_blockwise(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                                       const int32_t* offs, int n_groups, int64_t M, int64_t N, int64_t K, void* out,
                                       int out_dtype, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  BwGemm p;
  p.a = a; p.sa = sa; p.b = b; p.sb = sb; p.offs = offs; p.out = out;
  p.E = n_groups; p.M = (int)M; p.N = (int)N; p.K = (int)K;
  p.KB = (int)((K + kBwTile - 1) / kBwTile);
  p.NB = (int)((N + kBwTile - 1) / kBwTile);
  p.col_tiles = p.NB;
  const int64_t row_units = (M + kBwTile - 1) / kBwTile + n_groups;   // bound on the groups' 128-row tiles
  const unsigned grid = (unsigned)(row_units * p.col_tiles);
  if (out_dtype == 0)
    hipLaunchKernelGGL(bw_gemm_kernel<0>, dim3(grid), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL(bw_gemm_kernel<1>, dim3(grid), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace fp8moe

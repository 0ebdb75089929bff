// Grouped GEMMs on bf16 MFMA for two cases the FP8 kernel does not take.
//  * The "+GW" recipe: the weight-gradient GEMM kept in BF16 on unquantized,
//    token-major operands dY [M][N] and X [M][K] (GROUPED_K, no scales).
//    [P1 Details, Figure 1 "Rowwise FP8 + GW" bar; P3 "Gyorsulás sűrű és
//    MoE-modelleken" (weight update kept in BF16); P4 FAQ on where to start.]
//    gemm_bf16_gw: a persistent kernel; direct global->LDS loads move whole
//    token rows into an LDS ring, and gfx950's transposing LDS read
//    (ds_read_b64_tr_b16) turns the token-major tiles into MFMA fragments
//    that run along the token (contraction) dimension, so no register or VALU
//    transpose is needed.
//  * e4m3fnuz operands.  gfx950's FP8 matrix cores take the OCP formats only,
//    and e4m3fnuz cannot be re-biased into e4m3fn exactly (240 would need 480;
//    odd fnuz subnormals fall between fn subnormals), so fnuz (or mixed) codes
//    are decoded exactly to bf16 on the way into LDS (gemm_bf16_kernel).
//    Correctness path.
#include "device_common.hpp"
#include "gemm_common.hpp"
#include "kernels.hpp"

namespace fp8moe {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

namespace {

constexpr int kStageE = 64;   // contraction elements per stage
constexpr int kBand = 8;

__device__ __forceinline__ int lds_off16(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

__device__ __forceinline__ int xcd_remap16(int bid, int total) {
  const int per = total / 8, rem = total % 8;
  const int x = bid % 8, i = bid / 8;
  return x * per + min(x, rem) + i;
}

// Exact value of an FP8 code as bf16 bits.  e4m3fn: the hardware converter;
// e4m3fnuz: half the e4m3fn value of the same code, except 0x7F/0xFF = +-240
// and 0x80 = NaN.  Every value of both formats is exact in bf16.
template <int CODEC>
__device__ __forceinline__ uint32_t dec_bf16(uint32_t word, int byte) {
  float f;
  switch (byte) {
    case 0: f = __builtin_amdgcn_cvt_f32_fp8((int)word, 0); break;
    case 1: f = __builtin_amdgcn_cvt_f32_fp8((int)word, 1); break;
    case 2: f = __builtin_amdgcn_cvt_f32_fp8((int)word, 2); break;
    default: f = __builtin_amdgcn_cvt_f32_fp8((int)word, 3); break;
  }
  if constexpr (CODEC == 1) {
    const uint32_t c = (word >> (8 * byte)) & 0xFFu;
    f *= 0.5f;
    if ((c & 0x7Fu) == 0x7Fu) f = (c & 0x80u) ? -240.0f : 240.0f;
    if (c == 0x80u) f = __uint_as_float(0x7FC00000u);
  }
  return __float_as_uint(f) >> 16;
}

// 16 codes -> 16 bf16 (two 16-byte chunks)
template <int CODEC>
__device__ __forceinline__ void dec16(const u32x4& v, u32x4& lo, u32x4& hi) {
  uint32_t o[8];
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = dec_bf16<CODEC>(w[i], 0) | (dec_bf16<CODEC>(w[i], 1) << 16);
    o[2 * i + 1] = dec_bf16<CODEC>(w[i], 2) | (dec_bf16<CODEC>(w[i], 3) << 16);
  }
  lo = u32x4{o[0], o[1], o[2], o[3]};
  hi = u32x4{o[4], o[5], o[6], o[7]};
}

__device__ __forceinline__ u32x4 mask_bytes(u32x4 v, int pos, int lo, int hi) {
  const int s = lo - pos, e = hi - pos;
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int a = min(max(s - 4 * i, 0), 4), b = min(max(e - 4 * i, 0), 4);
    const uint32_t keep_hi = b >= 4 ? 0xFFFFFFFFu : ((1u << (8 * b)) - 1u);
    const uint32_t drop_lo = a >= 4 ? 0xFFFFFFFFu : ((1u << (8 * a)) - 1u);
    w[i] &= keep_hi & ~drop_lo;
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

// 8x8 transpose of 16-bit values: in[r] holds row r (8 values), out[c] column c.
__device__ __forceinline__ void transpose8x8(const u32x4 in[8], u32x4 out[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const u32x4& r0 = in[2 * p];
      const u32x4& r1 = in[2 * p + 1];
      const uint32_t a = (c >> 1) == 0 ? r0.x : (c >> 1) == 1 ? r0.y : (c >> 1) == 2 ? r0.z : r0.w;
      const uint32_t b = (c >> 1) == 0 ? r1.x : (c >> 1) == 1 ? r1.y : (c >> 1) == 2 ? r1.z : r1.w;
      // low half <- value c of row 2p, high half <- value c of row 2p+1
      w[p] = (c & 1) ? __builtin_amdgcn_perm(b, a, 0x07060302u) : __builtin_amdgcn_perm(b, a, 0x05040100u);
    }
    out[c] = u32x4{w[0], w[1], w[2], w[3]};
  }
}

__device__ __forceinline__ uint16_t to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

struct BParams {
  const void* a;
  const void* b;
  const float* sa;
  const float* sb;
  const int32_t* offs;
  void* out;
  int E, M, N, K;
  int row_units, col_tiles;
};

}  // namespace

// SRC 0: FP8 codes, contraction-contiguous (codecs CA/CB), fp32 scales.
// SRC 1: bf16 token-major operands, GROUPED_K only, no scales.
template <int MODE, int SRC, int CA, int CB, int OUT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_kernel(BParams p) {
  constexpr int BM = 256, BN = 256, WM = 128, WN = 128, TM = 4, TN = 4;
  constexpr int A_BYTES = BM * 128, STAGE = (BM + BN) * 128;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int total = gridDim.x;
  const int L = xcd_remap16(blockIdx.x, total);
  const int band = L / (kBand * p.col_tiles);
  const int first = band * kBand;
  const int gsz = min(p.row_units - first, kBand);
  const int inband = L % (kBand * p.col_tiles);
  const int ru = first + inband % gsz;
  const int ct = inband / gsz;

  int p_valid, q_valid, c_lo, c_hi;
  int64_t out_base, out_ld;
  const float* psf = nullptr;
  const float* qsf = nullptr;
  const uint8_t* P8 = nullptr;
  const uint8_t* Q8 = nullptr;
  int64_t ld8 = 0;
  const uint16_t* PT = nullptr;   // token-major bf16: element (m, row) at PT[m * ldT + row]
  const uint16_t* QT = nullptr;
  int64_t ldPT = 0, ldQT = 0;
  if constexpr (MODE == 0) {
    struct Ch {
      __device__ int operator()(int lo, int hi) const { return (hi - lo + BM - 1) / BM; }
    };
    struct NoPad {
      __device__ int operator()(int, int) const { return 0; }
    };
    const Unit un = find_unit<256>(p.offs, p.E, p.M, ru, Ch{}, NoPad{});
    if (un.e < 0) return;
    const int m0 = un.lo + un.j * BM, n0 = ct * BN;
    p_valid = min(BM, un.hi - m0);
    q_valid = min(BN, p.N - n0);
    P8 = static_cast<const uint8_t*>(p.a) + (int64_t)m0 * p.K;
    Q8 = static_cast<const uint8_t*>(p.b) + ((int64_t)un.e * p.N + n0) * p.K;
    ld8 = p.K;
    c_lo = 0;
    c_hi = p.K;
    out_ld = p.N;
    out_base = (int64_t)m0 * p.N + n0;
    psf = p.sa + m0;
    qsf = p.sb + (int64_t)un.e * p.N + n0;
  } else {
    const int ntn = (p.N + BM - 1) / BM;
    const int e = ru / ntn;
    const int n0 = (ru % ntn) * BM, k0 = ct * BN;
    __shared__ int s_red[4];
    int m = 0;
    if (p.offs != nullptr)
      for (int jj = t; jj < e; jj += 256) m = max(m, clamp_off(p.offs[jj], p.M));
    m = (int)wave_max_u32((uint32_t)m);
    if (lane == 0) s_red[wave] = m;
    __syncthreads();
    const int lo = max(max(s_red[0], s_red[1]), max(s_red[2], s_red[3]));
    const int hi = p.offs != nullptr ? max(lo, clamp_off(p.offs[e], p.M)) : p.M;
    p_valid = min(BM, p.N - n0);
    q_valid = min(BN, p.K - k0);
    c_lo = lo;
    c_hi = hi;
    out_ld = p.K;
    out_base = ((int64_t)e * p.N + n0) * p.K + k0;
    if constexpr (SRC == 0) {
      P8 = static_cast<const uint8_t*>(p.a) + (int64_t)n0 * p.M;
      Q8 = static_cast<const uint8_t*>(p.b) + (int64_t)k0 * p.M;
      ld8 = p.M;
      psf = p.sa + (int64_t)e * p.N + n0;
      qsf = p.sb + (int64_t)e * p.K + k0;
    } else {
      PT = static_cast<const uint16_t*>(p.a) + n0;
      QT = static_cast<const uint16_t*>(p.b) + k0;
      ldPT = p.N;
      ldQT = p.K;
    }
  }

  const int c_start = SRC == 0 ? (c_lo & ~15) : c_lo;
  const int nk = c_hi > c_lo ? (c_hi - c_start + kStageE - 1) / kStageE : 0;

  // SRC 0: thread t loads 16 codes (chunk t&3 of 64) of rows (t>>2) + 64*i -> 2 LDS chunks each.
  // SRC 1: thread t loads an 8 (tokens) x 8 (rows) block: token block t&7, row block t>>3.
  constexpr int NL = SRC == 0 ? 4 : 8;
  u32x4 ra[NL], rb[NL];

  auto load_stage = [&](int kt) {
    const int base = c_start + kt * kStageE;
    if constexpr (SRC == 0) {
      const int pos = base + 16 * (t & 3);
      const bool in = pos < c_hi;
      const bool partial = in && (pos < c_lo || pos + 16 > c_hi);
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int r = (t >> 2) + 64 * i;
        const int rp = min(r, p_valid - 1), rq = min(r, q_valid - 1);
        ra[i] = in ? *reinterpret_cast<const u32x4*>(P8 + rp * ld8 + pos) : u32x4{0, 0, 0, 0};
        rb[i] = in ? *reinterpret_cast<const u32x4*>(Q8 + rq * ld8 + pos) : u32x4{0, 0, 0, 0};
        if (partial) {
          ra[i] = mask_bytes(ra[i], pos, c_lo, c_hi);
          rb[i] = mask_bytes(rb[i], pos, c_lo, c_hi);
        }
      }
    } else {
      const int m0 = base + 8 * (t & 7);
      const int r0 = 8 * (t >> 3);   // 32 row blocks of 8 -> 256 rows
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int m = m0 + i;
        const bool ok = m < c_hi;   // row blocks are whole: N, K are multiples of 8, tiles start at multiples of 256
        ra[i] = (ok && r0 < p_valid) ? *reinterpret_cast<const u32x4*>(PT + (int64_t)m * ldPT + r0) : u32x4{0, 0, 0, 0};
        rb[i] = (ok && r0 < q_valid) ? *reinterpret_cast<const u32x4*>(QT + (int64_t)m * ldQT + r0) : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_stage = [&](int buf) {
    uint8_t* sa_ = smem + buf * STAGE;
    uint8_t* sb_ = sa_ + A_BYTES;
    if constexpr (SRC == 0) {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int r = (t >> 2) + 64 * i, c = 2 * (t & 3);
        u32x4 lo, hi;
        dec16<CA>(ra[i], lo, hi);
        *reinterpret_cast<u32x4*>(sa_ + lds_off16(r, c)) = lo;
        *reinterpret_cast<u32x4*>(sa_ + lds_off16(r, c + 1)) = hi;
        dec16<CB>(rb[i], lo, hi);
        *reinterpret_cast<u32x4*>(sb_ + lds_off16(r, c)) = lo;
        *reinterpret_cast<u32x4*>(sb_ + lds_off16(r, c + 1)) = hi;
      }
    } else {
      u32x4 ta[8], tb[8];
      transpose8x8(ra, ta);
      transpose8x8(rb, tb);
      const int r0 = 8 * (t >> 3), c = t & 7;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        *reinterpret_cast<u32x4*>(sa_ + lds_off16(r0 + i, c)) = ta[i];
        *reinterpret_cast<u32x4*>(sb_ + lds_off16(r0 + i, c)) = tb[i];
      }
    }
  };

  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int g = lane >> 5, lrow = lane & 31;
  if (nk > 0) {
    load_stage(0);
    store_stage(0);
    __syncthreads();
  }
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_stage(kt + 1);
    const uint8_t* sa_ = smem + buf * STAGE;
    const uint8_t* sb_ = sa_ + A_BYTES;
#pragma unroll
    for (int s = 0; s < 4; ++s) {   // 4 MFMA steps of 16 elements
      v8bf af[TM], bf[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(sa_ + lds_off16(wm * WM + 32 * i + lrow, 2 * s + g));
        af[i] = __builtin_bit_cast(v8bf, v);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(sb_ + lds_off16(wn * WN + 32 * j + lrow, 2 * s + g));
        bf[j] = __builtin_bit_cast(v8bf, v);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_stage(buf ^ 1);
    __syncthreads();
  }

  const bool empty = c_hi <= c_lo;
  float inv_q[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int cidx = min(wn * WN + 32 * j + lrow, q_valid - 1);
    inv_q[j] = SRC == 0 ? __frcp_rn(qsf[cidx]) : 1.0f;
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = wm * WM + 32 * i + 8 * (v >> 2) + 4 * g + (v & 3);
      if (r >= p_valid) continue;
      const float inv_p = SRC == 0 ? __frcp_rn(psf[r]) : 1.0f;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int c = wn * WN + 32 * j + lrow;
        if (c >= q_valid) continue;
        const float val = empty ? 0.0f : acc[i][j][v] * inv_p * inv_q[j];
        const int64_t o = out_base + (int64_t)r * out_ld + c;
        if constexpr (OUT == 0)
          static_cast<uint16_t*>(p.out)[o] = to_bf16_rne(val);
        else
          static_cast<float*>(p.out)[o] = val;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// "+GW": dW[e][n][k] = sum over tokens m of group e of dY[m][n] * X[m][k].
//
// Tiles of 256 (n) x 256 (k) outputs, 2 x 2 waves of 128 x 128, walked by a
// persistent grid (one workgroup per CU) in the FP8 kernel's XCD-banded order.
// A stage is 64 tokens of both operands: per operand 64 token rows x 512 bytes
// (256 bf16), 32 KiB, so a stage is 64 KiB and the ring holds two.
//
// LDS layout of an operand: token row t at t * 512 bytes; its 16-byte chunk c
// (tile rows 8c .. 8c+7) sits at physical chunk c ^ ((t & 3) << 2).  A wave's
// direct load fills 1 KiB (two token rows) contiguously, each lane fetching
// the global chunk that belongs at its slot.
//
// Fragments: v_mfma_f32_32x32x16_bf16 wants, per lane, 8 bf16 of one tile row
// along the contraction: lane l holds row l & 31 at k slots 8 (l >> 5) .. +7.
// ds_read_b64_tr_b16 works on groups of 16 lanes: output lane 4q + p receives
// element p of the 8-byte chunks addressed by source lanes q, q+4, q+8, q+12
// (checked on gfx950).  So source lane 4e + q of group g points at token
// t0 + e, rows 16 g + 4q .. +3; output lane i then holds row 16 g + i at tokens
// t0 .. t0+3.  Two such reads give a fragment's 8 tokens.  Both operands use
// the same token -> k-slot map, so every product pairs the same token.  Per
// read instruction the 64 lanes touch 8 token rows x 64 bytes; the swizzle puts
// the four tokens of a group on distinct bank groups (two cycles for 512 B).
//
// Group bounds: the contraction of group e is tokens [lo(e), hi(e)) (running
// maximum of the clamped offsets).  Stages start at lo(e); for token rows past
// hi(e) the dY row comes from a row of zeros in device memory and the X row
// from token hi(e)-1 (in bounds, finite), so those tokens add exact zeros.  Tile
// rows past N (or K) load the last valid 16-byte chunk and are never stored.
typedef float f32x2_gw __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_gw __attribute__((ext_vector_type(2)));

struct GwParams {
  const uint16_t* dy;   // [M][N] bf16
  const uint16_t* x;    // [M][K] bf16
  const int32_t* offs;
  void* out;            // [E][N][K]
  int E, M, N, K;
  int row_units;        // E * ceil(N / 256)
  int col_tiles;        // ceil(K / 256)
};

constexpr int kGwTile = 256, kGwStage = 64;   // tile edge, tokens per stage
constexpr int kGwOp = kGwStage * kGwTile * 2;  // bytes of one operand in one stage (32 KiB)

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f_gw __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int gw_phys(int t, int c) { return c ^ ((t & 3) << 2); }

// One token row of zeros (a tile row's 256 bf16): the source of dY rows of
// tokens past a group's end, so they add exact zeros with no masking in the
// k loop.  Never written.
__device__ __attribute__((aligned(16))) uint16_t g_gw_zero_row[kGwTile];

__device__ __forceinline__ v4s tr_read(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s*)((__attribute__((address_space(3))) uint8_t*)(p)));
}

template <int OUT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_gw(GwParams p) {
  constexpr int TM = 4, TN = 4, WM = 128, WN = 128, KS = kGwStage / 16;   // KS k steps of 16 tokens per stage
  static_assert(KS % 2 == 0, "fragment sets alternate k step by k step and stay aligned to stages");
  __shared__ __attribute__((aligned(1024))) uint8_t ring0[2 * kGwOp];
  __shared__ __attribute__((aligned(1024))) uint8_t ring1[2 * kGwOp];
  auto slot = [](int s) -> uint8_t* { return (s & 1) == 0 ? ring0 : ring1; };

  // group table: g_hi[e] = hi(e) (running maximum of the clamped offsets)
  constexpr int kTable = 256;
  __shared__ int g_hi[kTable];
  __shared__ int s_tmp[4];
  const bool table = p.E <= kTable;
  {
    const int t = threadIdx.x;
    const int v = t < p.E ? clamp_off(p.offs[t], p.M) : 0;
    const int hi = block_scan_max<256>(v, s_tmp);
    if (table && t < p.E) g_hi[t] = hi;
    __syncthreads();
  }
  const int ntiles = p.row_units * p.col_tiles;
  const int G = gridDim.x;
  const int ntn = (p.N + kGwTile - 1) / kGwTile;
  auto tile_of = [&](int it) {
    return (G & 7) == 0 ? G * it + (G >> 3) * (blockIdx.x & 7) + (blockIdx.x >> 3) : G * it + blockIdx.x;
  };

  struct Tile {
    int e, n0, k0, lo, hi, pv, qv, nk;
  };
  // Every thread calls it (without a group table it synchronizes the workgroup).
  auto setup = [&](int L, Tile& tl) {
    // logical tile -> (row unit, column tile) in bands of 8 row units
    const int band = L / (8 * p.col_tiles);
    const int first = band * 8;
    const int gsz = min(p.row_units - first, 8);
    const int inband = L - band * 8 * p.col_tiles;
    const int ru = first + inband % gsz, ct = inband / gsz;
    tl.e = ru / ntn;
    tl.n0 = (ru % ntn) * kGwTile;
    tl.k0 = ct * kGwTile;
    int lo, hi;
    if (table) {
      lo = tl.e == 0 ? 0 : g_hi[tl.e - 1];
      hi = g_hi[tl.e];
    } else {
      int m = 0;
      for (int j = threadIdx.x; j < tl.e; j += 256) m = max(m, clamp_off(p.offs[j], p.M));
      m = (int)wave_max_u32((uint32_t)m);
      if ((threadIdx.x & 63) == 0) s_tmp[threadIdx.x >> 6] = m;
      __syncthreads();
      lo = max(max(s_tmp[0], s_tmp[1]), max(s_tmp[2], s_tmp[3]));
      hi = max(lo, clamp_off(p.offs[tl.e], p.M));
      __syncthreads();
    }
    tl.lo = __builtin_amdgcn_readfirstlane(lo);
    tl.hi = __builtin_amdgcn_readfirstlane(hi);
    tl.e = __builtin_amdgcn_readfirstlane(tl.e);
    tl.n0 = __builtin_amdgcn_readfirstlane(tl.n0);
    tl.k0 = __builtin_amdgcn_readfirstlane(tl.k0);
    tl.pv = min(kGwTile, p.N - tl.n0);
    tl.qv = min(kGwTile, p.K - tl.k0);
    tl.nk = (tl.hi - tl.lo + kGwStage - 1) / kGwStage;
  };

  // Stage s of tile tl into LDS `sl`: wave w moves 1 KiB blocks w + 4 i (i < 16)
  // of the 64 KiB stage; blocks 0..31 (i < 8) are dY, token rows 8 i + 2 w + (lane >> 5),
  // blocks 32..63 (i >= 8) X, token rows 8 (i - 8) + 2 w + (lane >> 5).  A lane's byte
  // offset from its operand's row of the stage's first token is the same for every
  // i (the swizzle depends on the token only through t & 3) and every stage, so a
  // whole stage is a uniform base per load plus one per-lane offset per operand;
  // a stage reaching past the group end (the tile's last) takes the checked path,
  // which clamps the X rows to token hi - 1 and reads the dY rows from a row of zeros.
  struct LaneOff {
    uint32_t y, x;   // byte offsets of this lane's chunk from token row 2 w + (lane >> 5)
  };
  auto lane_offsets = [&](const Tile& tl) {
    int t_opq = threadIdx.x;
    asm volatile("" : "+v"(t_opq));
    const int lane = t_opq & 63, wave = __builtin_amdgcn_readfirstlane(t_opq >> 6);
    const int t = 2 * wave + (lane >> 5), pc = lane & 31;
    const int cy = min(gw_phys(t, pc), (tl.pv - 1) >> 3), cx = min(gw_phys(t, pc), (tl.qv - 1) >> 3);
    return LaneOff{(uint32_t)(t * p.N * 2 + 16 * cy), (uint32_t)(t * p.K * 2 + 16 * cx)};
  };
  auto issue = [&](const Tile& tl, const LaneOff& lo_, int s, uint8_t* sl) {
    int t_opq = threadIdx.x;
    asm volatile("" : "+v"(t_opq));
    const int lane = t_opq & 63, wave = __builtin_amdgcn_readfirstlane(t_opq >> 6);
    const int tok0 = tl.lo + s * kGwStage;   // uniform
    if (tok0 + kGwStage <= tl.hi) {
      const uint8_t* ybase = reinterpret_cast<const uint8_t*>(p.dy + (int64_t)tok0 * p.N + tl.n0);
      const uint8_t* xbase = reinterpret_cast<const uint8_t*>(p.x + (int64_t)tok0 * p.K + tl.k0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint8_t* b = i < 8 ? ybase + (int64_t)(8 * i) * p.N * 2 : xbase + (int64_t)(8 * (i - 8)) * p.K * 2;
        dma_16(b + (i < 8 ? lo_.y : lo_.x), sl + (wave + 4 * i) * 1024);
      }
      return;
    }
    const int tl2 = lane >> 5, pc = lane & 31;
    const int cmax_p = (tl.pv - 1) >> 3, cmax_q = (tl.qv - 1) >> 3;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int blk = wave + 4 * i;
      const bool is_x = i >= 8;
      const int t = 2 * (blk & 31) + tl2;                      // token row within the stage
      const int tok_u = tok0 + t;
      const int tok = min(tok_u, tl.hi - 1);
      const int c = min(gw_phys(t, pc), is_x ? cmax_q : cmax_p);   // logical chunk (the swizzle is an involution)
      const uint16_t* src = is_x ? p.x + (int64_t)tok * p.K + tl.k0 + 8 * c
                                 : (tok_u < tl.hi ? p.dy + (int64_t)tok * p.N + tl.n0 + 8 * c : g_gw_zero_row + 8 * c);
      dma_16(reinterpret_cast<const uint8_t*>(src), sl + blk * 1024);
    }
  };

  Tile cur, nxt;
  if (tile_of(0) >= ntiles) return;
  setup(tile_of(0), cur);
  LaneOff lcur = lane_offsets(cur), lnxt;
  if (cur.nk > 0) {
    issue(cur, lcur, 0, ring0);
    issue(cur, lcur, min(1, cur.nk - 1), ring1);
  }

  for (int it = 0;; ++it) {
    int t_opq = threadIdx.x;
    asm volatile("" : "+v"(t_opq));
    const int lane = t_opq & 63, wave = __builtin_amdgcn_readfirstlane(t_opq >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int nk = cur.nk;
    const bool has_next = tile_of(it + 1) < ntiles;

    // fragment addressing (see the header): source lane 4e + q of group g
    const int h = lane >> 5, grp = (lane >> 4) & 1, ee = (lane >> 2) & 3, qq = lane & 3;
    auto frag = [&](const uint8_t* op, int row0, int tok0) -> v8bf {
      const int row = row0 + 16 * grp + 4 * qq;                 // 4 rows = 8 bytes
      const int t0 = tok0 + 8 * h + ee, t1 = t0 + 4;             // this lane's source tokens
      const int cb = row >> 3, wb = (row & 7) * 2;
      const v4s r0 = tr_read(op + t0 * 512 + (gw_phys(t0, cb) << 4) + wb);
      const v4s r1 = tr_read(op + t1 * 512 + (gw_phys(t1, cb) << 4) + wb);
      return __builtin_bit_cast(v8bf, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    v8bf fa[2][TM], fb[2][TN];
    auto rd = [&](auto set_tag, const uint8_t* sl, int ks) {
      constexpr int SET = decltype(set_tag)::value;
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[SET][i] = frag(sl, wm * WM + 32 * i, 16 * ks);
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[SET][j] = frag(sl + kGwOp, wn * WN + 32 * j, 16 * ks);
    };
    v16f_gw acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    auto mma = [&](auto set_tag) {
      constexpr int SET = decltype(set_tag)::value;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)   // X fragment first: a lane holds 4 consecutive output columns per quad
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[SET][j], fa[SET][i], acc[i][j], 0, 0, 0);
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    constexpr int ND = 2 * (TM + TN);   // transposing LDS reads per k step

    // ---- start: stages 0 and 1 are in flight (stage 0 into slot 0; for later
    // tiles it landed during the previous epilogue).
    if (nk > 0) {
      if (it == 0) {                    // later tiles: stage 0 landed in the previous epilogue
        if (nk > 1) wait_vmcnt<16>();
        else wait_vmcnt<0>();
        raw_barrier();
      }
      rd(S0{}, ring0, 0);
    }
    // The next tile's description (its loads are issued before the epilogue).
    if (has_next) {
      setup(tile_of(it + 1), nxt);
      lnxt = lane_offsets(nxt);
    }

    // ---- k loop.  Stage s sits in slot s & 1.  Its first KS-1 k steps read the
    // next k step's fragments while the current one's MFMAs issue; then (all of
    // this wave's reads of the slot done, stage s+1 landed) one barrier, the
    // refill of the slot with stage s+2, the first fragments of stage s+1, and
    // the last k step's MFMAs, with the loads and reads spread between them.
    // The step is branch-free: past the end it reloads the last stage and reads
    // fragments nothing uses.
    for (int s = 0; s < nk; ++s) {
      uint8_t* sl = slot(s);
#pragma unroll
      for (int ks = 0; ks + 1 < KS; ks += 2) {
        rd(S1{}, sl, ks + 1);
        mma(S0{});
        interleave<TM * TN, ND, 0>();
        __builtin_amdgcn_sched_barrier(0);
        if (ks + 2 < KS) {
          rd(S0{}, sl, ks + 2);
          mma(S1{});
          interleave<TM * TN, ND, 0>();
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      wait_lgkmcnt0();
      wait_vmcnt<0>();                   // stage s+1 (the only loads in flight)
      raw_barrier();
      issue(cur, lcur, min(s + 2, nk - 1), sl);
      rd(S0{}, slot(s + 1), 0);
      mma(S1{});
      interleave<TM * TN, ND, 16>();
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vmcnt<0>();                     // the reloads past the end land before their slots are reused

    // ---- next tile's stage 0 into slot 0 (lands during the epilogue, which
    // stages through slot 1).
    wait_lgkmcnt0();
    raw_barrier();
    if (has_next && nxt.nk > 0) issue(nxt, lnxt, 0, ring0);

    // ---- epilogue: each wave's 32-row blocks through slot 1, written as whole
    // 16-byte pieces of output rows (unit u of staged row r at u ^ (r & 31), as in
    // the FP8 kernel: 8-byte units for bf16, 16-byte units for fp32).
    constexpr int ELEM = OUT == 0 ? 2 : 4;
    constexpr int RB = WN * ELEM;               // staged row bytes
    constexpr int NCH = RB / 16, VEC = 16 / ELEM, RPI = 64 / NCH;
    constexpr int TMP = OUT == 0 ? 2 : 1;       // 32-row blocks per pass (16 KiB per wave)
    uint8_t* const stg = ring1 + wave * (TMP * 32 * RB);
    const int g = lane >> 5, lrow = lane & 31;
    const int64_t out_ld = p.K;
    const int64_t out_base = ((int64_t)cur.e * p.N + cur.n0) * p.K + cur.k0;
    const int pv = cur.pv, qv = cur.qv;
#pragma unroll
    for (int pass = 0; pass < TM / TMP; ++pass) {
      if (pass > 0) wait_lgkmcnt0();
#pragma unroll
      for (int ii = 0; ii < TMP; ++ii) {
        const int i = pass * TMP + ii, lr = 32 * ii + lrow;
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int u = 8 * j + 2 * q + g;
            const float* a4 = reinterpret_cast<const float*>(&acc[i][j]) + 4 * q;
            if constexpr (OUT == 0) {   // round to nearest even (the hardware conversion)
              const bf16x2_gw lo2 = __builtin_convertvector(f32x2_gw{a4[0], a4[1]}, bf16x2_gw);
              const bf16x2_gw hi2 = __builtin_convertvector(f32x2_gw{a4[2], a4[3]}, bf16x2_gw);
              *reinterpret_cast<u32x2*>(stg + lr * RB + ((u ^ (lr & 31)) << 3)) =
                  u32x2{__builtin_bit_cast(uint32_t, lo2), __builtin_bit_cast(uint32_t, hi2)};
            } else {
              *reinterpret_cast<u32x4*>(stg + lr * RB + ((u ^ (lr & 31)) << 4)) =
                  u32x4{__float_as_uint(a4[0]), __float_as_uint(a4[1]), __float_as_uint(a4[2]), __float_as_uint(a4[3])};
            }
          }
      }
      wait_lgkmcnt0();
      if (pass == 0) wait_vmcnt<0>();   // the next tile's stage 0 (older than any store below)
      const int k = lane % NCH, c = wn * WN + k * VEC;
#pragma unroll
      for (int itr = 0; itr < TMP * 32 / RPI; ++itr) {
        const int lr = itr * RPI + lane / NCH;
        const int pc = OUT == 0 ? (k ^ ((lr & 31) >> 1)) : (k ^ (lr & 31));
        u32x4 d = *reinterpret_cast<const u32x4*>(stg + lr * RB + (pc << 4));
        if (OUT == 0 && (lr & 1)) d = u32x4{d.z, d.w, d.x, d.y};
        const int r = wm * WM + pass * TMP * 32 + lr;
        if (r < pv && c < qv)
          store_stream16(static_cast<uint8_t*>(p.out) + (out_base + (int64_t)r * out_ld + c) * ELEM, d);
      }
    }
    if (!has_next) break;
    wait_lgkmcnt0();
    raw_barrier();                          // slot 1 is free: the next tile's stage 1
    cur = nxt;
    lcur = lnxt;
    if (cur.nk > 1) issue(cur, lcur, 1, ring1);
  }
}

template <int OUT>
static hipError_t launch_gw(const GemmArgs& g, hipStream_t st) {
  GwParams p;
  p.dy = static_cast<const uint16_t*>(g.a);
  p.x = static_cast<const uint16_t*>(g.b);
  p.offs = g.offs;
  p.out = g.out;
  p.E = g.n_groups;
  p.M = (int)g.M;
  p.N = (int)g.N;
  p.K = (int)g.K;
  p.row_units = (int)(g.n_groups * ((g.N + kGwTile - 1) / kGwTile));
  p.col_tiles = (int)((g.K + kGwTile - 1) / kGwTile);
  const int64_t total = (int64_t)p.row_units * p.col_tiles;
  if (total == 0) return hipSuccess;
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  const int64_t grid = std::min<int64_t>(total, cus[dev]);
  hipLaunchKernelGGL((gemm_bf16_gw<OUT>), dim3((unsigned)grid), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <int MODE, int SRC, int CA, int CB, int OUT>
static hipError_t launch_b(const GemmArgs& g, hipStream_t st) {
  BParams p;
  p.a = g.a;
  p.b = g.b;
  p.sa = static_cast<const float*>(g.sa);
  p.sb = static_cast<const float*>(g.sb);
  p.offs = g.offs;
  p.out = g.out;
  p.E = g.n_groups;
  p.M = (int)g.M;
  p.N = (int)g.N;
  p.K = (int)g.K;
  if (MODE == 0) {
    p.row_units = (int)((g.M + 255) / 256 + g.n_groups);
    p.col_tiles = (int)((g.N + 255) / 256);
  } else {
    p.row_units = (int)(g.n_groups * ((g.N + 255) / 256));
    p.col_tiles = (int)((g.K + 255) / 256);
  }
  const int64_t total = (int64_t)p.row_units * p.col_tiles;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_bf16_kernel<MODE, SRC, CA, CB, OUT>), dim3((unsigned)total), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <int MODE, int OUT>
static hipError_t codecs(const GemmArgs& g, hipStream_t st) {
  if (g.a_fmt == 0 && g.b_fmt == 1) return launch_b<MODE, 0, 0, 1, OUT>(g, st);
  if (g.a_fmt == 1 && g.b_fmt == 0) return launch_b<MODE, 0, 1, 0, OUT>(g, st);
  return launch_b<MODE, 0, 1, 1, OUT>(g, st);
}

hipError_t launch_grouped_mm_bf16(const GemmArgs& g, hipStream_t st) {
  if (g.mode == 0 && g.M == 0) return hipSuccess;
  if (g.a_fmt == 2) {   // bf16 "+GW" wgrad (validated: GROUPED_K, no scales)
    return g.out_dtype == 0 ? launch_gw<0>(g, st) : launch_gw<1>(g, st);
  }
  if (g.mode == 0) return g.out_dtype == 0 ? codecs<0, 0>(g, st) : codecs<0, 1>(g, st);
  return g.out_dtype == 0 ? codecs<1, 0>(g, st) : codecs<1, 1>(g, st);
}

}  // namespace fp8moe

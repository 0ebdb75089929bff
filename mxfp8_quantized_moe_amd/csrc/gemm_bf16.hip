// Grouped GEMM on bf16 MFMA (v_mfma_f32_32x32x16_bf16) for two cases the FP8
// kernel does not take:
//  * the "+GW" recipe: the weight-gradient GEMM kept in BF16 on unquantized,
//    token-major operands dY [M][N] and X [M][K] (GROUPED_K, no scales).
//    [P1 Details, Figure 1 "Rowwise FP8 + GW" bar; P3 "Gyorsulás sűrű és
//    MoE-modelleken" (weight update kept in BF16); P4 FAQ on where to start.]
//  * e4m3fnuz operands.  gfx950's FP8 matrix cores take the OCP formats only,
//    and e4m3fnuz cannot be re-biased into e4m3fn exactly (240 would need 480;
//    odd fnuz subnormals fall between fn subnormals), so fnuz (or mixed) codes
//    are decoded exactly to bf16 on the way into LDS.  Correctness path.
// Same tile shape, LDS layout and tile order as the FP8 kernel; a stage holds
// 64 contraction elements (128 B of bf16) per tile row.
#include "device_common.hpp"
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
    return g.out_dtype == 0 ? launch_b<1, 1, 0, 0, 0>(g, st) : launch_b<1, 1, 0, 0, 1>(g, st);
  }
  if (g.mode == 0) return g.out_dtype == 0 ? codecs<0, 0>(g, st) : codecs<0, 1>(g, st);
  return g.out_dtype == 0 ? codecs<1, 0>(g, st) : codecs<1, 1>(g, st);
}

}  // namespace fp8moe

// Device-side building blocks shared by the quantization and GEMM kernels:
// the FP8 / e8m0 codec, bf16 unpacking, wave64 reductions and the device-side
// group-bounds rule.  gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8moe {

// ------------------------------------------------------------------ constants

// Largest finite magnitudes: e4m3fnuz 240 (the pages' e4m3fnuz property table),
// e4m3fn 448 (OCP 8-bit float).  [P1 Details; P4 "Тихая порча градиентов".]
__host__ __device__ constexpr float fmax_of(int codec) { return codec == 0 ? 448.0f : 240.0f; }

// Floor under the absolute maximum before the division, so an all-zero or
// empty reduction set still gets a finite scale (fmax / 1e-12).
constexpr float kAmaxFloor = 1e-12f;

struct alignas(16) u32x4 { uint32_t x, y, z, w; };
struct alignas(8) u32x2 { uint32_t x, y; };

// ------------------------------------------------------------------ bf16

__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xFFFF0000u); }

// Eight packed bf16 values times w: each product one fp32 operation, rounded to
// bf16 (nearest even) -- the combine backward's routed-row gradient w * dy.
typedef float dc_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 dc_bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_times(uint32_t v, float w) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(dc_f32x2{w * bf16_lo(v), w * bf16_hi(v)}, dc_bf16x2));
}
__device__ __forceinline__ u32x4 bf16x8_times(const u32x4& v, float w) {
  return u32x4{bf16x2_times(v.x, w), bf16x2_times(v.y, w), bf16x2_times(v.z, w), bf16x2_times(v.w, w)};
}

// Row r of a tensor of `cols` bf16 columns, 8 columns from `col`: x row r, or
// (gathered into moe_route's grouped layout, src non-null) token row
// src[r] / topk of x, times the slot's router weight w[src[r]] when w is
// non-null, and zeros for a row whose slot is < 0 or >= slots.
struct RowSrc {
  const uint16_t* x;
  const int32_t* src;
  const float* w;
  int topk;
  int64_t slots;
};
template <bool GATHER>
__device__ __forceinline__ u32x4 row_load8(const RowSrc& s, int64_t r, int64_t cols, int col) {
  if constexpr (!GATHER) {
    return *reinterpret_cast<const u32x4*>(s.x + r * cols + col);
  } else {
    const int sl = s.src[r];
    if (sl < 0 || (int64_t)sl >= s.slots) return u32x4{0, 0, 0, 0};
    const u32x4 v = *reinterpret_cast<const u32x4*>(s.x + (int64_t)(sl / s.topk) * cols + col);
    return s.w != nullptr ? bf16x8_times(v, s.w[sl]) : v;
  }
}

// Two independent 16-bit maxima packed in a u32 (v_pk_max_u16: one instruction).
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}

// max(|a|,|b|) over each 16-bit half of two packed bf16 pairs, as magnitudes
// compared by their bit patterns (valid for finite values: a larger bf16
// magnitude has a larger 15-bit pattern).
__device__ __forceinline__ uint32_t pk_absmax_bf16(uint32_t acc, uint32_t v) {
  return pk_max_u16(acc, v & 0x7FFF7FFFu);
}
__device__ __forceinline__ uint32_t pk_fold(uint32_t acc) { return max(acc & 0xFFFFu, acc >> 16); }

// ------------------------------------------------------------------ reductions
//
// Lane exchanges on the VALU instead of the LDS crossbar (no LDS wait): lane l
// meets lane l ^ 8 by a DPP rotation of its 16-lane row by 8, lane l ^ 16 and
// l ^ 32 by gfx950's row swaps (v_permlane16_swap / v_permlane32_swap: the two
// results hold, in every lane, the values of l and of its partner), and l ^ 1,
// l ^ 2 by DPP quad permutations.

// max over lanes {l, l ^ X} for X in {1, 2, 8, 16, 32}, unsigned 32-bit or packed 16-bit.
template <int X, bool PK16>
__device__ __forceinline__ uint32_t lane_max_xor(uint32_t v) {
  auto mx = [](uint32_t a, uint32_t b) { return PK16 ? pk_max_u16(a, b) : max(a, b); };
  if constexpr (X == 1) {
    return mx(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  } else if constexpr (X == 2) {
    return mx(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  } else if constexpr (X == 8) {
    return mx(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false));  // row_ror:8
  } else if constexpr (X == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return mx(p[0], p[1]);
  } else {
    static_assert(X == 32, "lane distance");
    const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return mx(p[0], p[1]);
  }
}

// Unsigned maximum over aligned groups of N lanes (N = 4, 16 or 64), in every
// lane of the group.  Within a 16-lane row, DPP rotations by 8, 4, 2, 1 leave
// every lane with the row maximum (after rotating by 2^k the value has period
// 2^k along the row).
template <int N>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
  static_assert(N == 4 || N == 16 || N == 64, "group size");
  if constexpr (N == 4) return lane_max_xor<2, false>(lane_max_xor<1, false>(v));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false));   // row_ror:8
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x124, 0xF, 0xF, false));   // row_ror:4
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x122, 0xF, 0xF, false));   // row_ror:2
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x121, 0xF, 0xF, false));   // row_ror:1
  if constexpr (N == 64) v = lane_max_xor<32, false>(lane_max_xor<16, false>(v));
  return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

// ------------------------------------------------------------------ scale

// s = fmax / max(amax, 1e-12f) with an IEEE round-to-nearest-even division.
__device__ __forceinline__ float scale_from_amax(float amax, int codec) {
  return __fdiv_rn(fmax_of(codec), fmaxf(amax, kAmaxFloor));
}

// ------------------------------------------------------------------ FP8 codec
//
// enc(y): round a value already clamped to [-fmax, fmax] to the nearest FP8
// value, ties to the even code.
//  * e4m3fn: gfx950's FP8 convert (v_cvt_pk_fp8_f32) is the OCP e4m3 format
//    with round-to-nearest-even; it keeps the sign of a zero result.  It was
//    checked against an integer reference encoder on every fp32 value in
//    [-448, 448], subnormal inputs included, with no mismatch.
//  * e4m3fnuz: every e4m3fnuz value is half the e4m3fn value of the same code
//    (bias 8 vs 7, same field widths), except code 0x7F (240), whose double
//    480 e4m3fn cannot hold, and the single unsigned zero.  So
//    enc_fnuz(y) = enc_fn(2y) for |y| <= 224 (doubling is exact and keeps
//    midpoints and ties), |y| in (224, 232] rounds to 224 (0x7E; 232 is the tie,
//    even code), |y| > 232 rounds to 240 (0x7F), and a zero result drops its
//    sign.  Checked the same way on every fp32 value in [-240, 240].
template <bool HI>
__device__ __forceinline__ uint32_t cvt_fn_pair(float a, float b, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

template <int CODEC>
__device__ __forceinline__ uint32_t enc_fp8(float y) {
  if constexpr (CODEC == 0) {
    return cvt_fn_pair<false>(y, y, 0u) & 0xFFu;
  } else {
    const float y2 = __builtin_amdgcn_fmed3f(2.0f * y, -448.0f, 448.0f);
    uint32_t c = cvt_fn_pair<false>(y2, y2, 0u) & 0xFFu;
    if (fabsf(y) > 232.0f) c = (c & 0x80u) | 0x7Fu;
    return (c & 0x7Fu) ? c : 0u;
  }
}

// y = clamp(fp32(x * s), -fmax, fmax): one rounded multiply, then the clamp.
template <int CODEC>
__device__ __forceinline__ float scale_clamp(float x, float s) {
  const float fm = fmax_of(CODEC);
  return __builtin_amdgcn_fmed3f(__fmul_rn(x, s), -fm, fm);
}

// Four values -> four FP8 codes packed little-endian in a u32.
template <int CODEC>
__device__ __forceinline__ uint32_t quant4(float a, float b, float c, float d, float s) {
  const float ya = scale_clamp<CODEC>(a, s), yb = scale_clamp<CODEC>(b, s);
  const float yc = scale_clamp<CODEC>(c, s), yd = scale_clamp<CODEC>(d, s);
  if constexpr (CODEC == 0) {
    return cvt_fn_pair<true>(yc, yd, cvt_fn_pair<false>(ya, yb, 0u));
  } else {
    return enc_fp8<1>(ya) | (enc_fp8<1>(yb) << 8) | (enc_fp8<1>(yc) << 16) | (enc_fp8<1>(yd) << 24);
  }
}

// Two packed bf16 pairs (4 values) -> four codes.
template <int CODEC>
__device__ __forceinline__ uint32_t quant_bf16x4(uint32_t p0, uint32_t p1, float s) {
  return quant4<CODEC>(bf16_lo(p0), bf16_hi(p0), bf16_lo(p1), bf16_hi(p1), s);
}

// ------------------------------------------------------------------ e8m0

// Shared MX exponent X of a block from the bit pattern of its |x| max (an
// fp32 built from bf16, so never NaN here):
//   FLOOR_OCP: X = floor(log2 amax) - 8;  CEIL: smallest X with amax*2^-X <= 448,
//   i.e. one more than FLOOR when the significand exceeds 1.75.
// amax == 0 -> -127; X clamped to [-127, 127].  Subnormal amax uses its
// leading-bit position.
__device__ __forceinline__ int mx_exponent(uint32_t amax_bits, int rule) {
  if (amax_bits == 0) return -127;
  const int e = (int)(amax_bits >> 23);
  const uint32_t m = amax_bits & 0x7FFFFFu;
  int lg;              // floor(log2 amax)
  uint32_t sig_frac;   // significand bits after the leading one, left-aligned in 23 bits
  if (e == 0) {
    const int p = 31 - __clz(m);            // leading-one position; amax = m * 2^-149
    lg = p - 149;
    sig_frac = (m << (23 - p)) & 0x7FFFFFu;
  } else {
    lg = e - 127;
    sig_frac = m;
  }
  int X = lg - 8;
  if (rule == 1 && sig_frac > 0x600000u) X += 1;   // significand > 1.75
  return max(-127, min(127, X));
}

// The same rule for a block maximum that is a bf16 value, given as its 16-bit
// pattern a16 (finite): floor(log2 amax) is the exponent field minus 127 for a
// normal value, and at most -127 for a subnormal one, so X = field - 135
// (+1 under CEIL when the 7-bit significand exceeds 0x60, i.e. 1.75) clamped
// below at -127; the largest finite bf16 gives X = 119, so the upper clamp
// never acts.  Equal to mx_exponent(a16 << 16, rule) for every such a16.
__device__ __forceinline__ int mx_exponent_bf16(uint32_t a16, int rule) {
  int X = (int)(a16 >> 7) - 135;
  if (rule == 1) X += (a16 & 0x7Fu) > 0x60u ? 1 : 0;
  return max(X, -127);
}

// 2^-X for X in [-127, 119] (a normal fp32, no branch).
__device__ __forceinline__ float exp2_neg_bf16(int X) { return __uint_as_float((uint32_t)(127 - X) << 23); }

// ------------------------------------------------------------------ MX cast on the scaled converter
//
// gfx950's v_cvt_scalef32_pk_fp8_bf16 converts two bf16 values to e4m3fn after
// dividing them by 2^(e - 127), where e is the exponent field of its fp32
// scale operand (the significand is ignored; e = 0 means 2^-127): given the
// block's e8m0 code E = X + 127 in that field, it computes enc(x * 2^-X) with
// round-to-nearest-even, the sign of a zero result kept.  The product is exact
// (a power-of-two scaling of a bf16 value, except where it falls below 2^-126,
// far under the smallest e4m3 step), so this equals the clamp-then-encode of
// the software path for every |x * 2^-X| <= 448.  Above, the converter returns
// 448 up to the rounding boundary 464 and the NaN code (0x7F, 0xFF) beyond;
// e4m3fn has no other NaN or infinity, so replacing a NaN code by the largest
// code of its sign (0x7E, 0xFE) gives the clamped result there too.  Checked
// on every bf16 value under scales 2^-127 .. 2^127, and the MX kernels that use
// it are checked bit for bit against the oracle.
typedef short mx_v2i16 __attribute__((ext_vector_type(2)));
typedef __bf16 mx_v2bf16 __attribute__((ext_vector_type(2)));

// The scale operand carrying e8m0 code E (0..254).
__device__ __forceinline__ float mx_scale_operand(int E) { return __uint_as_float((uint32_t)E << 23); }

// Four codes (little-endian) of the bf16 pairs p0 = (x0, x1), p1 = (x2, x3) under one scale operand,
// NaN codes replaced by +-448 (needed only when a value can exceed 448: the FLOOR rule).
template <bool SAT>
__device__ __forceinline__ uint32_t mx_cvt4(uint32_t p0, uint32_t p1, float sc) {
  mx_v2i16 o = {0, 0};
  o = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o, __builtin_bit_cast(mx_v2bf16, p0), sc, false);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o, __builtin_bit_cast(mx_v2bf16, p1), sc, true);
  uint32_t w = __builtin_bit_cast(uint32_t, o);
  if constexpr (SAT) {
    // a byte whose low 7 bits are all set (the NaN codes) gets its lowest bit cleared
    const uint32_t u = (w & 0x7F7F7F7Fu) + 0x01010101u;
    w ^= (u >> 7) & 0x01010101u;
  }
  return w;
}

// 2^-X as an fp32 for X in [-127, 127] (X = 127 gives the subnormal 2^-127 = 0x00400000).
__device__ __forceinline__ float exp2_neg(int X) {
  const int be = 127 - X;  // biased exponent of 2^-X, in [0, 254]
  return be > 0 ? __uint_as_float((uint32_t)be << 23) : __uint_as_float(0x00400000u);
}

// ------------------------------------------------------------------ groups

__device__ __forceinline__ int clamp_off(int v, int rows) { return min(max(v, 0), rows); }

// Block-wide inclusive scans over one value per thread (blockDim.x == NT, a
// multiple of 64, at most 1024).  `tmp` is NT/64 ints of shared memory.
template <int NT>
__device__ __forceinline__ int block_scan_max(int v, int* tmp) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int o = __shfl_up(v, d, 64);
    if (lane >= d) v = max(v, o);
  }
  if (lane == 63) tmp[w] = v;
  __syncthreads();
  int pre = 0;
  for (int i = 0; i < w; ++i) pre = max(pre, tmp[i]);
  __syncthreads();
  return max(v, pre);
}

template <int NT>
__device__ __forceinline__ int block_scan_sum(int v, int* tmp) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  if (lane == 63) tmp[w] = v;
  __syncthreads();
  int pre = 0;
  for (int i = 0; i < w; ++i) pre += tmp[i];
  __syncthreads();
  return v + pre;
}

// Work-unit scheduler.  Group e covers rows [lo(e), hi(e)) with hi(e) the
// running maximum of offs clamped to [0, rows] and lo(e) = hi(e-1) (disjoint
// groups; a decreasing offset gives an empty group).  Each group owns
// chunks(lo, hi) consecutive work units; unit u maps to (group e, chunk j).
// `pbase` is the exclusive prefix over groups of pad(lo, hi) (a padded row
// count, or 0 when unused).  offs == nullptr means one group of all rows.
// The host never reads the offsets: it sizes the grid from a bound on the unit
// count.  A unit past the real total comes back with e = -1, j = u - total
// units and pbase = the padded total, so a caller may give such units a tail
// job or exit.  Every thread of the block must call it (it synchronizes).
struct Unit {
  int e, j, lo, hi, pbase;
};

template <int NT, typename ChunkFn, typename PadFn>
__device__ __forceinline__ Unit find_unit(const int32_t* __restrict__ offs, int n_groups, int rows,
                                          int u, ChunkFn chunks, PadFn pad) {
  if (offs == nullptr) {
    const int c = chunks(0, rows);
    return u < c ? Unit{0, u, 0, rows, 0} : Unit{-1, u - c, 0, 0, pad(0, rows)};
  }
  __shared__ int tmp[NT / 64];
  __shared__ int s_hi[NT];
  __shared__ int s_total, s_ptotal;
  __shared__ Unit found;
  const int t = threadIdx.x;
  if (t == 0) found = Unit{-1, 0, 0, 0, 0};
  int base = 0, pbase = 0, carry = 0;   // units, padded rows and row maximum of previous slices
  for (int g0 = 0; g0 < n_groups; g0 += NT) {
    const int e = g0 + t;
    const int v = e < n_groups ? clamp_off(offs[e], rows) : 0;
    const int hi = max(block_scan_max<NT>(v, tmp), carry);
    s_hi[t] = hi;
    __syncthreads();
    const int lo = t == 0 ? carry : s_hi[t - 1];
    const int cnt = e < n_groups ? chunks(lo, hi) : 0;
    const int pd = e < n_groups ? pad(lo, hi) : 0;
    const int incl = block_scan_sum<NT>(cnt, tmp) + base;
    const int pincl = block_scan_sum<NT>(pd, tmp) + pbase;
    const int excl = incl - cnt;
    if (e < n_groups && u >= excl && u < incl) found = Unit{e, u - excl, lo, hi, pincl - pd};
    if (t == NT - 1) { s_total = incl; s_ptotal = pincl; }
    __syncthreads();
    base = s_total;
    pbase = s_ptotal;
    carry = s_hi[NT - 1];
    __syncthreads();
    if (u < base) break;       // uniform: every thread sees the same base
  }
  __syncthreads();
  Unit r = found;
  if (r.e < 0) r = Unit{-1, u - base, 0, 0, pbase};
  return r;
}

// find_unit for at most 64 groups, by one wave with no shared memory and no
// barrier: lane e holds group e, running maximum and sums by lane shuffles, the
// owning lane found by a ballot.  Every wave of a workgroup computes the same
// result on its own.  The same unit as find_unit (whose scans take about ten
// workgroup barriers before a quantizer workgroup can issue its first load).
template <typename ChunkFn, typename PadFn>
__device__ __forceinline__ Unit find_unit_wave(const int32_t* __restrict__ offs, int n_groups, int rows, int u,
                                               ChunkFn chunks, PadFn pad) {
  const int lane = threadIdx.x & 63;
  const bool in = lane < n_groups;
  int hi = in ? clamp_off(offs[lane], rows) : 0;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(hi, d, 64);
    if (lane >= d) hi = max(hi, o);
  }
  int lo = __shfl_up(hi, 1, 64);
  if (lane == 0) lo = 0;
  const int cnt = in ? chunks(lo, hi) : 0;
  const int pd = in ? pad(lo, hi) : 0;
  int incl = cnt, pincl = pd;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64), po = __shfl_up(pincl, d, 64);
    if (lane >= d) {
      incl += o;
      pincl += po;
    }
  }
  const int excl = incl - cnt;
  const unsigned long long hit = __ballot(in && u >= excl && u < incl);
  if (hit != 0ull) {
    const int src = __ffsll(hit) - 1;
    return Unit{src, u - __shfl(excl, src, 64), __shfl(lo, src, 64), __shfl(hi, src, 64),
                __shfl(pincl - pd, src, 64)};
  }
  return Unit{-1, u - __shfl(incl, 63, 64), 0, 0, __shfl(pincl, 63, 64)};
}

// The group lookup of the quantizers: one wave each for at most 64 groups,
// else the workgroup scan (a workgroup-uniform choice).
template <int NT, typename ChunkFn, typename PadFn>
__device__ __forceinline__ Unit find_unit_quant(const int32_t* __restrict__ offs, int n_groups, int rows, int u,
                                                ChunkFn chunks, PadFn pad) {
  if (offs != nullptr && n_groups <= 64) return find_unit_wave(offs, n_groups, rows, u, chunks, pad);
  return find_unit<NT>(offs, n_groups, rows, u, chunks, pad);
}

}  // namespace fp8moe

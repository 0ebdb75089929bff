// Offset-routed grouped GEMM on gfx950 FP8 MFMA, for the forward, dgrad and
// wgrad products of an MoE expert layer.
// [P1 Details, MoE paragraph: variable-size expert batches through one grouped
// GEMM launch with per-row activation scales, per-expert weight column scales
// and routing offsets; P4 "MoE: почему DeepSeek-V3 ломал пайплайн"; P3/P4 on
// the three GEMMs of a linear layer; P2 Details: 2D activations x 3D expert
// weights grouped by offsets, and the MXFP8 scaled grouped GEMM.]
//
// Both operands are read contraction-contiguous ("row operand" P: tile rows
// are output rows; "column operand" Q: tile rows are output columns):
//   GROUPED_M (fwd/dgrad): P = A[m][K] rows of group e, Q = B[e][n][K].
//   GROUPED_K (wgrad):     P = A phys [n][M], Q = B phys [k][M], contraction
//                          over the token range [lo(e), hi(e)) of group e.
//
// Two kernels, tiling derived from the hardware rather than searched:
//  * v_mfma_scale_f32_32x32x64_f8f6f4: each lane holds one row (lane & 31) and
//    two 16-byte halves of the 64-wide contraction at byte offsets 16*g and
//    32 + 16*g (g = lane >> 5); the e8m0 scale of (row i, 32-block b) comes
//    from lane i + 32*b.  FP8 operands pass scale 0 (2^0).
//  * 256 threads = 2x2 waves; a wave owns (BM/2) x (BN/2) outputs.  BM = BN =
//    256 gives 4x4 MFMA tiles per wave = 256 fp32 accumulators per lane, the
//    largest tile that fits one wave per SIMD (512 registers) and makes each
//    byte read from LDS feed 128 flops per wave.
//  * gemm_fp8_pipe (every FP8 call, and MX calls with K4 scales or 4-byte
//    aligned row-major scales): persistent, at most one workgroup per CU
//    walking its tiles with a grid stride.  Operands stream through an LDS ring
//    of 128-byte contraction stages (whole cache lines of the K-contiguous
//    operands): two 64 KiB slots for 256 x 256 tiles, three 48 KiB slots for
//    128 x 256 tiles, filled by gfx950's direct global->LDS loads
//    (global_load_lds_dwordx4) with no staging registers.  The steady-state
//    step is branch-free: one wait and barrier per stage, then the refill of
//    the freed slot and the fragment reads of the next k step interleaved
//    (sched_group_barrier) between the MFMAs of the current one.  Consecutive
//    tiles overlap: the next tile's first stages land during the epilogue,
//    which stages bf16 results through LDS so every store writes whole
//    128-byte row segments.  Details at the kernel.
//  * gemm_fp8_kernel (MX operands whose row-major e8m0 rows are not 4-byte
//    aligned per stage): one workgroup per tile, 64-byte stages in a 4-slot
//    ring, e8m0 scales loaded a byte at a time.
//  * Small groups (average rows per group below 512) use BM = 128 to waste
//    less of each tile on padding rows.
//  * Tiles are ordered in bands of 8 row tiles (GROUPED_M: cut at group
//    boundaries, so a band's tiles share one expert's weight panels), and
//    each XCD (dispatch is round-robin over 8) gets a contiguous range of
//    them, so the tiles running together on one XCD share operand rows in its
//    L2.
#include "device_common.hpp"
#include "gemm_common.hpp"
#include "kernels.hpp"

namespace fp8moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kBandRows = 8;   // row tiles per band in the tile order
constexpr int kGemmStageBytes = 64;   // contraction bytes per pipeline stage

struct KParams {
  const uint8_t* a;
  const uint8_t* b;
  const void* sa;
  const void* sb;
  const int32_t* offs;
  void* out;
  int E, M, N, K;
  int row_units;   // GROUPED_M: bound on row tiles over all groups; GROUPED_K: E * ceil(N / BM)
  int col_tiles;   // GROUPED_M: ceil(N / BN); GROUPED_K: ceil(K / BN)
  // ceil(2^32 / (kBandRows * col_tiles)): band = umulhi(L, band_magic) for
  // every logical tile L (exact while L * kBandRows * col_tiles < 2^32).
  uint32_t band_magic;
  uint32_t col_magic;   // ceil(2^32 / col_tiles) (col_tiles >= 2): L / col_tiles = umulhi(L, col_magic)
};

// Each XCD gets a contiguous range of logical tile ids (dispatch is round-robin).
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  const int per = total / 8, rem = total % 8;
  const int x = bid % 8, i = bid / 8;
  return x * per + min(x, rem) + i;
}

// Zero the bytes of a 16-byte chunk at contraction position pos outside [lo, hi).
__device__ __forceinline__ u32x4 mask_chunk(u32x4 v, int pos, int lo, int hi) {
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

// Zero the bytes outside the contraction range [lo, hi) of one stage in LDS:
// SROWS tile rows of CH 16-byte chunks at contraction positions base + 16 c
// (chunk c of row r at R::off(r, c)).  Whether a chunk needs work depends only
// on its column, a workgroup-uniform test: columns wholly outside the range
// are written with zeros (no read), and only the chunk columns holding an end
// of the range (at most two) are read, masked and written back.  Each thread
// handles whole rows; the loops stay rolled to keep register use low.
template <class R, int SROWS, int CH>
__device__ __forceinline__ void zero_outside(uint8_t* st, int base, int lo, int hi) {
  const int end = base + 16 * CH;
  const int ca = (lo > base && lo < end && (lo & 15) != 0) ? (lo - base) >> 4 : -1;
  const int cb = (hi > base && hi < end && (hi & 15) != 0) ? (hi - base) >> 4 : -1;
#pragma unroll 1
  for (int r = threadIdx.x; r < SROWS; r += 256) {
#pragma unroll 1
    for (int c = 0; c < CH; ++c) {
      const int pos = base + 16 * c;
      if (pos + 16 <= lo || pos >= hi) *reinterpret_cast<u32x4*>(st + R::off(r, c)) = u32x4{0, 0, 0, 0};
    }
    if (ca >= 0) {
      u32x4* q = reinterpret_cast<u32x4*>(st + R::off(r, ca));
      *q = mask_chunk(*q, base + 16 * ca, lo, hi);
    }
    if (cb >= 0 && cb != ca) {
      u32x4* q = reinterpret_cast<u32x4*>(st + R::off(r, cb));
      *q = mask_chunk(*q, base + 16 * cb, lo, hi);
    }
  }
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Pipeline shape: stages of BK = 64 contraction bytes (one MFMA K step) in a
// 4-slot LDS ring (4 x (BM + BN) x 64 B = 128 KiB for 256 x 256 tiles).
template <int BK>
struct Ring {
  static_assert(BK == 64, "64-byte stages (128-byte stages spill registers at 256 x 256)");
  static constexpr int CH = BK / 16;                  // 16-byte chunks per tile row
  static constexpr int SH = 2;                        // swizzle shift: log2(16 / CH)
  static constexpr int SLOTS = 4;
  static constexpr int RPB = 1024 / BK;               // tile rows per 1 KiB DMA block
  // Swizzled offset of chunk c of tile row r: 16 lanes reading one logical chunk
  // of 16 consecutive rows hit 16 distinct 16-byte bank groups.
  static __device__ __forceinline__ int off(int r, int c) { return r * BK + ((c ^ ((r >> SH) & (CH - 1))) << 4); }
};

template <int BM, int BN, int BK, int MODE, int SK, int OUT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_fp8_kernel(KParams p) {
  using R = Ring<BK>;
  constexpr int kBK = BK, kSlots = R::SLOTS, CH = R::CH;
  constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 32, TN = WN / 32;
  constexpr int A_BYTES = BM * kBK, STAGE = (BM + BN) * kBK;
  constexpr int BLOCKS = STAGE / 1024;                 // 1 KiB DMA blocks per stage
  constexpr int BPW = BLOCKS / 4;                      // per wave
  constexpr int SROWS = BM + BN;                       // e8m0 bytes per stage and 32-block
  constexpr int NB = kBK / 32;                         // e8m0 blocks per row per stage
  constexpr int SC_DMA = SK == 1 ? (NB * SROWS) / 64 / 4 : 0;   // byte DMAs per wave per stage
  constexpr int LPS = BPW + SC_DMA;                    // vector-memory ops per wave per stage
  // One array per ring slot, each accessed with a compile-time slot index, so the
  // compiler can tell a load landing in one slot from reads of another.
  __shared__ __attribute__((aligned(1024))) uint8_t ring0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t ring1[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t ring2[kSlots > 2 ? STAGE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t ring3[kSlots > 2 ? STAGE : 16];
  constexpr int SRB = SK == 1 ? 4 * NB * SROWS : 16;  // byte DMAs land one lane per dword
  __shared__ __attribute__((aligned(16))) uint8_t sring0[SRB];
  __shared__ __attribute__((aligned(16))) uint8_t sring1[SRB];
  __shared__ __attribute__((aligned(16))) uint8_t sring2[kSlots > 2 ? SRB : 16];
  __shared__ __attribute__((aligned(16))) uint8_t sring3[kSlots > 2 ? SRB : 16];
  uint8_t* const slot_data[4] = {ring0, ring1, ring2, ring3};
  uint8_t* const slot_scale[4] = {sring0, sring1, sring2, sring3};

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---------------------------------------------------------------- tile -> work
  const int total = gridDim.x;
  const int L = xcd_remap(blockIdx.x, total);
  const int band = L / (kBandRows * p.col_tiles);
  const int first = band * kBandRows;
  const int gsz = min(p.row_units - first, kBandRows);
  const int inband = L % (kBandRows * p.col_tiles);
  const int ru = first + inband % gsz;
  const int ct = inband / gsz;

  const uint8_t* P;
  const uint8_t* Q;
  int64_t p_ld, q_ld;
  int p_valid, q_valid, c_lo, c_hi, e;
  int64_t out_base, out_ld;
  const uint8_t* psc = nullptr;   // e8m0 rows
  const uint8_t* qsc = nullptr;
  int64_t sc_ld = 0;
  const float* psf = nullptr;     // fp32 scales of the tile's rows / columns
  const float* qsf = nullptr;
  if constexpr (MODE == 0) {
    struct Ch {
      __device__ int operator()(int lo, int hi) const { return (hi - lo + BM - 1) / BM; }
    };
    struct NoPad {
      __device__ int operator()(int, int) const { return 0; }
    };
    const Unit un = find_unit<256>(p.offs, p.E, p.M, ru, Ch{}, NoPad{});
    if (un.e < 0) return;
    e = un.e;
    const int m0 = un.lo + un.j * BM, n0 = ct * BN;
    p_valid = min(BM, un.hi - m0);
    q_valid = min(BN, p.N - n0);
    P = p.a + (int64_t)m0 * p.K;
    Q = p.b + ((int64_t)e * p.N + n0) * p.K;
    p_ld = q_ld = p.K;
    c_lo = 0;
    c_hi = p.K;
    out_ld = p.N;
    out_base = (int64_t)m0 * p.N + n0;
    if constexpr (SK == 1) {
      sc_ld = p.K / 32;
      psc = static_cast<const uint8_t*>(p.sa) + (int64_t)m0 * sc_ld;
      qsc = static_cast<const uint8_t*>(p.sb) + ((int64_t)e * p.N + n0) * sc_ld;
    } else {
      psf = static_cast<const float*>(p.sa) + m0;
      qsf = static_cast<const float*>(p.sb) + (int64_t)e * p.N + n0;
    }
  } else {
    const int ntn = (p.N + BM - 1) / BM;
    e = ru / ntn;
    const int n0 = (ru % ntn) * BM, k0 = ct * BN;
    // group range of e: lo = max over j < e of clamp(offs[j]); hi = max(lo, clamp(offs[e]))
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
    P = p.a + (int64_t)n0 * p.M;
    Q = p.b + (int64_t)k0 * p.M;
    p_ld = q_ld = p.M;
    c_lo = lo;
    c_hi = hi;
    out_ld = p.K;
    out_base = ((int64_t)e * p.N + n0) * p.K + k0;
    if constexpr (SK == 1) {
      sc_ld = p.M / 32;
      psc = static_cast<const uint8_t*>(p.sa) + (int64_t)n0 * sc_ld;
      qsc = static_cast<const uint8_t*>(p.sb) + (int64_t)k0 * sc_ld;
    } else {
      psf = static_cast<const float*>(p.sa) + (int64_t)e * p.N + n0;
      qsf = static_cast<const float*>(p.sb) + (int64_t)e * p.K + k0;
    }
  }

  const int c_start = c_lo & ~15;
  const int nk = c_hi > c_lo ? (c_hi - c_start + kBK - 1) / kBK : 0;

  // ---------------------------------------------------------------- DMA global -> LDS
  // Wave `wave` moves blocks wave + 4*i (i < BPW) of each stage; the first
  // BPW_A of them lie in the A tile, the rest in the B tile.  In a block, lane l
  // fills LDS bytes [16 l, 16 l + 16): tile row RPB*blk + l/CH, physical chunk
  // l%CH, i.e. logical chunk (l%CH) ^ ((row >> SH) & (CH-1)), which is the same
  // for every block of a wave.  Rows are 32-bit offsets from the uniform A/B
  // tile bases (host validation bounds the row strides).
  constexpr int BPW_A = BM / R::RPB / 4;
  const int dma_c = (lane % CH) ^ (((R::RPB * wave + lane / CH) >> R::SH) & (CH - 1));
  uint32_t roff[BPW];
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int r = R::RPB * (wave + 4 * i) + lane / CH;   // row in the concatenated [A; B] tile
    roff[i] = i < BPW_A ? (uint32_t)(min(r, p_valid - 1) * p_ld) : (uint32_t)(min(r - BM, q_valid - 1) * q_ld);
  }
  // e8m0: byte DMA d of a stage covers (block d/(SROWS/64) of the stage, rows 64*(d%(SROWS/64)) + lane)
  const uint8_t* srow[SK == 1 ? SC_DMA : 1];
  if constexpr (SK == 1) {
#pragma unroll
    for (int i = 0; i < SC_DMA; ++i) {
      const int d = wave + 4 * i;
      const int r = 64 * (d % (SROWS / 64)) + lane;
      srow[i] = r < BM ? psc + (int64_t)min(r, p_valid - 1) * sc_ld : qsc + (int64_t)min(r - BM, q_valid - 1) * sc_ld;
    }
  }

  // Issue the DMAs of stage kt into ring slot SLOT (== kt % kSlots).  Every lane
  // issues exactly one load per block (the per-stage wait counts rely on it):
  // positions outside [c_lo, c_hi) are clamped to a valid chunk of the same row
  // and zeroed in LDS by the boundary-stage fix-up.
  const int pos_max = max((c_hi - 1) & ~15, 0);   // the last chunk overlapping the range
  auto issue_stage = [&](auto slot_tag, int kt) {
    constexpr int SLOT = decltype(slot_tag)::value;
    uint8_t* dst = slot_data[SLOT];
    const int base = c_start + kt * kBK;
    const uint32_t pos = (uint32_t)min(base + 16 * dma_c, pos_max);
#pragma unroll
    for (int i = 0; i < BPW; ++i)
      dma_16((i < BPW_A ? P : Q) + (roff[i] + pos), dst + (wave + 4 * i) * 1024);
    if constexpr (SK == 1) {
      // e8m0 bytes past the range come from the row's last valid block; the
      // data they scale is zeroed, and the quantizer never emits the NaN code.
      uint8_t* sdst = slot_scale[SLOT];
      const int blk0 = (c_start + kt * kBK) >> 5, nblk = c_hi >> 5;
#pragma unroll
      for (int i = 0; i < SC_DMA; ++i) {
        const int d = wave + 4 * i;
        const int b = d / (SROWS / 64);
        dma_1(srow[i] + max(min(blk0 + b, nblk - 1), 0), sdst + 256 * d);
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

  // Wait until at most n later stages' loads are still outstanding.
  auto wait_stages = [&](int n) {
    if (n >= 3) wait_vmcnt<3 * LPS>();
    else if (n == 2) wait_vmcnt<2 * LPS>();
    else if (n == 1) wait_vmcnt<LPS>();
    else wait_vmcnt<0>();
  };
  // Zero the bytes of every chunk of stage kt (in LDS `st`) outside or straddling
  // [c_lo, c_hi).  Only the first and last stage of a range can hold such chunks.
  auto fix_boundary = [&](uint8_t* st, int kt) {
    const int base = c_start + kt * kBK;
    if (base >= c_lo && base + kBK <= c_hi) return;    // uniform
    zero_outside<R, SROWS, CH>(st, base, c_lo, c_hi);
    wait_lgkmcnt0();
    raw_barrier();
  };

  // Two register sets of MFMA fragments: stage k's MFMAs run from one while
  // stage k+1's fragments are read from LDS into the other.
  v8i fa0[TM], fb0[TN], fa1[TM], fb1[TN];
  int ea0[TM], eb0[TN], ea1[TM], eb1[TN];      // e8m0 scale operands
  auto read_frags = [&](v8i (&fa)[TM], v8i (&fb)[TN], int (&ea)[TM], int (&eb)[TN], const uint8_t* st,
                        const uint8_t* sc) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = wm * WM + 32 * i + lrow;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(st + R::off(r, g));
      const u32x4 hi = *reinterpret_cast<const u32x4*>(st + R::off(r, 2 + g));
      fa[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      if constexpr (SK == 1) ea[i] = sc[4 * (g * SROWS + r)];
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int r = wn * WN + 32 * j + lrow;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(st + A_BYTES + R::off(r, g));
      const u32x4 hi = *reinterpret_cast<const u32x4*>(st + A_BYTES + R::off(r, 2 + g));
      fb[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      if constexpr (SK == 1) eb[j] = sc[4 * (g * SROWS + BM + r)];
    }
  };
  auto mma = [&](v8i (&fa)[TM], v8i (&fb)[TN], int (&ea)[TM], int (&eb)[TN]) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (SK == 1)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 0, 0, 0, ea[i], 0,
                                                                      eb[j]);
        else
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 0, 0, 0, 0, 0, 0);
      }
  };

  // One pipeline step for stage kt, held in ring slot SLOT (== kt % 4), whose
  // fragments are already in register set SLOT % 2:
  //  1. wait for stage kt+1 and for this wave's reads of slot SLOT, barrier
  //     (stage kt+1 is visible; no wave still reads slot SLOT);
  //  2. refill slot SLOT with stage kt+4;
  //  3. read stage kt+1's fragments into the other set, then run stage kt's MFMAs.
  auto step = [&](auto slot_tag, int kt) {
    constexpr int SLOT = decltype(slot_tag)::value;
    constexpr int NS = (SLOT + 1) % kSlots;
    wait_lgkmcnt0();   // on every path, so the MFMAs below never wait on the reads issued next
    if (kt + 1 < nk) {
      wait_stages(min(2, nk - 2 - kt));
      raw_barrier();
      fix_boundary(slot_data[NS], kt + 1);
      if (kt + kSlots < nk) issue_stage(slot_tag, kt + kSlots);
      if constexpr (SLOT % 2 == 0) read_frags(fa1, fb1, ea1, eb1, slot_data[NS], slot_scale[NS]);
      else read_frags(fa0, fb0, ea0, eb0, slot_data[NS], slot_scale[NS]);
    }
    if constexpr (SLOT % 2 == 0) mma(fa0, fb0, ea0, eb0);
    else mma(fa1, fb1, ea1, eb1);
  };

  if (nk > 0) {
    issue_stage(std::integral_constant<int, 0>{}, 0);
    if (1 < nk) issue_stage(std::integral_constant<int, 1>{}, 1);
    if (2 < nk) issue_stage(std::integral_constant<int, 2>{}, 2);
    if (3 < nk) issue_stage(std::integral_constant<int, 3>{}, 3);
    wait_stages(min(3, nk - 1));
    raw_barrier();
    fix_boundary(slot_data[0], 0);
    read_frags(fa0, fb0, ea0, eb0, slot_data[0], slot_scale[0]);
  }
  for (int kt = 0; kt < nk; kt += kSlots) {
    step(std::integral_constant<int, 0>{}, kt);
    if (kt + 1 < nk) step(std::integral_constant<int, 1>{}, kt + 1);
    if (kt + 2 < nk) step(std::integral_constant<int, 2>{}, kt + 2);
    if (kt + 3 < nk) step(std::integral_constant<int, 3>{}, kt + 3);
  }

  // ---------------------------------------------------------------- epilogue
  // fp32 scales are multipliers of the quantized operands: divide by both.
  const bool empty = c_hi <= c_lo;
  float inv_q[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int cidx = min(wn * WN + 32 * j + lrow, q_valid - 1);
    inv_q[j] = SK == 0 ? __frcp_rn(qsf[cidx]) : 1.0f;
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = wm * WM + 32 * i + 8 * (v >> 2) + 4 * g + (v & 3);
      if (r >= p_valid) continue;
      const float inv_p = SK == 0 ? __frcp_rn(psf[r]) : 1.0f;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int c = wn * WN + 32 * j + lrow;
        if (c >= q_valid) continue;
        const float val = empty ? 0.0f : acc[i][j][v] * inv_p * inv_q[j];
        const int64_t o = out_base + (int64_t)r * out_ld + c;
        if constexpr (OUT == 0)
          static_cast<uint16_t*>(p.out)[o] = f32_to_bf16_rne(val);
        else
          static_cast<float*>(p.out)[o] = val;
      }
    }
  }
}

// ============================================================================
// Interleaved pipeline: 128-byte contraction stages.
//
// Measured on gfx950 (one workgroup per CU, operands resident in L2):
//  * a direct global->LDS load moving 64-byte row segments delivers about half
//    the bytes per clock of one moving whole 128-byte lines, so a stage spans
//    BK = 128 contraction bytes (whole lines of K-contiguous operands);
//  * issuing a stage's loads and LDS fragment reads as one burst ahead of its
//    MFMAs stalls instruction issue and leaves the matrix cores idle for about
//    a third of the loop; spreading them between the MFMAs of the same
//    scheduling region (sched_group_barrier) keeps the matrix cores at ~95%.
// A stage is (BM + BN) x 128 B: 64 KiB for 256 x 256 tiles, so the ring holds
// two stages (one computing, one landing); 128 x 256 tiles hold three.  Each
// stage runs as two 64-byte MFMA k steps; fragments of the next k step are read
// from LDS while the current one's MFMAs issue.  The steady-state step is
// branch-free so the interleave spans it; the first and last stages (which may
// straddle the contraction range) go through a checked path.
//
// Swizzle of a 128-byte LDS row: logical chunk c of row r sits at physical
// chunk c ^ ((r >> 1) & 7).  A 16-byte read serves 16 lanes per clock from 64
// banks (256 bytes, two 128-byte rows): 16 consecutive rows reading one logical
// chunk land on 16 distinct (row parity, chunk) slots.  The XOR term depends
// on the row only through bits 1..3, so a fragment's address is affine in its
// 32-row tile index and the compiler folds it into immediate offsets.
template <int BK>
struct PipeRing {
  static_assert(BK == 64 || BK == 128, "stage width");
  static constexpr int CH = BK / 16;          // 16-byte chunks per tile row
  static constexpr int RPB = 1024 / BK;       // tile rows per 1 KiB DMA block
  static __device__ __forceinline__ int phys(int r, int c) {
    if constexpr (BK == 64) return c ^ ((r >> 2) & 3);
    else return c ^ ((r >> 1) & 7);
  }
  static __device__ __forceinline__ int off(int r, int c) { return r * BK + (phys(r, c) << 4); }
};

// Zero the bytes outside the contraction range [lo, hi) of one ring stage
// (SROWS tile rows of CH 16-byte chunks at contraction positions base + 16 c).
// Wave w takes chunk columns w, w + 4, ..., so the test of a column is
// wave-uniform: a column wholly outside the range is overwritten with zeros,
// a column holding an end of the range is read, masked with one mask for all
// its rows and written back, and any other column is left alone.  Lane l
// takes rows l, l + 64, ...: the swizzle term of a row repeats every 16 rows,
// so a lane's chunks of one column lie 64 BK bytes apart.
template <class R, int SROWS, int CH>
__device__ __forceinline__ void zero_outside_ring(uint8_t* st, int base, int lo, int hi) {
  static_assert(SROWS % 64 == 0 && CH % 4 == 0, "whole row groups and column sets per wave");
  constexpr int RPL = SROWS / 64;               // rows per lane
  constexpr int STEP = 64 * R::CH * 16;         // bytes between a lane's rows
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  const int lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const uint32_t st_l = lds_off(st);
#pragma unroll
  for (int cc = 0; cc < CH / 4; ++cc) {
    const int c = wave + 4 * cc;                // wave-uniform column
    const int pos = base + 16 * c;
    const uint32_t a0 = st_l + R::off(lane, c);
    if (pos + 16 <= lo || pos >= hi) {
#pragma unroll
      for (int k = 0; k < RPL; ++k) lds_write16(a0 + k * STEP, lds_u4{0u, 0u, 0u, 0u});
    } else if (pos < lo || pos + 16 > hi) {
      const u32x4 m = mask_chunk(u32x4{~0u, ~0u, ~0u, ~0u}, pos, lo, hi);
      const lds_u4 mv = lds_u4{m.x, m.y, m.z, m.w};
      lds_u4 v[RPL];
#pragma unroll
      for (int k = 0; k < RPL; ++k) v[k] = lds_read16(a0 + k * STEP);
      lds_wait();
#pragma unroll
      for (int k = 0; k < RPL; ++k) {
        lds_ready(v[k]);
        lds_write16(a0 + k * STEP, v[k] & mv);
      }
    }
  }
}

__device__ __forceinline__ void dma_4(const uint8_t* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 4, 0, 0);
}

// A wave-uniform value moved to scalar registers.
__device__ __forceinline__ int64_t uniform_i64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  return reinterpret_cast<T*>(uniform_i64(reinterpret_cast<int64_t>(p)));
}

template <int BM, int BN, int BK, int SLOTS, int MODE, int SK, int OUT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_fp8_pipe(KParams p) {
  using R = PipeRing<BK>;
  constexpr int CH = R::CH, KS = BK / 64;
  constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 32, TN = WN / 32;
  constexpr int A_BYTES = BM * BK, STAGE = (BM + BN) * BK;
  constexpr int BPW = STAGE / 1024 / 4, BPW_A = A_BYTES / 1024 / 4;   // 1 KiB DMA blocks per wave
  constexpr int SROWS = BM + BN;
  // e8m0: one 4-byte load per tile row and stage (the stage's four 32-blocks),
  // 64 rows per wave-wide load, every wave issuing the same count.
  constexpr bool E8 = SK != 0;                        // e8m0 scales (SK 1: row-major, SK 2: K4 layout)
  constexpr int SC_DMA = E8 ? (SROWS / 64 + 3) / 4 : 0;
  constexpr int LPS = BPW + SC_DMA;                   // vector-memory ops per wave per stage
  constexpr int SCB = E8 ? SC_DMA * 4 * 256 : 16;
  constexpr int NM = TM * TN;                         // MFMAs per k step
  // LDS reads per k step: the fragments, plus (e8m0, a stage's first k step) one scale word per
  // fragment row, which serves both k steps of the stage
  constexpr int ND = 2 * (TM + TN);
  constexpr int ND0 = ND + (E8 ? TM + TN : 0);
  static_assert(STAGE % 4096 == 0 && BPW_A * 4096 == A_BYTES, "stage must split into 4 waves of 1 KiB blocks");
  static_assert(!E8 || BK == 128, "e8m0 scales need 128-byte stages");
  static_assert((SLOTS * KS) % 2 == 0 && SLOTS >= 2 && SLOTS <= 4, "fragment sets alternate across the ring");
  static_assert(SLOTS * (STAGE + SCB) <= 150 * 1024, "LDS budget");

  __shared__ __attribute__((aligned(1024))) uint8_t ring0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t ring1[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t ring2[SLOTS > 2 ? STAGE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t ring3[SLOTS > 3 ? STAGE : 16];
  __shared__ __attribute__((aligned(16))) uint8_t sring0[SCB];
  __shared__ __attribute__((aligned(16))) uint8_t sring1[SCB];
  __shared__ __attribute__((aligned(16))) uint8_t sring2[SLOTS > 2 ? SCB : 16];
  __shared__ __attribute__((aligned(16))) uint8_t sring3[SLOTS > 3 ? SCB : 16];
  uint8_t* const slot_data[4] = {ring0, ring1, ring2, ring3};
  uint8_t* const slot_scale[4] = {sring0, sring1, sring2, sring3};
  // Epilogue staging, 4 KiB per wave: its own buffer beside a 2-slot ring (so
  // both slots can take the next tile's first stages meanwhile), else the
  // last ring slot.
  constexpr int kStgWave = 4096;
  __shared__ __attribute__((aligned(16))) uint8_t stg_own[SLOTS == 2 ? 4 * kStgWave : 16];
  // Ring slots refilled with the next tile's first stages before the
  // epilogue; any others (the staging slot) after it.
  constexpr int NPRE = SLOTS == 2 ? 2 : SLOTS - 1;

  // ---------------------------------------------------------------- tiles
  // Persistent: the grid is at most one workgroup per CU and each walks the
  // tiles with a stride of the grid.  Round k gives XCD x (dispatch is
  // round-robin over 8) the contiguous logical tiles [G k + G/8 x, + G/8)
  // (for a skewed GROUPED_K, odd rounds backwards: [G k + G/8 (7 - x), ...)),
  // so the tiles one XCD runs together share operand rows in its L2; logical
  // tiles run in bands of kBandRows row tiles.  GROUPED_M counts its real row
  // tiles on the device (the host knows only a bound), so no round is spent
  // on empty tiles.
  //
  // Consecutive tiles of a workgroup overlap: once a tile's last stage has
  // been read, the ring slots not used for staging are refilled with the next
  // tile's first stages, which land while the epilogue runs.  (Loads and
  // stores share one counter on gfx9 and may complete out of order with
  // respect to each other, so each wave waits for its part of the next stage
  // 0 before its first store.)
  struct Ch {
    __device__ int operator()(int lo, int hi) const { return (hi - lo + BM - 1) / BM; }
  };
  struct NoPad {
    __device__ int operator()(int, int) const { return 0; }
  };
  // Group table (up to kTableGroups groups): g_hi[e] = hi(e) and, for
  // GROUPED_M, g_pre[e] = row tiles of groups before e (g_pre[E] = all), built
  // once per launch so a tile finds its group by a binary search in LDS.
  // More groups: the block-wide scan per tile (find_unit).
  constexpr int kTableGroups = 256;
  __shared__ int g_hi[kTableGroups];
  __shared__ int g_pre[kTableGroups + 1];
  const bool table = p.E <= kTableGroups;
  int skewed = 0;   // GROUPED_K: groups sorted by size, every other round backwards
  if (table) {
    __shared__ int s_tmp[4];
    const int t = threadIdx.x;
    const int v = t < p.E ? (p.offs != nullptr ? clamp_off(p.offs[t], p.M) : p.M) : 0;
    const int hi = block_scan_max<256>(v, s_tmp);
    if (t < p.E) g_hi[t] = hi;
    __syncthreads();
    if constexpr (MODE == 0) {
      const int lo = t == 0 ? 0 : g_hi[t - 1];
      const int cnt = t < p.E ? (hi - lo + BM - 1) / BM : 0;
      const int incl = block_scan_sum<256>(cnt, s_tmp);
      if (t < p.E) g_pre[t + 1] = incl;
      if (t == 0) g_pre[0] = 0;
      __syncthreads();
    } else {
      // GROUPED_K: a tile's cost grows with its group's token count.  When the
      // largest group holds more than twice the mean of the non-empty ones,
      // g_pre[r] = the group of rank r in decreasing token count (ties: lower
      // index first); tiles run in that order and the grid stride below runs
      // every other round backwards, so the long contractions come first and
      // even out across the CUs.  Otherwise g_pre[r] = r.
      __shared__ int s_skew;
      const int c = t < p.E ? hi - (t == 0 ? 0 : g_hi[t - 1]) : 0;
      const int cmax = block_scan_max<256>(c, s_tmp);
      const int nz = block_scan_sum<256>(c > 0 ? 1 : 0, s_tmp);
      if (t == 255) s_skew = (int64_t)cmax * nz > 2 * (int64_t)g_hi[p.E - 1] ? 1 : 0;
      __syncthreads();
      skewed = s_skew;
      if (t < p.E) {
        int rank = t;
        if (skewed) {
          rank = 0;
          for (int j = 0; j < p.E; ++j) {
            const int cj = g_hi[j] - (j == 0 ? 0 : g_hi[j - 1]);
            rank += cj > c || (cj == c && j < t) ? 1 : 0;
          }
        }
        g_pre[rank] = t;
      }
      __syncthreads();
    }
  }
  skewed = __builtin_amdgcn_readfirstlane(skewed);
  int row_units = p.row_units;
  if constexpr (MODE == 0) {
    constexpr int kFar = 1 << 30;
    row_units = table ? g_pre[p.E] : kFar - find_unit<256>(p.offs, p.E, p.M, kFar, Ch{}, NoPad{}).j;
    row_units = __builtin_amdgcn_readfirstlane(row_units);
  }
  const int ntiles = row_units * p.col_tiles;
  const int G = gridDim.x;
  auto tile_of = [&](int it) {
    int pos = (G & 7) == 0 ? (G >> 3) * (int)(blockIdx.x & 7) + (int)(blockIdx.x >> 3) : (int)blockIdx.x;
    if (skewed && (it & 1)) pos = G - 1 - pos;   // XCD x takes chunk 7 - x: still contiguous
    return G * it + pos;
  };
  // Contraction-contiguous row stride of both operands, output row stride and
  // e8m0 row length: fixed per launch.
  const int ld = MODE == 0 ? p.K : p.M;
  const int64_t out_ld = MODE == 0 ? p.N : p.K;
  // e8m0 row stride: a row's blocks (row-major), or one stage's four blocks (K4,
  // where the next stage of the same rows lies 4 * rows further on).
  const int sc_ld = SK == 2 ? 4 : (MODE == 0 ? p.K / 32 : p.M / 32);
  const uint32_t k4_p = SK == 2 ? (uint32_t)(4 * (MODE == 0 ? p.M : p.N)) : 0u;          // K4 stage stride, P
  const uint32_t k4_q = SK == 2 ? (uint32_t)(4 * (MODE == 0 ? (int64_t)p.E * p.N : p.K)) : 0u;   // and Q

  // Everything a tile needs, from its logical index.
  struct Tile {
    const uint8_t* P;       // first row of the row operand (A rows / output rows)
    const uint8_t* Q;       // first row of the column operand (B rows / output columns)
    const uint8_t* psc;     // e8m0 rows of P and Q
    const uint8_t* qsc;
    int64_t out_base;
    int pv, qv;             // valid rows of P and Q in the tile
    int c_lo, c_hi;         // contraction range
    int c_start, nk;        // first stage position (BK-aligned) and stage count
    const float* psf;       // fp32 scales of the tile's rows and columns
    const float* qsf;
  };
  __shared__ __attribute__((aligned(16))) float s_inv[2][SK == 0 ? BM + BN : 4];
  constexpr int SPT = (BM + BN + 255) / 256;   // fp32 scales per thread
  // Fill `tl` for logical tile L.  Every thread calls it (without a group
  // table it synchronizes the workgroup).
  auto setup = [&](int L, Tile& tl) {
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    // band, row unit and column tile of L without a division by a runtime
    // value in the common case (a loop-invariant reciprocal would occupy a
    // register across the whole tile loop)
    static_assert((kBandRows & (kBandRows - 1)) == 0, "band rows: a power of two");
    int ru, ct, grp = -1;
    if (MODE == 0 && table) {
      // GROUPED_M bands do not cross groups: a group's row tiles form bands
      // of kBandRows from its first one (the last band of a group shorter), so
      // the tiles an XCD runs together share one expert's weight panels.
      // Band [b0, b1) holds the logical tiles [b0 C, b1 C) (C column tiles).
      const int C = p.col_tiles;
      // L / C: a row unit of L's band (the magic needs C >= 2)
      const int u = C == 1 ? L : (int)__umulhi((uint32_t)L, p.col_magic);
      int a = 0, b = p.E;   // g_pre[a] <= u < g_pre[b]
      while (b - a > 1) {
        const int mid = (a + b) >> 1;
        if (g_pre[mid] <= u) a = mid;
        else b = mid;
      }
      const int b0 = g_pre[a] + ((u - g_pre[a]) & ~(kBandRows - 1));
      const int gsz = min(g_pre[a + 1] - b0, kBandRows);
      const int inband = L - b0 * C;
      if (gsz == kBandRows) {
        ru = b0 + (inband & (kBandRows - 1));
        ct = inband / kBandRows;
      } else {
        ru = b0 + inband % gsz;
        ct = inband / gsz;
      }
      grp = a;
    } else {
      const int band = (int)__umulhi((uint32_t)L, p.band_magic);
      const int first = band * kBandRows;
      const int gsz = min(row_units - first, kBandRows);
      const int inband = L - band * (kBandRows * p.col_tiles);
      if (gsz == kBandRows) {
        ru = first + (inband & (kBandRows - 1));
        ct = inband / kBandRows;
      } else {
        ru = first + inband % gsz;
        ct = inband / gsz;
      }
    }
    const float* psf = nullptr;   // fp32 scales of the tile's rows / columns
    const float* qsf = nullptr;
    if constexpr (MODE == 0) {
      Unit un;
      if (table) {
        const int a = grp;
        un = Unit{a, ru - g_pre[a], a == 0 ? 0 : g_hi[a - 1], g_hi[a], 0};
      } else {
        un = find_unit<256>(p.offs, p.E, p.M, ru, Ch{}, NoPad{});
      }
      const int e = max(un.e, 0);   // un.e >= 0: ru < row_units
      const int m0 = un.e < 0 ? 0 : un.lo + un.j * BM, n0 = ct * BN;
      tl.pv = un.e < 0 ? 0 : min(BM, un.hi - m0);
      tl.qv = min(BN, p.N - n0);
      tl.P = p.a + (int64_t)m0 * p.K;
      tl.Q = p.b + ((int64_t)e * p.N + n0) * p.K;
      tl.c_lo = 0;
      tl.c_hi = tl.pv > 0 ? p.K : 0;
      tl.out_base = (int64_t)m0 * p.N + n0;
      tl.psc = static_cast<const uint8_t*>(p.sa) + (int64_t)m0 * sc_ld;
      tl.qsc = static_cast<const uint8_t*>(p.sb) + ((int64_t)e * p.N + n0) * sc_ld;
      psf = static_cast<const float*>(p.sa) + m0;
      qsf = static_cast<const float*>(p.sb) + (int64_t)e * p.N + n0;
    } else {
      const int ntn = (p.N + BM - 1) / BM;
      const int e = table ? g_pre[ru / ntn] : ru / ntn;
      const int n0 = (ru % ntn) * BM, k0 = ct * BN;
      // group range of e: lo = max over j < e of clamp(offs[j]); hi = max(lo, clamp(offs[e]))
      int lo, hi;
      if (table) {
        lo = e == 0 ? 0 : g_hi[e - 1];
        hi = g_hi[e];
      } else {
        __shared__ int s_red[4];
        int m = 0;
        if (p.offs != nullptr)
          for (int jj = t; jj < e; jj += 256) m = max(m, clamp_off(p.offs[jj], p.M));
        m = (int)wave_max_u32((uint32_t)m);
        if (lane == 0) s_red[wave] = m;
        __syncthreads();
        lo = max(max(s_red[0], s_red[1]), max(s_red[2], s_red[3]));
        hi = p.offs != nullptr ? max(lo, clamp_off(p.offs[e], p.M)) : p.M;
        __syncthreads();   // s_red is reused by the next tile's setup
      }
      tl.pv = min(BM, p.N - n0);
      tl.qv = min(BN, p.K - k0);
      tl.P = p.a + (int64_t)n0 * p.M;
      tl.Q = p.b + (int64_t)k0 * p.M;
      tl.c_lo = lo;
      tl.c_hi = hi;
      tl.out_base = ((int64_t)e * p.N + n0) * p.K + k0;
      tl.psc = static_cast<const uint8_t*>(p.sa) + (int64_t)n0 * sc_ld;
      tl.qsc = static_cast<const uint8_t*>(p.sb) + (int64_t)k0 * sc_ld;
      psf = static_cast<const float*>(p.sa) + (int64_t)e * p.N + n0;
      qsf = static_cast<const float*>(p.sb) + (int64_t)e * p.K + k0;
    }
    // Stages start on BK-aligned contraction positions (whole cache lines when
    // the row stride is a multiple of 128); stage 0 may begin below c_lo and
    // the last may end past c_hi: those bytes are zeroed in LDS before use.
    tl.c_start = tl.c_lo & ~(BK - 1);
    tl.nk = tl.c_hi > tl.c_lo ? (tl.c_hi - tl.c_start + BK - 1) / BK : 0;
    // The description is workgroup-uniform (part of it came through LDS):
    // keep it in scalar registers.
    tl.P = uniform_ptr(tl.P);
    tl.Q = uniform_ptr(tl.Q);
    tl.psc = uniform_ptr(tl.psc);
    tl.qsc = uniform_ptr(tl.qsc);
    tl.out_base = uniform_i64(tl.out_base);
    tl.pv = __builtin_amdgcn_readfirstlane(tl.pv);
    tl.qv = __builtin_amdgcn_readfirstlane(tl.qv);
    tl.c_lo = __builtin_amdgcn_readfirstlane(tl.c_lo);
    tl.c_hi = __builtin_amdgcn_readfirstlane(tl.c_hi);
    tl.c_start = __builtin_amdgcn_readfirstlane(tl.c_start);
    tl.nk = __builtin_amdgcn_readfirstlane(tl.nk);
    tl.psf = psf;
    tl.qsf = qsf;
  };

  // Start loading a tile's fp32 scales straight into LDS (s_raw) with
  // direct-to-LDS loads, so no register holds them across the k loop (a
  // spilled one would force a full wait, draining the previous tile's stores,
  // right after its load).  Wave w loads entries 64 (w + 4 i) + lane, exactly
  // the entries its own threads turn into reciprocals (scale_commit, after a
  // full wait), so no barrier is needed in between.
  __shared__ __attribute__((aligned(16))) float s_raw[SK == 0 ? BM + BN : 4];
  auto load_scales = [&](const Tile& tl) {
    if constexpr (SK == 0) {
      int t_opq = threadIdx.x;
      asm volatile("" : "+v"(t_opq));
      const int lane = t_opq & 63, wave = __builtin_amdgcn_readfirstlane(t_opq >> 6);
      const int pv1 = max(tl.pv, 1) - 1, qv1 = max(tl.qv, 1) - 1;
      constexpr int NB = (BM + BN) / 64;   // 64-entry blocks
      static_for<(NB + 3) / 4>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        const int blk = wave + 4 * i;
        if (blk < NB) {
          const int idx = 64 * blk + lane;
          const float* src = idx < BM ? tl.psf + min(idx, pv1) : tl.qsf + min(idx - BM, qv1);
          dma_4(reinterpret_cast<const uint8_t*>(src), reinterpret_cast<uint8_t*>(s_raw) + 256 * blk);
        }
      });
    }
  };
  // Reciprocals of the scales in s_raw, into `sinv`.
  auto scale_commit = [&](float* sinv) {
    if constexpr (SK == 0) {
#pragma unroll
      for (int s = 0; s < SPT; ++s) {
        const int idx = threadIdx.x + 256 * s;
        if (idx < BM + BN) sinv[idx] = __frcp_rn(s_raw[idx]);
      }
    }
  };

  // ---------------------------------------------------------------- DMA global -> LDS
  // Wave `wave` moves 1 KiB blocks wave + 4 i (i < BPW) of each stage (the
  // first BPW_A lie in the A tile).  In a block, lane l fills LDS bytes
  // [16 l, 16 l + 16): tile row RPB * blk + l / CH at physical chunk l % CH,
  // i.e. logical chunk phys(row, l % CH) (the swizzle is an involution).  The
  // swizzle term depends on row bits that a block step of 4 * RPB rows never
  // changes, so the logical chunk is one per lane for all blocks.
  // Block i covers rows r0 + 4 RPB i; its 32-bit offset (host validation
  // bounds the row strides) is rebuilt for every stage from a copy of r0 that
  // the compiler cannot hoist, which keeps BPW loop-invariant offsets out of
  // the register file at the cost of a few VALU ops between MFMAs.  Checked
  // stages clamp positions past the range to the last chunk that overlaps it
  // (zeroed in LDS later), so every lane still issues one load per block (the
  // wait counts rely on it).
  // e8m0: load d (global index wave + 4 d) covers tile rows 64 (wave + 4 d)
  // + lane, one 4-byte word (the stage's four 32-blocks) per row; loads past
  // the tile fetch row 0 into spare LDS.  Row offsets are 32-bit from the
  // tile's (uniform) scale-row bases.
  auto scale_row_off = [&](const Tile& tl, int wave, int lane, int i) -> uint32_t {
    const int rb = 64 * (wave + 4 * i);                    // wave-uniform
    const bool in_a = rb < BM, in_b = !in_a && rb < SROWS;
    const int rr = in_a ? min(rb + lane, tl.pv - 1) : (in_b ? min(rb - BM + lane, tl.qv - 1) : 0);
    return (uint32_t)(rr * sc_ld);
  };
  auto issue_stage = [&](const Tile& tl, auto slot_tag, int kt, auto checked_tag, const uint32_t* soff = nullptr) {
    constexpr int S = decltype(slot_tag)::value;
    constexpr bool CHECKED = decltype(checked_tag)::value;
    int t_opq = threadIdx.x;
    asm volatile("" : "+v"(t_opq));
    const int lane = t_opq & 63, wave = __builtin_amdgcn_readfirstlane(t_opq >> 6);
    const int r0 = R::RPB * wave + lane / CH;
    const int lc16 = 16 * R::phys(r0, lane % CH);
    const int pv1 = tl.pv - 1, qv1 = tl.qv - 1;
    const int base = tl.c_start + kt * BK;
    uint32_t pos = (uint32_t)base;
    if constexpr (CHECKED) pos = (uint32_t)min(base + lc16, max((tl.c_hi - 1) & ~15, 0)) - (uint32_t)lc16;
    uint8_t* dst = slot_data[S];
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const uint32_t ro = i < BPW_A ? (uint32_t)(min(r0 + 4 * R::RPB * i, pv1) * ld + lc16)
                                    : (uint32_t)(min(r0 + 4 * R::RPB * (i - BPW_A), qv1) * ld + lc16);
      dma_16((i < BPW_A ? tl.P : tl.Q) + (ro + pos), dst + (wave + 4 * i) * 1024);
    }
    if constexpr (E8) {
      const uint32_t blk0 = (uint32_t)(base >> 5);
      uint8_t* sdst = slot_scale[S];
#pragma unroll
      for (int i = 0; i < SC_DMA; ++i) {
        const int rb = 64 * (wave + 4 * i);
        const bool in_q = rb >= BM && rb < SROWS;
        const uint8_t* sbase = in_q ? tl.qsc : tl.psc;
        const uint32_t so = soff != nullptr ? soff[i] : scale_row_off(tl, wave, lane, i);
        const uint32_t st_off = SK == 2 ? (blk0 >> 2) * (in_q ? k4_q : k4_p) : blk0;
        dma_4(sbase + (so + st_off), sdst + 256 * (wave + 4 * i));
      }
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using Checked = std::true_type;
  using Unchecked = std::false_type;

  // Wait until at most n later stages' loads are still outstanding.
  auto wait_stages = [&](int n) {
    if (n >= 3) wait_vmcnt<3 * LPS>();
    else if (n == 2) wait_vmcnt<2 * LPS>();
    else if (n == 1) wait_vmcnt<LPS>();
    else wait_vmcnt<0>();
  };

  Tile cur, nxt;
  if (tile_of(0) >= ntiles) return;
  setup(tile_of(0), cur);
  load_scales(cur);
  wait_vmcnt<0>();
  scale_commit(s_inv[0]);
  // Stage of step s in the processing order nk-1, 0, 1, ..., nk-2 (see below).
  auto first_stage = [](const Tile& tl, int s) { return s == 0 ? tl.nk - 1 : s - 1; };
  if (cur.nk > 0) {
    issue_stage(cur, I0{}, first_stage(cur, 0), Checked{});
    issue_stage(cur, I1{}, first_stage(cur, min(1, cur.nk - 1)), Checked{});
    if constexpr (SLOTS > 2)
      issue_stage(cur, std::integral_constant<int, 2>{}, first_stage(cur, min(2, cur.nk - 1)), Checked{});
    if constexpr (SLOTS > 3)
      issue_stage(cur, std::integral_constant<int, 3>{}, first_stage(cur, min(3, cur.nk - 1)), Checked{});
  }

  for (int it = 0;; ++it) {
  // A GROUPED_M tile with at most BM / 2 valid rows (a group's last, short
  // tile) runs HALF: the four waves share its first BM / 2 rows and each takes
  // a quarter of the columns, so no MFMA is spent on its padding rows; with at
  // most BM / 4 valid rows (256-row MX tiles) the waves share the first BM / 4.
  auto tile_body = [&](auto lay_tag) -> bool {
  constexpr int LAY = decltype(lay_tag)::value;
  constexpr bool HALF = LAY > 0;
  constexpr int TME = LAY == 2 ? TM / 2 : TM;                          // 32-row blocks per wave
  constexpr int TNE = HALF ? TN / 2 : TN, WNE = HALF ? WN / 2 : WN;   // column blocks and columns per wave
  constexpr int NME = TME * TNE, NDE = 2 * (TME + TNE), ND0E = NDE + (E8 ? TME + TNE : 0);
  // Thread indices pass through an opaque copy each tile, so the compiler
  // derives per-lane addresses inside the tile instead of hoisting (and
  // spilling) all of them across the tile loop.
  int t_opq = threadIdx.x;
  asm volatile("" : "+v"(t_opq));
  const int t = t_opq, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // wave-uniform: scalar registers
  const int wm = HALF ? 0 : wave >> 1, wn = HALF ? wave : wave & 1;
  const int c_lo = cur.c_lo, c_hi = cur.c_hi, c_start = cur.c_start, nk = cur.nk;
  const float* const sinv = s_inv[it & 1];
  uint32_t soff[E8 ? SC_DMA : 1];
  if constexpr (E8) {
#pragma unroll
    for (int i = 0; i < SC_DMA; ++i) soff[i] = scale_row_off(cur, wave, lane, i);
  }

  // Zero the bytes of every chunk of stage kt (in LDS `st`) outside or
  // straddling [c_lo, c_hi).  Only the first and last stage can hold such chunks.
  auto fix_boundary = [&](uint8_t* st, int kt) {
    const int base = c_start + kt * BK;
    if (kt >= nk || (base >= c_lo && base + BK <= c_hi)) return;    // uniform
    zero_outside_ring<R, SROWS, CH>(st, base, c_lo, c_hi);
    wait_lgkmcnt0();
    raw_barrier();
  };

  v16f acc[TME][TNE];
#pragma unroll
  for (int i = 0; i < TME; ++i)
#pragma unroll
    for (int j = 0; j < TNE; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int g = lane >> 5, lrow = lane & 31;
  // Two register sets of MFMA fragments (one 64-byte k step each).
  v8i fa[2][TME], fb[2][TNE];
  // e8m0 scale operands: byte i of ea[set] is fragment i's scale (the MFMA
  // picks it with op_sel), likewise eb.  In LDS a tile row's four scale bytes
  // of a stage are one word, byte 2 h + b for 32-block b of k step h, and the
  // lane supplies block b = g of its row.  A stage's first k step reads the
  // word of each fragment row once (ahead of that step's fragment reads) and
  // packs the bytes of both k steps with byte permutes; the second k step's
  // operands wait in ea_n / eb_n.
  static_assert((TME == 4 || TME == 2) && (TNE == 4 || TNE == 2), "at most four scale bytes per register");
  int ea[2], eb[2], ea_n = 0, eb_n = 0;
  // byte selectors: t = [w0.b(g), w1.b(g), w0.b(2+g), w1.b(2+g)] from words w0 (low), w1
  const uint32_t sel_pair = 0x06020400u + 0x01010101u * (uint32_t)g;
  // Four words of one operand's fragment rows -> (k step 0 bytes, k step 1 bytes), byte i = row i.
  auto pack4 = [&](const uint32_t (&w)[4], int& k0, int& k1) {
    const uint32_t t01 = __builtin_amdgcn_perm(w[1], w[0], sel_pair);
    const uint32_t t23 = __builtin_amdgcn_perm(w[3], w[2], sel_pair);
    k0 = (int)__builtin_amdgcn_perm(t23, t01, 0x05040100u);
    k1 = (int)__builtin_amdgcn_perm(t23, t01, 0x07060302u);
  };
  auto pack2 = [&](const uint32_t (&w)[4], int& k0, int& k1) {
    const uint32_t t01 = __builtin_amdgcn_perm(w[1], w[0], sel_pair);
    k0 = (int)t01;
    k1 = (int)(t01 >> 16);
  };
  // Fragments of k step h of the stage in LDS `st` (scales in `sc`) into set SET.
  auto rd = [&](auto set_tag, const uint8_t* st, const uint8_t* sc, int h) {
    constexpr int SET = decltype(set_tag)::value;
    uint32_t wa[4] = {0u, 0u, 0u, 0u}, wb[4] = {0u, 0u, 0u, 0u};
    if constexpr (E8) {
      if (h == 0) {
#pragma unroll
        for (int i = 0; i < TME; ++i)
          wa[i] = *reinterpret_cast<const uint32_t*>(sc + 4 * (wm * WM + 32 * i + lrow));
#pragma unroll
        for (int j = 0; j < TNE; ++j)
          wb[j] = *reinterpret_cast<const uint32_t*>(sc + 4 * (BM + wn * WNE + 32 * j + lrow));
      }
    }
#pragma unroll
    for (int i = 0; i < TME; ++i) {
      const int r = wm * WM + 32 * i + lrow;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(st + R::off(r, 4 * h + g));
      const u32x4 hi = *reinterpret_cast<const u32x4*>(st + R::off(r, 4 * h + 2 + g));
      fa[SET][i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int j = 0; j < TNE; ++j) {
      const int r = wn * WNE + 32 * j + lrow;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(st + A_BYTES + R::off(r, 4 * h + g));
      const u32x4 hi = *reinterpret_cast<const u32x4*>(st + A_BYTES + R::off(r, 4 * h + 2 + g));
      fb[SET][j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    if constexpr (E8) {
      if (h == 0) {
        if constexpr (TME == 4) pack4(wa, ea[SET], ea_n);
        else pack2(wa, ea[SET], ea_n);
        if constexpr (TNE == 4) pack4(wb, eb[SET], eb_n);
        else pack2(wb, eb[SET], eb_n);
      } else {
        ea[SET] = ea_n;
        eb[SET] = eb_n;
      }
    }
  };
  auto mma = [&](auto set_tag) {
    constexpr int SET = decltype(set_tag)::value;
    static_for<TME>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      static_for<TNE>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        // B fragment first: the 32x32 result then holds output row (lane & 31)
        // and output columns 8 (v / 4) + 4 (lane >> 5) + v % 4 in register v,
        // i.e. four consecutive columns per register quad (the epilogue packs them).
        if constexpr (E8)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[SET][j], fa[SET][i], acc[i][j], 0, 0, j,
                                                                      eb[SET], i, ea[SET]);
        else
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[SET][j], fa[SET][i], acc[i][j], 0, 0, 0, 0,
                                                                      0, 0);
      });
    });
  };

  // k steps of stage kt (ring slot S) before its last: read the next k step of
  // the same stage into the other set while this one's MFMAs issue.
  auto inner_halves = [&](auto slot_tag) {
    constexpr int S = decltype(slot_tag)::value;
    if constexpr (KS == 2) {
      constexpr int CUR = (S * KS) & 1;
      rd(std::integral_constant<int, 1 - CUR>{}, slot_data[S], slot_scale[S], 1);
      mma(std::integral_constant<int, CUR>{});
      interleave<NME, NDE, 0>();
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Stages are processed in the order nk-1, 0, 1, ..., nk-2: the two that can
  // straddle the contraction range (the last and the first) come first and
  // are fixed up before the uniform steps start.
  auto stage_of = [&](int s) { return s == 0 ? nk - 1 : s - 1; };
  // Step s of the order, stage stage_of(s) in ring slot S (== s % SLOTS), the
  // same code for the whole range so it stays branch-free and interleaved:
  //  1. k steps of the stage but the last;
  //  2. wait for step s+1's stage and this wave's reads of slot S, barrier
  //     (that stage visible everywhere; no wave still reads slot S); the
  //     first step also zeroes the out-of-range bytes of the next stage;
  //  3. refill slot S with the stage of step min(s+SLOTS, nk-1) (past the end a
  //     reload that nothing reads, so every step issues the same loads and
  //     every wait count is static), read the next stage's first k step into
  //     the other set and run the last k step's MFMAs, all interleaved.
  auto step = [&](auto slot_tag, int kt, auto fix_tag) {
    constexpr int S = decltype(slot_tag)::value, NS = (S + 1) % SLOTS;
    constexpr int CUR = (S * KS + KS - 1) & 1;
    inner_halves(slot_tag);
    wait_lgkmcnt0();
    // The tile's first step needs no stage wait: every wave waited for its
    // part of the next stage before the tile-start barrier (in the prologue or
    // in the previous epilogue), so the epilogue's stores are not drained here.
    if constexpr (!decltype(fix_tag)::value) wait_vmcnt<(SLOTS - 2) * LPS>();
    raw_barrier();
    if constexpr (decltype(fix_tag)::value) {
      if (kt + 1 < nk) fix_boundary(slot_data[NS], stage_of(kt + 1));
    }
    issue_stage(cur, slot_tag, stage_of(min(kt + SLOTS, nk - 1)), Checked{}, soff);
    rd(std::integral_constant<int, 1 - CUR>{}, slot_data[NS], slot_scale[NS], 0);
    mma(std::integral_constant<int, CUR>{});
    interleave<NME, ND0E, LPS>();
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- start of the tile.  First tile: stages 0 .. SLOTS-1 are in flight;
  // wait for stages 0 and 1.  Later tiles: stages 0 .. NPRE-1 were issued
  // before the previous epilogue, and every wave already waited for its part
  // of them there (before that epilogue's stores, which may complete in any
  // order with respect to loads); refill the staging slot, if the ring has one.
  if (it == 0) wait_vmcnt<(SLOTS - 2) * LPS>();
  raw_barrier();
  // The next tile's description now, and its scale loads (issued before this
  // tile's later stages, so they land first and never delay a stage wait).
  const bool has_next = tile_of(it + 1) < ntiles;
  if (has_next) {
    setup(tile_of(it + 1), nxt);
    load_scales(nxt);
  }
  if (it > 0 && nk > 0) {
    static_for<SLOTS - NPRE>([&](auto sc) {
      constexpr int S = NPRE + decltype(sc)::value;
      issue_stage(cur, std::integral_constant<int, S>{}, first_stage(cur, min(S, nk - 1)), Checked{});
    });
  }
  if (nk > 0) {
    fix_boundary(slot_data[0], nk - 1);
    rd(I0{}, slot_data[0], slot_scale[0], 0);
  }
  // Step 0 (with the fix-up of the next stage), then whole rounds of SLOTS
  // steps (static slots 1, 2, ..., 0), then the partial round.
  using Fix = std::true_type;
  using NoFix = std::false_type;
  if (nk > 0) step(I0{}, 0, Fix{});
  int kt = 1;
  for (; kt + SLOTS <= nk; kt += SLOTS) {
    step(I1{}, kt, NoFix{});
    if constexpr (SLOTS > 2) step(std::integral_constant<int, 2>{}, kt + 1, NoFix{});
    if constexpr (SLOTS > 3) step(std::integral_constant<int, 3>{}, kt + 2, NoFix{});
    step(I0{}, kt + SLOTS - 1, NoFix{});
  }
  if (kt < nk) {
    step(I1{}, kt, NoFix{});
    if constexpr (SLOTS > 2) if (kt + 1 < nk) step(std::integral_constant<int, 2>{}, kt + 1, NoFix{});
    if constexpr (SLOTS > 3) if (kt + 2 < nk) step(std::integral_constant<int, 3>{}, kt + 2, NoFix{});
  }
  wait_vmcnt<0>();   // the reloads past the end land before their slots are reused

  // ---- the next tile: its scale reciprocals, then (once no wave reads the
  // ring any more) its first stages, which land during the epilogue.
  if (has_next) scale_commit(s_inv[(it + 1) & 1]);
  wait_lgkmcnt0();
  raw_barrier();
  if (has_next && nxt.nk > 0) {
    static_for<NPRE>([&](auto sc) {
      constexpr int S = decltype(sc)::value;
      issue_stage(nxt, std::integral_constant<int, S>{}, first_stage(nxt, min(S, nxt.nk - 1)), Checked{});
    });
  }

  // ---------------------------------------------------------------- epilogue
  // fp32 scales are multipliers of the quantized operands: divide by both
  // (reciprocals were loaded with the tile's description).  An empty
  // contraction range gives zeros (its reciprocals are zeroed too, so no
  // 0 * inf appears).
  const int p_valid = cur.pv, q_valid = cur.qv;
  const int64_t out_base = cur.out_base;
  const float keep = c_hi > c_lo ? 1.0f : 0.0f;
  constexpr int ELEM = OUT == 0 ? 2 : 4;
  if ((out_ld * ELEM) % 16 == 0) {
    // Lane indices from a fresh opaque copy of the thread index: values kept
    // across the k loop may be spilled, and a reload would wait for the
    // stages now in flight.
    int t_epi = threadIdx.x;
    asm volatile("" : "+v"(t_epi));
    const int lane = t_epi & 63, g = lane >> 5, lrow = lane & 31;
    // Each pass stages one 32-row block of a wave's results, PC columns wide
    // (128 bytes per row), and writes whole 128-byte row segments.  A lane
    // holds four consecutive columns of one row per register quad: bf16
    // packs them into 8 bytes, written at unit u ^ (row & 14) of its staged
    // row (fp32: 16 bytes at unit u ^ (row & 7)).  The even mask keeps the two
    // 8-byte halves of a 16-byte chunk (lanes g = 0, 1 of one row) in order,
    // and rows 0..15 of one write instruction still cover all 64 banks once
    // (row parity picks the bank half, row & 14 the chunk), so the 512 bytes
    // take the minimum two cycles; 8 lanes read back one whole row, logical
    // chunk k at physical chunk k ^ ((row & 14) >> 1).
    // LDS accesses go through lds_* while the next tile's stages land.
    constexpr int PC = 128 / ELEM;              // output columns per pass
    constexpr int JPP = PC / 32;                // 32-column blocks per pass
    constexpr int VEC = 16 / ELEM;              // elements per 16-byte piece
    uint8_t* const stg = (SLOTS == 2 ? stg_own : slot_data[SLOTS - 1]) + wave * kStgWave;
    const uint32_t stg_l = lds_off(stg), sinv_l = lds_off(sinv);
    const bool full = p_valid == BM && q_valid == BN;
    const int rr = lane >> 3, k = lane & 7;     // read-back: staged row 8 itr + rr, chunk k
    constexpr int NP = TME * (TNE / JPP);         // passes
    // GROUPED_M with bf16 output: the read-back pieces of every pass are held
    // (128 registers, where the dead MFMA fragments were) and stored together
    // once the next tile's stages have landed.  Otherwise (measured slower for
    // the short weight-gradient tiles, whose next k step then waits for the
    // whole burst of stores; too many registers for fp32) the pieces of the
    // last two passes, each pass's stores issued behind the next one's LDS work.
    constexpr bool HOLD = MODE == 0 && NP <= 8;
    constexpr int ND_ = HOLD ? NP : 2;
    lds_u4 dv[ND_][4];
    // Stores of pass n (32-row block n % TME, columns PC (n / TME) ..), once
    // its read-back has landed.  All pre-issued stages of the next tile (this
    // wave's part) land before the first store: until then only loads are in
    // flight, and they complete in order.
    auto store_pass = [&](auto nc) {
      constexpr int n = decltype(nc)::value, i = n % TME, jp = n / TME;
      constexpr int d = HOLD ? n : (n & 1);
#pragma unroll
      for (int itr = 0; itr < 4; ++itr) lds_ready(dv[d][itr]);
      if constexpr (!HOLD && n == 0) wait_vmcnt<0>();
      const int c = wn * WNE + PC * jp + VEC * k;
      uint8_t* const row0 = static_cast<uint8_t*>(p.out) +
                            (out_base + (int64_t)(wm * WM + 32 * i + rr) * out_ld + c) * ELEM;
      if (full) {
#pragma unroll
        for (int itr = 0; itr < 4; ++itr)
          store_stream16(row0 + (int64_t)itr * 8 * out_ld * ELEM, __builtin_bit_cast(u32x4, dv[d][itr]));
        return;
      }
#pragma unroll
      for (int itr = 0; itr < 4; ++itr) {
        const int r = wm * WM + 32 * i + 8 * itr + rr;
        if (r >= p_valid) continue;
        uint8_t* dst = row0 + (int64_t)itr * 8 * out_ld * ELEM;
        const lds_u4 dd = dv[d][itr];
        if (c + VEC <= q_valid) {
          store_stream16(dst, __builtin_bit_cast(u32x4, dd));
        } else {
          const uint32_t w[4] = {dd.x, dd.y, dd.z, dd.w};
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            if (c + e >= q_valid) break;
            if constexpr (OUT == 0)
              reinterpret_cast<uint16_t*>(dst)[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
            else
              reinterpret_cast<uint32_t*>(dst)[e] = w[e];
          }
        }
      }
    };
    static_for<TNE / JPP>([&](auto jpc) {
      constexpr int jp = decltype(jpc)::value;
      // reciprocals of the lane's columns in this pass (register quad q of
      // block jj: columns 32 jj + 8 q + 4 g + e of the pass) and of its rows
      f32x4 inv_q[JPP][4];
      float inv_p[TME];
      if constexpr (SK == 0) {
        lds_u4 rq[JPP][4];
        uint32_t rp[TME];
#pragma unroll
        for (int jj = 0; jj < JPP; ++jj)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            rq[jj][q] = lds_read16(sinv_l + 4 * (BM + wn * WNE + 32 * (JPP * jp + jj) + 8 * q + 4 * g));
#pragma unroll
        for (int i = 0; i < TME; ++i) rp[i] = lds_read4(sinv_l + 4 * (wm * WM + 32 * i + lrow));
        lds_wait();
#pragma unroll
        for (int jj = 0; jj < JPP; ++jj)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            lds_ready(rq[jj][q]);
            inv_q[jj][q] = __builtin_bit_cast(f32x4, rq[jj][q]) * keep;
          }
#pragma unroll
        for (int i = 0; i < TME; ++i) {
          lds_ready(rp[i]);
          inv_p[i] = __builtin_bit_cast(float, rp[i]) * keep;
        }
      } else {
#pragma unroll
        for (int jj = 0; jj < JPP; ++jj)
#pragma unroll
          for (int q = 0; q < 4; ++q) inv_q[jj][q] = f32x4{keep, keep, keep, keep};
#pragma unroll
        for (int i = 0; i < TME; ++i) inv_p[i] = 1.0f;
      }
      static_for<TME>([&](auto ic) {
        constexpr int i = decltype(ic)::value, n = TME * jp + i;   // pass n
        // stage: block (i, JPP jp + jj), quad q -> staged row lrow
#pragma unroll
        for (int jj = 0; jj < JPP; ++jj) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            f32x4 v;
            // e8m0 scales were applied inside the MFMAs; an empty contraction
            // range leaves the zero accumulators untouched
#pragma unroll
            for (int e = 0; e < 4; ++e)
              v[e] = SK == 0 ? acc[i][JPP * jp + jj][4 * q + e] * inv_p[i] * inv_q[jj][q][e]
                             : acc[i][JPP * jp + jj][4 * q + e];
            const int u = 8 * jj + 2 * q + g;
            if constexpr (OUT == 0) {
              const bf16x2 lo = __builtin_convertvector(f32x2{v[0], v[1]}, bf16x2);
              const bf16x2 hi = __builtin_convertvector(f32x2{v[2], v[3]}, bf16x2);
              lds_write8(stg_l + lrow * 128 + ((u ^ (lrow & 14)) << 3),
                         lds_u2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)});
            } else {
              lds_write16(stg_l + lrow * 128 + ((u ^ (lrow & 7)) << 4), __builtin_bit_cast(lds_u4, v));
            }
          }
        }
        // read back whole 16-byte pieces: 8 lanes per staged row.  (A wave's
        // LDS accesses execute in order, so these reads see this pass's
        // writes and the previous pass's reads saw its own.)
#pragma unroll
        for (int itr = 0; itr < 4; ++itr) {
          const int lr = 8 * itr + rr;
          const int pc = OUT == 0 ? (k ^ ((lr & 14) >> 1)) : (k ^ (lr & 7));
          if constexpr (HOLD)
            dv[n][itr] = *reinterpret_cast<const lds_u4*>(stg + lr * 128 + (pc << 4));
          else
            dv[n & 1][itr] = lds_read16(stg_l + lr * 128 + (pc << 4));
        }
        // fp32: the previous pass's pieces leave now, behind this pass's LDS work
        if constexpr (!HOLD && n > 0) {
          wait_lgkmcnt<4 * JPP + 4>();
          store_pass(std::integral_constant<int, n - 1>{});
        }
      });
    });
    wait_lgkmcnt<0>();
    if constexpr (HOLD) {
      // bf16: every pass was staged and read back before the first store, so
      // the conversion ran while the next tile's stages were still landing.
      wait_vmcnt<0>();
      static_for<NP>([&](auto nc) { store_pass(nc); });
    } else {
      store_pass(std::integral_constant<int, NP - 1>{});
    }
  } else {
    // Output rows not 16-byte aligned: element stores straight from registers.
    wait_vmcnt<0>();   // the next tile's pre-issued stages (older than any store below)
    auto quad = [&](int i, int j, int q, float inv_p, const float* inv_q) {
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e] * inv_p * inv_q[4 * q + e];
      return v;
    };
#pragma unroll
    for (int j = 0; j < TNE; ++j) {
      float inv_q[16];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int cc = min(wn * WNE + 32 * j + 8 * q + 4 * g + e, BN - 1);
          inv_q[4 * q + e] = (SK == 0 ? sinv[BM + cc] : 1.0f) * keep;
        }
#pragma unroll
      for (int i = 0; i < TME; ++i) {
        const int r = wm * WM + 32 * i + lrow;
        const float inv_p = (SK == 0 ? sinv[r] : 1.0f) * keep;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 v = quad(i, j, q, inv_p, inv_q);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int c = wn * WNE + 32 * j + 8 * q + 4 * g + e;
            if (r >= p_valid || c >= q_valid) continue;
            const int64_t o = out_base + (int64_t)r * out_ld + c;
            if constexpr (OUT == 0)
              static_cast<__bf16*>(p.out)[o] = (__bf16)v[e];
            else
              static_cast<float*>(p.out)[o] = v[e];
          }
        }
      }
    }
  }
  return has_next;
  };
  bool has_next;
  if constexpr (MODE == 0) {
    // Quarter layout for MX operands only: the FP8 kernels measured slower
    // with the third tile body beside the other two.
    bool quarter = false;
    if constexpr (TM == 4 && E8) {
      quarter = cur.pv <= BM / 4;
      if (quarter) has_next = tile_body(std::integral_constant<int, 2>{});
    }
    if (!quarter) {
      if (cur.pv <= BM / 2) has_next = tile_body(std::integral_constant<int, 1>{});
      else has_next = tile_body(std::integral_constant<int, 0>{});
    }
  } else {
    has_next = tile_body(std::integral_constant<int, 0>{});
  }
  if (!has_next) break;
  cur = nxt;
  }   // tile loop
}

static void fill_params(KParams& p, const GemmArgs& g, int BM, int BN) {
  p.a = static_cast<const uint8_t*>(g.a);
  p.b = static_cast<const uint8_t*>(g.b);
  p.sa = g.sa;
  p.sb = g.sb;
  p.offs = g.offs;
  p.out = g.out;
  p.E = g.n_groups;
  p.M = (int)g.M;
  p.N = (int)g.N;
  p.K = (int)g.K;
  if (g.mode == 0) {
    p.row_units = (int)((g.M + BM - 1) / BM + g.n_groups);
    p.col_tiles = (int)((g.N + BN - 1) / BN);
  } else {
    p.row_units = (int)(g.n_groups * ((g.N + BM - 1) / BM));
    p.col_tiles = (int)((g.K + BN - 1) / BN);
  }
  const uint64_t band_tiles = (uint64_t)kBandRows * (uint64_t)std::max(p.col_tiles, 1);
  p.band_magic = (uint32_t)(((1ull << 32) + band_tiles - 1) / band_tiles);
  const uint64_t ct = (uint64_t)p.col_tiles;
  p.col_magic = ct >= 2 ? (uint32_t)(((1ull << 32) + ct - 1) / ct) : 0u;   // unused below 2
}

// The band magic is exact for every tile index below 2^32 / (kBandRows * col_tiles).
static bool band_magic_exact(const KParams& p) {
  return (uint64_t)p.row_units * (uint64_t)p.col_tiles * (uint64_t)kBandRows * (uint64_t)p.col_tiles < (1ull << 32);
}

// 64-byte-stage kernel with byte-wise e8m0 loads: MX operands whose scale rows
// are not 4-byte aligned per 128-byte stage.
template <int BM, int BN, int MODE, int OUT>
static hipError_t launch_mx_bytewise(const GemmArgs& g, hipStream_t st) {
  KParams p;
  fill_params(p, g, BM, BN);
  const int64_t total = (int64_t)p.row_units * p.col_tiles;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_fp8_kernel<BM, BN, kGemmStageBytes, MODE, 1, OUT>), dim3((unsigned)total), dim3(256), 0, st, p);
  return hipGetLastError();
}

// Compute units of the current device (cached per device).
static int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

template <int BM, int BN, int BK, int SLOTS, int MODE, int SK, int OUT>
static hipError_t launch_pipe(const GemmArgs& g, hipStream_t st) {
  KParams p;
  fill_params(p, g, BM, BN);
  const int64_t total = (int64_t)p.row_units * p.col_tiles;   // GROUPED_M: a bound
  if (total == 0) return hipSuccess;
  if (!band_magic_exact(p)) return hipErrorInvalidValue;   // far beyond any expert layer
  // One workgroup fits per CU (LDS); a persistent grid of at most one per CU.
  const int64_t grid = std::min<int64_t>(total, cu_count());
  hipLaunchKernelGGL((gemm_fp8_pipe<BM, BN, BK, SLOTS, MODE, SK, OUT>), dim3((unsigned)grid), dim3(256), 0, st, p);
  return hipGetLastError();
}

// GROUPED_K with one group and fp32 scales (a dense weight gradient): when the
// 256x256 tiles leave the last round of the persistent grid at most half full,
// that round would cost as much as a full one.  The output rows then split into
// whole rounds of 256-row tiles and a tail of 128-row tiles, a second launch
// that fills the CUs again with tiles of half the work.  Returns false when the
// shape does not call for it (nothing launched).
template <int OUT>
static bool launch_k_round_split(const GemmArgs& g, hipStream_t st, hipError_t* err) {
  const int64_t G = cu_count();
  const int64_t rt = (g.N + 255) / 256, ct = (g.K + 255) / 256, tiles = rt * ct;
  const int64_t rem = tiles % G;
  if (g.n_groups != 1 || tiles < 2 * G || rem == 0 || rem > G / 2) return false;
  const int64_t r1 = tiles / G * G / ct;   // 256-row units that make whole rounds
  if (r1 <= 0 || r1 >= rt) return false;
  const int64_t n0 = r1 * 256;
  constexpr int64_t ELEM = OUT == 0 ? 2 : 4;
  GemmArgs head = g, tail = g;
  head.N = n0;
  tail.N = g.N - n0;
  tail.a = static_cast<const uint8_t*>(g.a) + n0 * g.M;          // A phys [N][M]
  tail.sa = static_cast<const float*>(g.sa) + n0;                  // fp32 [1][N]
  tail.out = static_cast<uint8_t*>(g.out) + n0 * g.K * ELEM;       // out [1][N][K]
  *err = launch_pipe<256, 256, 128, 2, 1, 0, OUT>(head, st);
  if (*err == hipSuccess) *err = launch_pipe<128, 256, 128, 3, 1, 0, OUT>(tail, st);
  return true;
}

template <int MODE, int SK, int OUT>
static hipError_t pick_tile(const GemmArgs& g, hipStream_t st) {
  // GROUPED_M with small average groups wastes less of a 128-row tile.
  const bool small = MODE == 0 && g.n_groups > 1 && g.M / g.n_groups < 512;
  if constexpr (SK == 1) {
    // Each 128-byte stage takes one aligned 4-byte word of every e8m0 row.
    const int64_t clen = MODE == 0 ? g.K : g.M;
    const bool aligned = clen % 128 == 0 && (reinterpret_cast<uintptr_t>(g.sa) & 3) == 0 &&
                         (reinterpret_cast<uintptr_t>(g.sb) & 3) == 0;
    if (!aligned)
      return small ? launch_mx_bytewise<128, 256, MODE, OUT>(g, st) : launch_mx_bytewise<256, 256, MODE, OUT>(g, st);
  }
  if constexpr (MODE == 1 && SK == 0) {
    hipError_t err = hipSuccess;
    if (launch_k_round_split<OUT>(g, st, &err)) return err;
  }
  return small ? launch_pipe<128, 256, 128, 3, MODE, SK, OUT>(g, st)
               : launch_pipe<256, 256, 128, 2, MODE, SK, OUT>(g, st);
}

template <int MODE>
static hipError_t dispatch_fp8(const GemmArgs& g, hipStream_t st) {
  if (g.scale_kind == 1)
    return g.out_dtype == 0 ? pick_tile<MODE, 1, 0>(g, st) : pick_tile<MODE, 1, 1>(g, st);
  if (g.scale_kind == 3)   // e8m0 in the K4 layout: every contraction length takes the pipeline
    return g.out_dtype == 0 ? pick_tile<MODE, 2, 0>(g, st) : pick_tile<MODE, 2, 1>(g, st);
  return g.out_dtype == 0 ? pick_tile<MODE, 0, 0>(g, st) : pick_tile<MODE, 0, 1>(g, st);
}

hipError_t launch_grouped_mm_bf16(const GemmArgs& g, hipStream_t st);

hipError_t launch_grouped_mm(const GemmArgs& g, hipStream_t st) {
  const bool fn = g.a_fmt == 0 && g.b_fmt == 0;
  if (g.a_fmt == 2 || !fn) return launch_grouped_mm_bf16(g, st);
  if (g.M == 0 && g.mode == 0) return hipSuccess;
  return g.mode == 0 ? dispatch_fp8<0>(g, st) : dispatch_fp8<1>(g, st);
}

}  // namespace fp8moe

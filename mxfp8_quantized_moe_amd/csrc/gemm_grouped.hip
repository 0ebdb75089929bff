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
// Tiling, derived from the hardware rather than searched:
//  * v_mfma_scale_f32_32x32x64_f8f6f4: each lane holds one row (lane & 31) and
//    two 16-byte halves of the 64-wide contraction at byte offsets 16*g and
//    32 + 16*g (g = lane >> 5); the e8m0 scale of (row i, 32-block b) comes
//    from lane i + 32*b.  The 32x32 fp32 result sits in 16 registers: column
//    lane & 31, row 8*(v/4) + 4*(lane>>5) + v%4.
//  * 256 threads = 2x2 waves; a wave owns (BM/2) x (BN/2) outputs.  BM = BN =
//    256 gives 4x4 MFMA tiles per wave = 256 fp32 accumulators per lane, the
//    largest tile that fits one wave per SIMD (512 registers) and makes each
//    byte read from LDS feed 128 flops per wave.
//  * With one wave per SIMD nothing else hides memory latency, so operands
//    stream through a 4-slot LDS ring of 64-byte contraction stages
//    ((BM + BN) x 64 B = 32 KiB per stage, 128 KiB in all) with 4 stages in
//    flight: gfx950's direct global->LDS loads (global_load_lds_dwordx4) move
//    the data without staging registers, one barrier per stage.  MFMA
//    fragments are double-buffered in registers: stage k's MFMAs issue while
//    stage k+1's fragments are read, so LDS latency stays off the MFMA path.
//  * LDS rows are 64 B (4 chunks of 16 B); chunk c of row r is stored at chunk
//    c ^ ((r >> 2) & 3), so 16 consecutive lanes reading one logical chunk of
//    16 consecutive rows touch 16 distinct 16-byte bank groups.  A wave's
//    DMA fills 1 KiB contiguously (16 rows); each lane fetches the global chunk
//    that belongs at its LDS slot, which realises the swizzle for free.
//  * Small groups (average rows per group below 512) use BM = 128 to waste
//    less of each tile on padding rows.
//  * Workgroups are numbered so that each XCD (round-robin dispatch over 8)
//    gets a contiguous range of tiles, ordered in bands of 8 row tiles, so the
//    tiles running together on one XCD share operand rows in its L2.
#include "device_common.hpp"
#include "kernels.hpp"

namespace fp8moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

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

// s_waitcnt immediates (gfx9 encoding: vmcnt bits [3:0] and [15:14], expcnt [6:4],
// lgkmcnt [11:8]).  The builtin is visible to the compiler's own wait
// insertion, which then knows which direct-to-LDS loads have landed.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4)); }

// Direct global->LDS loads (a wave fills 64 consecutive 16-byte or 1-byte LDS
// slots, one per lane, from per-lane global addresses).  Wrapped in plain
// device functions: clang drops a kernel's host launch stub when this builtin
// is called straight from a generic lambda in the kernel body.
__device__ __forceinline__ void dma_16(const uint8_t* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}
// A 1-byte DMA still gives each lane a dword of LDS: lane l's byte lands at dst + 4 l.
__device__ __forceinline__ void dma_1(const uint8_t* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 1, 0, 0);
}

// Workgroup barrier without a memory fence (a fence would wait for every
// in-flight global load, draining the pipeline); the empty asm statements keep
// the compiler from moving memory accesses across it.
__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

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
    for (int idx = t; idx < SROWS * CH; idx += 256) {
      const int r = idx / CH, c = idx % CH, pos = base + 16 * c;
      if (pos < c_lo || pos + 16 > c_hi) {
        u32x4* q = reinterpret_cast<u32x4*>(st + R::off(r, c));
        *q = mask_chunk(*q, pos, c_lo, c_hi);
      }
    }
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

template <int BM, int BN, int MODE, int SK, int OUT>
static hipError_t launch_fp8(const GemmArgs& g, hipStream_t st) {
  KParams p;
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
  if (MODE == 0) {
    p.row_units = (int)((g.M + BM - 1) / BM + g.n_groups);
    p.col_tiles = (int)((g.N + BN - 1) / BN);
  } else {
    p.row_units = (int)(g.n_groups * ((g.N + BM - 1) / BM));
    p.col_tiles = (int)((g.K + BN - 1) / BN);
  }
  const int64_t total = (int64_t)p.row_units * p.col_tiles;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_fp8_kernel<BM, BN, kGemmStageBytes, MODE, SK, OUT>), dim3((unsigned)total), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <int MODE, int SK, int OUT>
static hipError_t pick_tile(const GemmArgs& g, hipStream_t st) {
  // GROUPED_M with small average groups wastes less of a 128-row tile.
  const bool small = MODE == 0 && g.n_groups > 1 && g.M / g.n_groups < 512;
  return small ? launch_fp8<128, 256, MODE, SK, OUT>(g, st) : launch_fp8<256, 256, MODE, SK, OUT>(g, st);
}

template <int MODE>
static hipError_t dispatch_fp8(const GemmArgs& g, hipStream_t st) {
  if (g.scale_kind == 1)
    return g.out_dtype == 0 ? pick_tile<MODE, 1, 0>(g, st) : pick_tile<MODE, 1, 1>(g, st);
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

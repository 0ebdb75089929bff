// Colwise dynamic FP8 quantization for the backward GEMMs: one fp32 scale per
// (group, column) over the group's rows, FP8 output written transposed
// (phys [C][rows]) so the wgrad/dgrad GEMMs read contraction-contiguous
// operands with no separate transpose copy.
// [P1 Details (colwise scales kernel: LDS-transposed output tile, single-pass
// variant without the second HBM read; relaxed atomics on AMD); P4 "Три уровня
// оптимизации Triton-ядер" (removal of the .t().contiguous().t() copy; fused
// scale-and-cast; relaxed atomic ordering for commutative reductions).]
//
// Work units: a 64-column strip x a chunk of up to 512 rows of one group (256
// or 128 rows when the groups are short on average).
// Chunks of group e are anchored at floor16(lo(e)) so every 16-row output
// segment is 16-byte aligned; the (rare) segments shared with a neighbouring
// group are stored byte by byte.
//   * Normally one single-pass kernel does everything (below): every chunk is
//     loaded once into registers and reduced; a group that spans several
//     chunks exchanges its column maxima between them through tagged slots in
//     device memory; then each chunk casts from registers, transposes through
//     LDS and stores (2 B read + 1 B written per element).
//   * Groups taller than 128 chunks, or calls with more chunks than there are
//     slots, take two passes: a partial-max kernel where every chunk merges its
//     column maxima into the scale buffer with a relaxed device-scope atomic
//     max on the fp32 bit pattern, tagged with the sign bit (order
//     independent, exact), then a cast kernel that turns the tag into the
//     scale (a reader sees either the tagged max or the final scale, and both
//     give the same scale).  The cast kernel visits units in reverse order so
//     its second read starts with the data the partial-max kernel touched last.
// The gathered form (GATHER) reads the grouped rows through moe_route's
// routing (row r = token row src[r] / topk, optionally times the slot's router
// weight), so the grouped bf16 tensor is never written (row_load8).
#include "device_common.hpp"
#include "kernels.hpp"
#include "tile_lds.hpp"

#include <atomic>

namespace fp8moe {

constexpr int kCwThreads = 256;
constexpr int kCwIters = kTileRows / 128;   // 4 iterations of 128 rows
constexpr uint32_t kTag = 0x80000000u;      // marks a merged |x| max (not yet a scale)

// Chunks of CR rows (512, or 256 or 128 for calls whose groups are short on average).
template <int CR = kTileRows>
__device__ __forceinline__ int cw_chunks(int lo, int hi) {
  if (hi <= lo) return 1;                    // an empty group still owns one unit: its scale
  const int a = lo & ~15;
  return (hi - a + CR - 1) / CR;
}
template <int CR = kTileRows>
struct CwChunks {
  __device__ int operator()(int lo, int hi) const { return cw_chunks<CR>(lo, hi); }
};
struct NoPad {
  __device__ int operator()(int, int) const { return 0; }
};

__global__ __launch_bounds__(256) void colwise_reset_kernel(uint32_t* __restrict__ s, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) s[i] = kTag;   // tagged zero max
}

struct CwGeom {
  int e, j, olo, ohi;      // group, chunk, output row range of the group
  int64_t in_base;         // input row of output row 0 of this group's output space
  uint8_t* q;              // output base of the group: q[c * ld_q + r]
  float* s;                // scale base of the group: s[c]
  bool ok;
};

template <bool GROUPED, int CR = kTileRows>
__device__ __forceinline__ CwGeom cw_geom(int u, int64_t batch, int rows, int cols,
                                          const int32_t* offs, int n_groups, uint8_t* q_t,
                                          int64_t ld_q, float* scale) {
  CwGeom g;
  if constexpr (GROUPED) {
    const Unit un = find_unit_quant<kCwThreads>(offs, n_groups, rows, u, CwChunks<CR>{}, NoPad{});
    g.ok = un.e >= 0;
    g.e = un.e; g.j = un.j; g.olo = un.lo; g.ohi = un.hi;
    g.in_base = 0;
    g.q = q_t;
    g.s = scale + (int64_t)max(un.e, 0) * cols;
  } else {
    const int upb = cw_chunks<CR>(0, rows);
    const int64_t b = u / upb;
    g.ok = b < batch;
    g.e = (int)b; g.j = u % upb; g.olo = 0; g.ohi = rows;
    g.in_base = b * rows;
    g.q = q_t + b * cols * ld_q;
    g.s = scale + b * cols;
  }
  return g;
}

// Reduce the per-thread packed maxima (4 u32 = 8 columns) over the 32 row
// slots; returns the bf16 |x| max bit pattern of column t (t < 64) in `out`.
__device__ __forceinline__ void cw_reduce_cols(uint32_t m[4], uint32_t* red /* [4][8][4] */, uint32_t* out) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, cc = t & 7;
#pragma unroll
  for (int p = 0; p < 4; ++p)
    m[p] = lane_max_xor<32, true>(lane_max_xor<16, true>(lane_max_xor<8, true>(m[p])));
  if (lane < 8) {
#pragma unroll
    for (int p = 0; p < 4; ++p) red[(w * 8 + cc) * 4 + p] = m[p];
  }
  __syncthreads();
  if (t < 64) {
    const int c8 = t >> 3, p = (t & 7) >> 1, half = t & 1;
    uint32_t r = 0;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) r = max(r, (red[(ww * 8 + c8) * 4 + p] >> (16 * half)) & 0xFFFFu);
    out[t] = r;
  }
  __syncthreads();
}

// PHASE 0: partial maxima of multi-chunk groups.  PHASE 1: cast (and the whole
// job for single-chunk and empty groups).
template <int CODEC, bool GROUPED, int PHASE, bool GATHER>
__global__ __launch_bounds__(256) void colwise_kernel(RowSrc xs, int64_t batch,
                                                      int rows, int cols, const int32_t* __restrict__ offs,
                                                      int n_groups, uint8_t* __restrict__ q_t, int64_t ld_q,
                                                      float* __restrict__ scale, int n_strips, int units) {
  __shared__ uint32_t red[4 * 8 * 4];
  __shared__ uint32_t s_amax[64];
  __shared__ float s_scale[64];
  __shared__ __attribute__((aligned(16))) uint8_t tile[PHASE == 1 ? kTileBytes : 16];

  const int strip = blockIdx.x % n_strips;
  int u = blockIdx.x / n_strips;
  if (PHASE == 1) u = units - 1 - u;
  const CwGeom g = cw_geom<GROUPED>(u, batch, rows, cols, offs, n_groups, q_t, ld_q, scale);
  if (!g.ok) return;

  const int t = threadIdx.x, cc = t & 7, rs = t >> 3;
  const int c0 = strip * kTileCols;
  const bool empty = g.ohi <= g.olo;
  const int nch = cw_chunks(g.olo, g.ohi);
  if (PHASE == 0 && (empty || nch == 1)) return;
  if (empty) {   // PHASE 1: the scale of an empty group (no rows, no data)
    if (t < 64 && c0 + t < cols) g.s[c0 + t] = scale_from_amax(0.0f, CODEC);
    return;
  }

  const int A = (g.olo & ~15) + g.j * kTileRows;          // output row of tile row 0
  const int r_begin = max(A, g.olo), r_end = min(A + kTileRows, g.ohi);
  const int col = c0 + cc * 8;
  const bool col_ok = col < cols;

  u32x4 v[kCwIters][4];
  uint32_t m[4] = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < kCwIters; ++i) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = A + 128 * i + 4 * rs + k;
      const bool ok = col_ok && r >= r_begin && r < r_end;
      v[i][k] = ok ? row_load8<GATHER>(xs, g.in_base + r, cols, col) : u32x4{0, 0, 0, 0};
      m[0] = pk_absmax_bf16(m[0], v[i][k].x);
      m[1] = pk_absmax_bf16(m[1], v[i][k].y);
      m[2] = pk_absmax_bf16(m[2], v[i][k].z);
      m[3] = pk_absmax_bf16(m[3], v[i][k].w);
    }
  }

  if (PHASE == 0) {
    cw_reduce_cols(m, red, s_amax);
    if (t < 64 && c0 + t < cols)
      __hip_atomic_fetch_max(reinterpret_cast<uint32_t*>(g.s) + c0 + t, kTag | (s_amax[t] << 16),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  } else {
    if (nch == 1) {
      cw_reduce_cols(m, red, s_amax);
      if (t < 64) s_scale[t] = scale_from_amax(__uint_as_float(s_amax[t] << 16), CODEC);
    } else if (t < 64) {
      float sc = 0.0f;
      if (c0 + t < cols) {
        const uint32_t b = __hip_atomic_load(reinterpret_cast<uint32_t*>(g.s) + c0 + t, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        sc = (b & kTag) ? scale_from_amax(__uint_as_float(b & ~kTag), CODEC) : __uint_as_float(b);
      }
      s_scale[t] = sc;
    }
    __syncthreads();
    if (g.j == 0 && t < 64 && c0 + t < cols) g.s[c0 + t] = s_scale[t];

    // cast: per column, the 4 rows of a slot become one little-endian word
    float sc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) sc[k] = s_scale[cc * 8 + k];
#pragma unroll
    for (int i = 0; i < kCwIters; ++i) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t w = quant4<CODEC>(col_of(v[i][0], k), col_of(v[i][1], k), col_of(v[i][2], k),
                                         col_of(v[i][3], k), sc[k]);
        tile_put4(tile, cc * 8 + k, 128 * i + 4 * rs, w);
      }
    }
    __syncthreads();

    // transposed store: each pass writes 8 columns x 32 segments of 16 rows
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int ci = p * 8 + (t >> 5), sg = t & 31;
      const int c = c0 + ci, R0 = A + 16 * sg;
      if (c < cols && R0 < r_end && R0 + 16 > r_begin) {
        const u32x4 d = tile_get16(tile, ci, 16 * sg);
        store_segment(g.q + (int64_t)c * ld_q + R0, R0, r_begin, r_end, d);
      }
    }
  }
}


// ---------------------------------------------------------------- single pass
// One workgroup per chunk, numbered so that the chunks of one (group, strip)
// job are consecutive workgroups, which the hardware dispatches together.  A
// chunk keeps its 512 x 64 values in registers, reduces its column maxima and,
// when its group spans several chunks, publishes them to its own slot of a
// library-owned array (one 64-bit word per column: the call's generation in
// the high half, the bf16 |x| max in the low bits).  It then reads the slots of
// every chunk of its job until all carry this call's generation, takes the
// maximum, and casts from registers: HBM sees 2 bytes read + 1 byte written
// per element.  There are no read-modify-write atomics and no counters: every
// slot is written once per call and validated by its tag, so calls need no
// reset and rely on no state left by earlier calls.
//   The wait is bounded.  A chunk whose peers do not all publish in time (not
// resident together, or another call on the same slots) re-reads its group's
// rows to compute the same maxima itself, so every wave finishes and the
// result never depends on timing.
constexpr int kSlotItems = 32768;           // chunk slots (16 MiB); more chunks take the two-pass path
constexpr int kMaxChunks = 128;             // taller groups take the two-pass path
constexpr int kPolls = 4096;                // default: sleeps of ~512 cycles (plus a load) before the fallback
__device__ unsigned long long g_cw_part[kSlotItems][kTileCols];

// Maxima of 64 columns over rows [lo, hi) of group rows in_base + r, read
// again from global memory (the fallback of a wait that ran out).
template <bool GATHER>
__device__ __forceinline__ void cw_column_max(const RowSrc& xs, int64_t in_base, int lo, int hi,
                                              int cols, int c0, uint32_t* red, uint32_t* out) {
  const int t = threadIdx.x, cc = t & 7, rs = t >> 3;
  const int col = c0 + cc * 8;
  uint32_t m[4] = {0, 0, 0, 0};
  if (col < cols) {
    for (int r = lo + rs; r < hi; r += 32) {
      const u32x4 v = row_load8<GATHER>(xs, in_base + r, cols, col);
      m[0] = pk_absmax_bf16(m[0], v.x);
      m[1] = pk_absmax_bf16(m[1], v.y);
      m[2] = pk_absmax_bf16(m[2], v.z);
      m[3] = pk_absmax_bf16(m[3], v.w);
    }
  }
  cw_reduce_cols(m, red, out);
}

// Wave 0 (64 lanes, one per column): the maximum over the published slots of
// the nch chunks starting at item0, 8 slots per round trip.  Returns whether
// all arrived within the poll budget (then out[t] holds the maximum).
__device__ __forceinline__ bool cw_gather(const unsigned long long* __restrict__ part, int item0, int nch,
                                          uint32_t gen, int max_polls, uint32_t* out) {
  const int t = threadIdx.x;
  uint32_t mx = 0;
  int k = 0;
  for (int polls = 0; k < nch && polls < max_polls;) {
    unsigned long long b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      b[i] = k + i < nch ? __hip_atomic_load(part + (int64_t)(item0 + k + i) * kTileCols + t, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT)
                         : (unsigned long long)gen << 32;
    int have = 1;
#pragma unroll
    for (int i = 0; i < 8; ++i) have &= (uint32_t)(b[i] >> 32) == gen;
    if (__all(have)) {
#pragma unroll
      for (int i = 0; i < 8; ++i) mx = max(mx, (uint32_t)b[i] & 0xFFFFu);
      k += 8;
    } else {
      ++polls;
      __builtin_amdgcn_s_sleep(8);
    }
  }
  out[t] = mx;
  return k >= nch;
}

template <int CODEC, bool GROUPED, int CR, bool GATHER>
__global__ __launch_bounds__(256) void colwise_single_kernel(RowSrc xs, int64_t batch,
                                                             int rows, int cols, const int32_t* __restrict__ offs,
                                                             int n_groups, uint8_t* __restrict__ q_t, int64_t ld_q,
                                                             float* __restrict__ scale, int units, uint32_t gen,
                                                             int max_polls) {
  constexpr int kIters = CR / 128;
  __shared__ uint32_t red[4 * 8 * 4];
  __shared__ uint32_t s_amax[64];
  __shared__ float s_scale[64];
  __shared__ int s_ok;
  __shared__ __attribute__((aligned(16))) uint8_t tile[kTileCols * CR];
  const int t = threadIdx.x, cc = t & 7, rs = t >> 3;
  // The chunks of one (group or batch item, strip) job are consecutive
  // workgroups (the exchange relies on it).  Batched tensors (weights) run
  // their jobs in bands of 8 strips per batch item, so the workgroups running
  // together read 1 KiB of each row instead of 128 bytes.
  int strip, u;
  if constexpr (GROUPED) {
    strip = blockIdx.x / units;
    u = blockIdx.x % units;
  } else {
    const int n_strips = (int)(gridDim.x / units), upb = (int)(units / batch);
    const int per_b = n_strips * upb;
    const int b = (int)blockIdx.x / per_b, r = (int)blockIdx.x % per_b;
    const int band = r / (8 * upb), r2 = r % (8 * upb);
    strip = 8 * band + r2 / upb;
    u = b * upb + r2 % upb;
  }
  const CwGeom g = cw_geom<GROUPED, CR>(u, batch, rows, cols, offs, n_groups, q_t, ld_q, scale);
  if (!g.ok) return;
  const int c0 = strip * kTileCols;
  if (g.ohi <= g.olo) {   // the scale of an empty group (no rows, no data)
    if (t < 64 && c0 + t < cols) g.s[c0 + t] = scale_from_amax(0.0f, CODEC);
    return;
  }
  const int nch = cw_chunks<CR>(g.olo, g.ohi);
  const int A = (g.olo & ~15) + g.j * CR;                  // output row of tile row 0
  const int r_begin = max(A, g.olo), r_end = min(A + CR, g.ohi);
  const int col = c0 + cc * 8;
  const bool col_ok = col < cols;

  // Gathered rows: the chunk's token rows and weights are looked up once, with
  // coalesced loads, into LDS (the front of the codes tile, which is written
  // only after the column reduction's barriers), so each row's data load waits
  // for an LDS read rather than a dependent global one.
  int* const s_tok = reinterpret_cast<int*>(tile);
  float* const s_w = reinterpret_cast<float*>(tile) + CR;
  static_assert(!GATHER || 8 * CR <= kTileCols * CR, "token table fits the tile");
  if constexpr (GATHER) {
    for (int i = t; i < CR; i += 256) {
      const int r = A + i;
      int tk = -1;
      float wv = 1.0f;
      if (r >= r_begin && r < r_end) {
        const int sl = xs.src[r];
        if (sl >= 0 && (int64_t)sl < xs.slots) {
          tk = sl / xs.topk;
          if (xs.w != nullptr) wv = xs.w[sl];
        }
      }
      s_tok[i] = tk;
      s_w[i] = wv;
    }
    __syncthreads();
  }
  u32x4 v[kIters][4];
  uint32_t m[4] = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < kIters; ++i) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = A + 128 * i + 4 * rs + k;
      const bool ok = col_ok && r >= r_begin && r < r_end;
      if constexpr (GATHER) {
        const int tk = s_tok[128 * i + 4 * rs + k];
        v[i][k] = ok && tk >= 0 ? *reinterpret_cast<const u32x4*>(xs.x + (int64_t)tk * cols + col)
                                : u32x4{0, 0, 0, 0};
        if (xs.w != nullptr) v[i][k] = bf16x8_times(v[i][k], s_w[128 * i + 4 * rs + k]);
      } else {
        v[i][k] = ok ? row_load8<false>(xs, g.in_base + r, cols, col) : u32x4{0, 0, 0, 0};
      }
      m[0] = pk_absmax_bf16(m[0], v[i][k].x);
      m[1] = pk_absmax_bf16(m[1], v[i][k].y);
      m[2] = pk_absmax_bf16(m[2], v[i][k].z);
      m[3] = pk_absmax_bf16(m[3], v[i][k].w);
    }
  }
  cw_reduce_cols(m, red, s_amax);
  if (nch > 1) {
    unsigned long long* part = &g_cw_part[0][0];
    if (t < 64) {
      __hip_atomic_store(part + (int64_t)blockIdx.x * kTileCols + t, ((unsigned long long)gen << 32) | s_amax[t],
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const bool ok = cw_gather(part, (int)blockIdx.x - g.j, nch, gen, max_polls, s_amax);
      if (t == 0) s_ok = ok;
    }
    __syncthreads();
    if (!s_ok) cw_column_max<GATHER>(xs, g.in_base, g.olo, g.ohi, cols, c0, red, s_amax);
  }
  if (t < 64) s_scale[t] = scale_from_amax(__uint_as_float(s_amax[t] << 16), CODEC);
  __syncthreads();
  if (g.j == 0 && t < 64 && c0 + t < cols) g.s[c0 + t] = s_scale[t];

  // cast: per column, the 4 rows of a slot become one little-endian word
  float sc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) sc[k] = s_scale[cc * 8 + k];
#pragma unroll
  for (int i = 0; i < kIters; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t w = quant4<CODEC>(col_of(v[i][0], k), col_of(v[i][1], k), col_of(v[i][2], k),
                                       col_of(v[i][3], k), sc[k]);
      *reinterpret_cast<uint32_t*>(tile + tile_off_r<CR>(cc * 8 + k, 128 * i + 4 * rs)) = w;
    }
  }
  __syncthreads();
  // transposed store: each pass writes 256 / (CR / 16) columns x CR / 16 segments of 16 rows
  constexpr int kSegs = CR / 16, kColsPerPass = 256 / kSegs;
#pragma unroll
  for (int pp = 0; pp < kTileCols / kColsPerPass; ++pp) {
    const int ci = pp * kColsPerPass + t / kSegs, sg = t % kSegs;
    const int c = c0 + ci, R0 = A + 16 * sg;
    if (c < cols && R0 < r_end && R0 + 16 > r_begin) {
      const u32x4 d = *reinterpret_cast<const u32x4*>(tile + tile_off_r<CR>(ci, 16 * sg));
      store_segment(g.q + (int64_t)c * ld_q + R0, R0, r_begin, r_end, d);
    }
  }
}

// One generation per call of the single-pass kernel (0 never names a call).
// A generation is a kernel argument, so a launch captured into a graph would
// replay with the same one and could accept a previous replay's slots: calls
// made while their stream is capturing take the two-pass path instead, whose
// reset is an ordinary kernel and which keeps no state between launches.
static std::atomic<uint32_t> g_generation{0};
static std::atomic<int> g_poll_budget{kPolls};
static std::atomic<int> g_chunk_rows{0};   // 0: chosen per call; 128, 256 or 512: forced (a test hook)
static uint32_t next_generation() {
  uint32_t g = g_generation.fetch_add(1) + 1;
  if (g == 0) g = g_generation.fetch_add(1) + 1;
  return g;
}

int64_t colwise_units_bound(int64_t batch, int64_t rows, const int32_t* offs, int32_t n_groups,
                            int64_t cr = kTileRows) {
  if (offs) return (rows + 16LL * n_groups + cr - 1) / cr + n_groups;
  const int64_t upb = rows > 0 ? (rows + cr - 1) / cr : 1;
  return batch * upb;
}

// Chunk height of a single-pass call from the average rows per group (or batch
// item): at most 128 -> 128-row chunks, at most 512 -> 256, else 512.  A
// 512-row chunk of a short group is mostly padding; for groups of a few hundred
// rows 256-row chunks beat 128 (half as many chunks exchange maxima, with the
// same eight workgroups per CU).  A forced height from the test hook wins.
static int colwise_chunk_rows(int64_t rows, int64_t groups) {
  const int forced = g_chunk_rows.load();
  if (forced == 128 || forced == 256 || forced == kTileRows) return forced;
  const int64_t g = std::max<int64_t>(groups, 1);
  return rows <= 128 * g ? 128 : rows <= 512 * g ? 256 : kTileRows;
}

template <int CODEC, bool GROUPED, bool GATHER = false>
static hipError_t launch_cw(const RowSrc& xs, int64_t batch, int64_t rows, int64_t cols,
                            const int32_t* offs, int32_t n_groups, uint8_t* q_t, int64_t ld_q, float* scale,
                            hipStream_t st) {
  const int64_t n_scale = (GROUPED ? n_groups : batch) * cols;
  if (n_scale == 0) return hipSuccess;
  const int n_strips = (int)((cols + kTileCols - 1) / kTileCols);
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cap) != hipSuccess) return hipGetLastError();
  const bool capturing = cap != hipStreamCaptureStatusNone;
  // the single pass, at the chosen chunk height or else at 512 rows
  const int pref = colwise_chunk_rows(rows, GROUPED ? n_groups : 1);
  for (int cr : {pref, kTileRows}) {
    const int64_t units = colwise_units_bound(batch, rows, offs, n_groups, cr);
    const int64_t items = units * n_strips;
    // most chunks one group can span: a grouped group may start 15 rows past a 16-row anchor
    const int64_t nch_bound = ((GROUPED ? rows + 15 : rows) + cr - 1) / cr;
    if (!capturing && nch_bound <= kMaxChunks && (nch_bound <= 1 || items <= kSlotItems) && items < (1LL << 31)) {
      auto k = cr == 128   ? colwise_single_kernel<CODEC, GROUPED, 128, GATHER>
               : cr == 256 ? colwise_single_kernel<CODEC, GROUPED, 256, GATHER>
                           : colwise_single_kernel<CODEC, GROUPED, kTileRows, GATHER>;
      hipLaunchKernelGGL(k, dim3((unsigned)items), dim3(256), 0, st, xs, batch, (int)rows, (int)cols, offs, n_groups,
                         q_t, ld_q, scale, (int)units, next_generation(), g_poll_budget.load());
      return hipGetLastError();
    }
    if (cr == kTileRows) break;
  }
  const int64_t units = colwise_units_bound(batch, rows, offs, n_groups);
  hipLaunchKernelGGL(colwise_reset_kernel, dim3((unsigned)((n_scale + 255) / 256)), dim3(256), 0, st,
                     reinterpret_cast<uint32_t*>(scale), n_scale);
  const dim3 grid((unsigned)(units * n_strips));
  hipLaunchKernelGGL((colwise_kernel<CODEC, GROUPED, 0, GATHER>), grid, dim3(256), 0, st, xs, batch, (int)rows,
                     (int)cols, offs, n_groups, q_t, ld_q, scale, n_strips, (int)units);
  hipLaunchKernelGGL((colwise_kernel<CODEC, GROUPED, 1, GATHER>), grid, dim3(256), 0, st, xs, batch, (int)rows,
                     (int)cols, offs, n_groups, q_t, ld_q, scale, n_strips, (int)units);
  return hipGetLastError();
}

int set_colwise_poll_budget(int polls) { return g_poll_budget.exchange(polls < 0 ? kPolls : polls); }

int set_colwise_chunk_rows(int rows) {
  return g_chunk_rows.exchange(rows == 128 || rows == 256 || rows == kTileRows ? rows : 0);
}

hipError_t launch_quantize_colwise(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols,
                                   const int32_t* offs, int32_t n_groups, int codec, uint8_t* q_t,
                                   int64_t ld_q, float* scale, hipStream_t st) {
  if (cols == 0) return hipSuccess;
  const RowSrc xs{x, nullptr, nullptr, 1, 0};
  if (offs) {
    return codec == 0 ? launch_cw<0, true>(xs, 1, rows, cols, offs, n_groups, q_t, ld_q, scale, st)
                      : launch_cw<1, true>(xs, 1, rows, cols, offs, n_groups, q_t, ld_q, scale, st);
  }
  return codec == 0 ? launch_cw<0, false>(xs, batch, rows, cols, nullptr, 0, q_t, ld_q, scale, st)
                    : launch_cw<1, false>(xs, batch, rows, cols, nullptr, 0, q_t, ld_q, scale, st);
}

hipError_t launch_moe_permute_colwise(const uint16_t* x, int64_t tokens, int64_t cols, int topk, const int32_t* src,
                                      const float* weights, int64_t rows, const int32_t* offs, int32_t n_groups,
                                      int codec, uint8_t* q_t, int64_t ld_q, float* scale, hipStream_t st) {
  if (cols == 0) return hipSuccess;
  const RowSrc xs{x, src, weights, topk, tokens * topk};
  return codec == 0 ? launch_cw<0, true, true>(xs, 1, rows, cols, offs, n_groups, q_t, ld_q, scale, st)
                    : launch_cw<1, true, true>(xs, 1, rows, cols, offs, n_groups, q_t, ld_q, scale, st);
}

}  // namespace fp8moe

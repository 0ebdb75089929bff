// A 64-column x 512-row tile of FP8 codes in LDS, written in 4-row words by
// the cast and read back as 16-row segments of one column, so the transposed
// output leaves the chip in contiguous 16-byte stores.  [P1 Details and P4
// "Три уровня оптимизации Triton-ядер": the colwise kernel's lanes used to
// store K bytes apart; the fix transposes the output tile in LDS first.]
//
// Thread layout of the 256-thread workgroup that fills the tile: cc = t & 7
// picks an 8-column slice, rs = t >> 3 (0..31) a slot of 4 consecutive rows;
// iteration i covers tile rows 128*i + 4*rs + {0..3}.
//
// Bank-conflict-free swizzle (64 banks of 4 bytes): column c, row r lives at
//   c*512 + (((r >> 4) ^ (2*(c >> 3))) << 4) + (r & 15).
// * writes: one b32 per (column, 4-row slot).  Across a wave, (segment ^ 2*cc)
//   takes 16 distinct values mod 16 and the 4 row-slots of a segment fill its
//   4 banks, so the 64 lanes hit 64 distinct banks.
// * reads: one b128 per (column, segment); 16 consecutive lanes read 16
//   consecutive segments of one column, permuted within an aligned block of 16.
#pragma once

#include "device_common.hpp"

namespace fp8moe {

constexpr int kTileCols = 64;
constexpr int kTileRows = 512;
constexpr int kTileBytes = kTileCols * kTileRows;   // 32 KiB

__device__ __forceinline__ int tile_off(int c, int r) {
  return c * kTileRows + ((((r >> 4) ^ (2 * (c >> 3))) & 31) << 4) + (r & 15);
}

// The same layout for a tile of TR rows (TR / 16 segments per column).  For
// TR = 128 the segment is XOR-ed with the 8-column slice index (8 values over
// 8 segments), which keeps a wave's 4-row writes of one slice column on 32
// distinct banks and a quarter-wave's 16-byte reads (two columns) on all 64.
// TR = 256 takes the same XOR within its 16 segments: the writes again reach
// 32 banks, and a quarter-wave's reads (16 segments of one column) all 64.
template <int TR>
__device__ __forceinline__ int tile_off_r(int c, int r) {
  if constexpr (TR == kTileRows) {
    return tile_off(c, r);
  } else {
    static_assert(TR == 128 || TR == 256, "tile heights: 512, 256 or 128 rows");
    return c * TR + ((((r >> 4) ^ (c >> 3)) & (TR / 16 - 1)) << 4) + (r & 15);
  }
}

// Codes of 4 consecutive rows (r..r+3, r % 4 == 0) of one column.
__device__ __forceinline__ void tile_put4(uint8_t* tile, int c, int r, uint32_t word) {
  *reinterpret_cast<uint32_t*>(tile + tile_off(c, r)) = word;
}

// 16 consecutive rows (r % 16 == 0) of one column.
__device__ __forceinline__ u32x4 tile_get16(const uint8_t* tile, int c, int r) {
  return *reinterpret_cast<const u32x4*>(tile + tile_off(c, r));
}

// Byte k (0..7) of the 8 bf16 columns held in a u32x4, as fp32.
__device__ __forceinline__ float col_of(const u32x4& v, int k) {
  const uint32_t w = k < 2 ? v.x : k < 4 ? v.y : k < 6 ? v.z : v.w;
  return (k & 1) ? bf16_hi(w) : bf16_lo(w);
}

// Store the 16 bytes of tile rows [R0, R0+16) to dst, keeping only rows inside
// [r_begin, r_end) (global row numbers).  Full segments take one 16-byte store.
__device__ __forceinline__ void store_segment(uint8_t* dst, int R0, int r_begin, int r_end, const u32x4& d) {
  if (R0 >= r_begin && R0 + 16 <= r_end) {
    *reinterpret_cast<u32x4*>(dst) = d;
    return;
  }
  const uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
  for (int b = 0; b < 16; ++b) {
    const int r = R0 + b;
    if (r >= r_begin && r < r_end) dst[b] = (uint8_t)(w[b >> 2] >> (8 * (b & 3)));
  }
}

}  // namespace fp8moe

// Address arithmetic of the GEMM operand loads, shared by the kernels and by a host-side test
// that sweeps shapes, tiles, K steps, waves and lanes and checks every source byte against the
// bounds of its buffer.  Plain C++: compiles for the host and for gfx950.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define BSFP8_HD __host__ __device__ __forceinline__
#else
#define BSFP8_HD inline
#endif

namespace bsfp8 {

// XOR swizzle of the 16-byte chunks of a 128-byte LDS row: 16 consecutive rows (the rows that
// one fragment read spreads over the banks) see all eight chunk positions twice.
BSFP8_HD int swz(int row) { return (row ^ (row >> 3)) & 7; }

// One 16-byte DMA lane of an operand tile: LDS region g holds tile rows 8g .. 8g + 7; lane
// `lane` of the instruction fills slot lane (row 8g + lane / 8, swizzled chunk lane % 8).
// Returns the byte offset of its source, relative to the tile's first row, for K step k0:
//   row: clamped to `last` (the last valid row of the tile, >= 0);
//   K  : the chunk's K offset, or 0 (the row start) when the chunk lies at or past kext.
// Both parts are non-negative; the row part is below 2^32 when 256 * ld < 2^32.
BSFP8_HD uint64_t tile_dma_offset(int g, int lane, int last, int64_t ld, int64_t k0, int64_t kext) {
  const int lrow = lane >> 3, lslot = lane & 7;
  int row = g * 8 + lrow;
  row = row < last ? row : last;
  const int64_t kof = k0 + 16 * (lslot ^ ((lrow ^ g) & 7));
  const uint32_t row_part = (uint32_t)row * (uint32_t)ld;
  return (uint64_t)row_part + (uint64_t)(kof < kext ? kof : 0);
}

// Whether that lane's chunk is a K tail chunk (zeroed in LDS after the DMA lands).
BSFP8_HD bool tile_dma_is_tail(int g, int lane, int64_t k0, int64_t kext) {
  const int lrow = lane >> 3, lslot = lane & 7;
  return k0 + 16 * (lslot ^ ((lrow ^ g) & 7)) >= kext;
}

// First row of the four E8M0 scale rows one 4-byte DMA lane moves: rows part*256 + 4*lane ..
// + 3, pulled back so that all four are valid (`last` + 1 is a multiple of 4 and >= 4).
BSFP8_HD int scale_dma_row(int part, int lane, int last) {
  const int r4 = part * 256 + 4 * lane;
  return r4 + 3 <= last ? r4 : last - 3;
}

}  // namespace bsfp8

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

// Byte offset, within a 128-byte K step of a row, of the 16-byte chunk that DMA lane `lane` of
// LDS region g moves: LDS region g holds tile rows 8g .. 8g + 7, and lane `lane` fills slot
// lane (row 8g + lane / 8, swizzled chunk lane % 8), which holds K chunk (lane % 8) ^ swz(row).
BSFP8_HD int dma_chunk(int g, int lane) { return 16 * ((lane & 7) ^ (((lane >> 3) ^ g) & 7)); }

// Source offset of that lane for K step k0, relative to the tile's first row (row-major rows of
// ld bytes).  Rows past the valid ones and chunks past the K extent are not redirected: the
// kernels read through a buffer resource whose range ends with the tile's last valid row, so
// the hardware returns zeros past it; a chunk past the K extent of a valid row (fprop tail)
// holds bytes of the next row and is masked when the fragments are read.  Below 2^32 when
// 256 * ld + 128 <= 2^32.
BSFP8_HD uint32_t tile_dma_voffset(int g, int lane, uint32_t ld, uint32_t k0) {
  return (uint32_t)(g * 8 + (lane >> 3)) * ld + (uint32_t)dma_chunk(g, lane) + k0;
}

// Byte range of the buffer resource over an operand tile: `rows` valid rows of ld bytes from
// the tile's first row, clamped to the 32-bit range field (the tile's own offsets stay below
// 256 * ld + 128 <= 2^32 - 2^15, so a clamped range cuts off none of them).
BSFP8_HD uint32_t tile_range(int64_t rows, int64_t ld) {
  const int64_t b = rows * ld;
  return b > (int64_t)0xFFFFFFFF ? 0xFFFFFFFFu : (uint32_t)b;
}

// First row of the four E8M0 scale rows one 4-byte DMA lane moves: rows part*256 + 4*lane ..
// + 3, pulled back so that all four are valid (`last` + 1 is a multiple of 4 and >= 4).
BSFP8_HD int scale_dma_row(int part, int lane, int last) {
  const int r4 = part * 256 + 4 * lane;
  return r4 + 3 <= last ? r4 : last - 3;
}

// First of the 16 E8M0 scale rows one 16-byte DMA lane moves (the scaled-MFMA paths: 16 lanes per
// 256-row block): rows 16 * (lane % 16) .. + 15, pulled back so that all 16 are valid (`last` + 1,
// the tile's valid rows counted from its first, is a multiple of 32 and >= 32).
BSFP8_HD int scale_dma16_row(int lane, int last) {
  const int r = 16 * (lane & 15);
  return r + 15 <= last ? r : last + 1 - 16;
}

}  // namespace bsfp8

// Host sweep of the GEMM operand-load geometry (csrc/tile_addr.hpp), run by tests/test_tile_addr.py.
// For every shape, tile, K step, wave, DMA instruction and lane it checks that
//  * the 32-bit source offset does not wrap and is the one of LDS slot (row, c ^ swz(row)):
//    row `row` of the tile, K chunk c -- the slot the fragment reads take chunk c from;
//  * every chunk the fragments use (a valid row, K below the extent) lies inside the buffer
//    range (the other chunks are either inside it or wholly past its end, where the hardware
//    returns zeros) and is delivered exactly once;
//  * the 4-row E8M0 scale groups stay inside the valid rows.
// Exit status 0 when no violation is found.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "tile_addr.hpp"

using namespace bsfp8;

static long g_fail = 0, g_checked = 0;

// One operand (valid rows of ld bytes, K extent kext) tiled BM rows at a time, loaded by NW waves.
static void check_operand(const char* what, int BM, int NW, int64_t valid, int64_t ld, int64_t kext) {
  const int ins = BM / 8 / NW;
  const int64_t nk = (kext + 127) / 128;
  for (int64_t row0 = 0; row0 < valid; row0 += BM) {
    const int last = (int)(valid - 1 - row0);
    const uint64_t range = tile_range(valid - row0, ld);
    if (range != (uint64_t)((valid - row0) * ld) && (uint64_t)((valid - row0) * ld) <= 0xFFFFFFFFull) {
      if (g_fail++ < 10) std::printf("%s: range %llu != rows * ld\n", what, (unsigned long long)range);
    }
    for (int64_t kk = 0; kk < nk; ++kk) {
      const int64_t k0 = kk * 128;
      std::vector<int> seen((size_t)BM * 8, 0);
      for (int wave = 0; wave < NW; ++wave)
        for (int u = 0; u < ins; ++u) {
          const int g = wave * ins + u;
          for (int lane = 0; lane < 64; ++lane) {
            ++g_checked;
            const uint64_t off = (uint64_t)tile_dma_voffset(g, lane, (uint32_t)ld, 0) + (uint64_t)k0;
            // the kernels add k0 in 32 bits: no wrap
            if (off >= (uint64_t(1) << 32) || (uint64_t)tile_dma_voffset(g, lane, (uint32_t)ld, (uint32_t)k0) != off) {
              if (g_fail++ < 10) std::printf("%s: 32-bit offset wraps ld=%lld k0=%lld\n", what, (long long)ld, (long long)k0);
              continue;
            }
            if (off % 16 != 0) {
              if (g_fail++ < 10) std::printf("%s: misaligned offset\n", what);
            }
            const int lds = g * 1024 + 16 * lane, trow = lds / 128, slot = (lds % 128) / 16;
            const int chunk = slot ^ swz(trow);
            // the source: row row0 + trow, K bytes k0 + 16 * chunk .. + 15 of it
            if (off != (uint64_t)trow * (uint64_t)ld + (uint64_t)(k0 + 16 * chunk) || dma_chunk(g, lane) != 16 * chunk) {
              if (g_fail++ < 10)
                std::printf("%s: slot (%d,%d) reads offset %llu, want row %d chunk %d\n", what, trow, slot,
                            (unsigned long long)off, trow, chunk);
              continue;
            }
            const bool in_range = off + 16 <= range;
            const bool wanted = trow <= last && k0 + 16 * chunk < kext;  // a byte the fragments use
            // wanted bytes come from inside the range; a byte past the range is read as zero by
            // the hardware, and a partial overlap cannot happen (range and offsets are 16-aligned)
            if (wanted && !in_range) {
              if (g_fail++ < 10) std::printf("%s: wanted chunk outside the range\n", what);
            }
            if (off < range && off + 16 > range) {
              if (g_fail++ < 10) std::printf("%s: chunk straddles the range end\n", what);
            }
            if (wanted) seen[(size_t)trow * 8 + chunk]++;
          }
        }
      for (int r = 0; r < BM && r <= last; ++r)
        for (int c = 0; c < 8; ++c)
          if (k0 + 16 * c < kext && seen[(size_t)r * 8 + c] != 1) {
            if (g_fail++ < 10) std::printf("%s: row %d chunk %d delivered %d times\n", what, r, c, seen[(size_t)r * 8 + c]);
          }
    }
    // E8M0 scale rows of the widened path: 4 per lane, the 256 bytes [256 v, +256) of the
    // [block][BM rows] area per instruction v (a 128-row tile: two blocks per instruction); a
    // valid row comes from its own place, a row past `last` from valid rows
    if (valid % 32 == 0) {
      for (int v = 0; v < 4 * BM / 256; ++v) {
        for (int lane = 0; lane < 64; ++lane) {
          const int flat = v * 256 + 4 * lane, row = flat % BM;
          const int r4 = scale_dma_row(0, row >> 2, last);
          ++g_checked;
          if (r4 < 0 || r4 % 4 != 0 || r4 + 3 > last || (row <= last && r4 != row)) {
            if (g_fail++ < 10) std::printf("%s: scale rows %d..%d for row %d (last %d)\n", what, r4, r4 + 3, row, last);
          }
        }
      }
      // 16 rows per lane (the scaled-MFMA paths): in range, 16-aligned, and every valid row of the
      // tile's 256 delivered by some lane
      if (BM == 256) {
        std::vector<int> got(256, 0);
        for (int lane = 0; lane < 16; ++lane) {
          const int r = scale_dma16_row(lane, last);
          ++g_checked;
          if (r < 0 || r % 16 != 0 || r + 15 > last) {
            if (g_fail++ < 10) std::printf("%s: 16-byte scale rows %d..%d past last %d\n", what, r, r + 15, last);
            continue;
          }
          for (int i = 0; i < 16 && r + i < 256; ++i) got[r + i] = 1;
        }
        for (int i = 0; i < 256 && i <= last; ++i)
          if (!got[i]) {
            if (g_fail++ < 10) std::printf("%s: scale row %d not loaded (last %d)\n", what, i, last);
          }
      }
    }
  }
}

int main() {
  // wgrad MX: 256 x 256 tiles, 8 waves; operands rows = n or h (multiples of 32), K = Kp_e
  const int64_t cols[] = {32, 64, 96, 256, 320, 2048, 7168};
  const int64_t kps[] = {128, 256, 384, 8704, 19200};
  for (int64_t c : cols)
    for (int64_t kp : kps) check_operand("wgrad-mx", 256, 8, c, kp, kp);
  // wgrad MX on a launch of few tiles: 128 x 128 tiles, 4 waves
  for (int64_t c : cols)
    for (int64_t kp : kps) check_operand("wgrad-mx128", 128, 4, c, kp, kp);
  // wgrad per-channel: 128 x 128 tiles, 4 waves
  for (int64_t c : cols)
    for (int64_t kp : kps) check_operand("wgrad-pc", 128, 4, c, kp, kp);
  // fprop (256 x 256 tiles, 8 waves): A rows = a group's live rows (any count), B rows = n; K any multiple of 32 (tails)
  const int64_t rows[] = {1, 2, 31, 32, 33, 127, 255, 256, 257, 600, 8409};
  const int64_t ks[] = {32, 96, 128, 160, 256, 288, 4096, 7168, 7200};
  for (int64_t r : rows)
    for (int64_t k : ks) check_operand("fprop-a", 256, 8, r, k, k);
  for (int64_t n : cols)
    for (int64_t k : ks) check_operand("fprop-b", 256, 8, n, k, k);
  std::printf("checked %ld lane loads, %ld violations\n", g_checked, g_fail);
  return g_fail == 0 ? 0 : 1;
}

// Host sweep of the GEMM operand-load geometry (csrc/tile_addr.hpp), run by tests/test_tile_addr.py.
// For every shape, tile, K step, wave, DMA instruction and lane it checks that
//  * the 16 source bytes lie inside the operand (a valid row, K bytes below the K extent);
//  * for a valid row and a non-tail chunk, LDS slot (row, c ^ swz(row)) receives K chunk c of
//    that row -- the slot the fragment reads take chunk c from -- and every (row, chunk) of the
//    tile is delivered exactly once;
//  * the 4-row E8M0 scale groups stay inside the valid rows.
// Exit status 0 when no violation is found.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "tile_addr.hpp"

using namespace bsfp8;

static long g_fail = 0, g_checked = 0;

static void check_operand(const char* what, int BM, int NW, int64_t valid, int64_t ld, int64_t kext, bool tail) {
  const int ins = BM / 8 / NW;
  const int64_t nk = (kext + 127) / 128;
  for (int64_t row0 = 0; row0 < valid; row0 += BM) {
    const int last = (int)(valid - 1 - row0);
    for (int64_t kk = 0; kk < nk; ++kk) {
      const int64_t k0 = kk * 128;
      std::vector<int> seen((size_t)BM * 8, 0);
      for (int wave = 0; wave < NW; ++wave)
        for (int u = 0; u < ins; ++u) {
          const int g = wave * ins + u;
          for (int lane = 0; lane < 64; ++lane) {
            ++g_checked;
            const uint64_t off = tile_dma_offset(g, lane, last, ld, k0, tail ? kext : INT64_MAX);
            const uint64_t abs = (uint64_t)row0 * (uint64_t)ld + off;
            const int64_t row = (int64_t)(abs / (uint64_t)ld), kb = (int64_t)(abs % (uint64_t)ld);
            if (row < 0 || row >= valid || kb + 16 > kext || kb % 16 != 0) {
              if (g_fail++ < 10)
                std::printf("%s: out of bounds valid=%lld ld=%lld kext=%lld row0=%lld k0=%lld g=%d lane=%d -> row %lld k %lld\n",
                            what, (long long)valid, (long long)ld, (long long)kext, (long long)row0, (long long)k0, g,
                            lane, (long long)row, (long long)kb);
              continue;
            }
            const int lds = g * 1024 + 16 * lane, trow = lds / 128, slot = (lds % 128) / 16;
            const int chunk = slot ^ swz(trow);
            const bool is_tail = tile_dma_is_tail(g, lane, k0, kext);
            if (is_tail != (k0 + 16 * chunk >= kext)) {
              if (g_fail++ < 10) std::printf("%s: tail flag mismatch\n", what);
            }
            if (row0 + trow < valid && !is_tail) {
              if (row != row0 + trow || kb != k0 + 16 * chunk) {
                if (g_fail++ < 10)
                  std::printf("%s: slot (%d,%d) got row %lld k %lld, want row %lld k %lld\n", what, trow, slot,
                              (long long)row, (long long)kb, (long long)(row0 + trow), (long long)(k0 + 16 * chunk));
              }
              seen[(size_t)trow * 8 + chunk]++;
            }
          }
        }
      for (int r = 0; r < BM && row0 + r < valid; ++r)
        for (int c = 0; c < 8; ++c)
          if (k0 + 16 * c < kext && seen[(size_t)r * 8 + c] != 1) {
            if (g_fail++ < 10) std::printf("%s: row %d chunk %d delivered %d times\n", what, r, c, seen[(size_t)r * 8 + c]);
          }
    }
    // E8M0 scale rows: 4 per lane, 256 per instruction
    if (valid % 32 == 0) {
      for (int part = 0; part < BM / 256 || part == 0; ++part) {
        if (BM < 256) break;
        for (int lane = 0; lane < 64; ++lane) {
          const int r4 = scale_dma_row(part, lane, last);
          if (r4 < 0 || r4 % 4 != 0 || r4 + 3 > last) {
            if (g_fail++ < 10) std::printf("%s: scale rows %d..%d past last %d\n", what, r4, r4 + 3, last);
          }
        }
      }
    }
  }
}

int main() {
  // wgrad MX: 256 x 256 tiles, 4 waves; operands rows = n or h (multiples of 32), K = Kp_e
  const int64_t cols[] = {32, 64, 96, 256, 320, 2048, 7168};
  const int64_t kps[] = {128, 256, 384, 8704, 19200};
  for (int64_t c : cols)
    for (int64_t kp : kps) check_operand("wgrad-mx", 256, 4, c, kp, kp, false);
  // wgrad per-channel: 128 x 128 tiles, 4 waves
  for (int64_t c : cols)
    for (int64_t kp : kps) check_operand("wgrad-pc", 128, 4, c, kp, kp, false);
  // fprop: A rows = a group's live rows (any count), B rows = n; K any multiple of 32 (tails)
  const int64_t rows[] = {1, 2, 31, 32, 33, 127, 255, 256, 257, 600, 8409};
  const int64_t ks[] = {32, 96, 128, 160, 256, 288, 4096, 7168, 7200};
  for (int64_t r : rows)
    for (int64_t k : ks) check_operand("fprop-a", 256, 4, r, k, k, true);
  for (int64_t n : cols)
    for (int64_t k : ks) check_operand("fprop-b", 256, 4, n, k, k, true);
  std::printf("checked %ld lane loads, %ld violations\n", g_checked, g_fail);
  return g_fail == 0 ? 0 : 1;
}

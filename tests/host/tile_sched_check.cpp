// Host check of the XCD-aware tile order (csrc/tile_sched.hpp), run by tests/test_tile_addr.py:
// over a launch of xcd_launch_size() workgroups every tile is produced exactly once, spare
// workgroups map past the tile count, workgroup 0 gets tile 0, each XCD walks whole runs of
// consecutive logical tiles in increasing order (one run per round of 8, in snake order), and
// the XCDs' shares of the real tiles differ by at most one run -- for runs of 32 (the default)
// and every shorter run length that divides 32 (kSkewRun among them).
#include <cstdint>
#include <cstdio>
#include <vector>

#include "tile_sched.hpp"

using namespace bsfp8;

static long g_fail = 0;

static void check_wgrad(int E, int TM, int TN, int run) {
  const int64_t G = (int64_t)E * TM * TN, B = xcd_launch_size(G);
  std::vector<int> seen((size_t)G, 0);
  for (int64_t b = 0; b < B; ++b) {
    const int64_t L = xcd_logical(b, run);
    if (b == 0 && L != 0) ++g_fail;
    if (L < 0 || L >= B) { ++g_fail; continue; }
    if (L >= G) continue;
    int e, tm, tn;
    wgrad_tile(L, TM, TN, &e, &tm, &tn);
    if (e < 0 || e >= E || tm < 0 || tm >= TM || tn < 0 || tn >= TN) {
      if (g_fail++ < 10) std::printf("wgrad E=%d TM=%d TN=%d: L=%lld -> (%d,%d,%d) out of range\n", E, TM, TN, (long long)L, e, tm, tn);
      continue;
    }
    seen[((size_t)e * TM + tm) * TN + tn]++;
  }
  for (int64_t i = 0; i < G; ++i)
    if (seen[(size_t)i] != 1 && g_fail++ < 10) std::printf("wgrad E=%d TM=%d TN=%d: tile %lld seen %d\n", E, TM, TN, (long long)i, seen[(size_t)i]);
}

static void check_fprop(int64_t MT, int TN) {
  const int64_t gm = fprop_run_mtiles(TN);
  const int64_t G = (MT + gm - 1) / gm * gm * TN, B = xcd_launch_size(G);
  const int64_t mt_cap = (MT + gm - 1) / gm * gm;
  std::vector<int> seen((size_t)(mt_cap * TN), 0);
  for (int64_t b = 0; b < B; ++b) {
    const int64_t L = xcd_logical(b);
    if (L >= G) continue;
    int64_t mt;
    int tn;
    fprop_tile(L, TN, &mt, &tn);
    if (mt < 0 || mt >= mt_cap || tn < 0 || tn >= TN) {
      if (g_fail++ < 10) std::printf("fprop MT=%lld TN=%d: L=%lld -> (%lld,%d)\n", (long long)MT, TN, (long long)L, (long long)mt, tn);
      continue;
    }
    seen[(size_t)(mt * TN + tn)]++;
  }
  for (size_t i = 0; i < seen.size(); ++i)
    if (seen[i] != 1 && g_fail++ < 10) std::printf("fprop MT=%lld TN=%d: tile %zu seen %d\n", (long long)MT, TN, i, seen[i]);
}

int main() {
  // xcd_logical is a bijection of [0, B); XCD x takes one run per round (x, then 15 - x, ...)
  // in increasing order; for any tile count the real tiles per XCD differ by at most one run
  if (xcd_logical(0) != 0 || kCusPerXcd % kSkewRun != 0) ++g_fail;
  for (int run : {32, 16, 8, 4, 2, 1}) {
    for (int64_t tiles : {1, 31, 32, 255, 256, 257, 1000, 3072, 27328, 33792}) {
      const int64_t B = xcd_launch_size(tiles);
      if (B % 256 != 0 || B < tiles || B - tiles >= 256) ++g_fail;
      std::vector<int> seen((size_t)B, 0);
      std::vector<int64_t> real(kXcds, 0), prev(kXcds, -1);
      for (int64_t b = 0; b < B; ++b) {
        const int64_t L = xcd_logical(b, run);
        if (L < 0 || L >= B) { ++g_fail; continue; }
        if (b == 0 && L != 0) ++g_fail;
        seen[(size_t)L]++;
        const int x = (int)(b % kXcds);
        // run r of round q = r / 8 belongs to XCD r % 8 (q even) or 7 - r % 8 (q odd): snake order
        const int64_t r = L / run, q = r / kXcds;
        if (((q & 1) ? kXcds - 1 - r % kXcds : r % kXcds) != x) ++g_fail;
        if (L <= prev[x]) ++g_fail;                     // each XCD walks increasing tiles
        prev[x] = L;
        if (L < tiles) real[x]++;
      }
      for (int v : seen) if (v != 1) ++g_fail;
      int64_t lo = real[0], hi = real[0];
      for (int64_t c : real) { lo = c < lo ? c : lo; hi = c > hi ? c : hi; }
      if (hi - lo > run) {
        if (g_fail++ < 10)
          std::printf("run %d tiles=%lld: XCD shares %lld..%lld\n", run, (long long)tiles, (long long)lo, (long long)hi);
      }
    }
  }
  const int dims[][3] = {{1, 1, 1}, {4, 1, 1}, {4, 8, 8}, {1, 4, 4}, {128, 8, 28}, {32, 6, 16}, {5, 2, 3},
                         {7, 1, 3}, {1024, 1, 1}, {3, 40, 2}, {2, 33, 33}};
  for (auto& d : dims) {
    check_wgrad(d[0], d[1], d[2], kCusPerXcd);
    check_wgrad(d[0], d[1], d[2], kSkewRun);
  }
  for (int64_t MT : {1, 2, 3, 4, 5, 31, 33, 260, 4224})
    for (int TN : {1, 2, 6, 8, 9, 12, 28, 40}) check_fprop(MT, TN);
  std::printf("tile order: %ld violations\n", g_fail);
  return g_fail == 0 ? 0 : 1;
}

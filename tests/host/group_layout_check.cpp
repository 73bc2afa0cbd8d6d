// Host sweep of the per-group colwise layout (csrc/group_layout.hpp), run by
// tests/test_group_layout.py.  For ragged splits (empty groups, 1, 31, 127, 128, 129 rows, one
// large group, 1024 groups) and several channel counts it checks that
//  * the writer's element index of every (group, token t < Kp_e, channel) is a bijection onto
//    [0, C sum Kp_e), each group inside [C P_e, C (P_e + Kp_e)), pad lanes included;
//  * the reader's view (group base + channel * row bytes + t / epb) is the same byte, for one
//    and two codes per byte (in the two-per-byte case each byte holds exactly tokens 2j, 2j+1);
//  * E8M0 bytes (32-row blocks) and per-channel fp32 scales (128-row blocks) are bijections onto
//    [0, C sum Kp_e / 32) and [0, C sum Kp_e / 128), and the reader's group base plus block
//    stride lands on the writer's entry;
//  * the dgrad weight view (split sizes n, ..., n: P_e = e Kp(n)) uses the same strides;
//  * sum Kp_e never exceeds the capacity bound col_rows_bound(R, E) for R = sum k_e.
// Exit status 0 when no violation is found.
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "group_layout.hpp"

using namespace bsfp8;

static long g_fail = 0, g_checked = 0;
#define CHECK(cond, ...)                                   \
  do {                                                     \
    ++g_checked;                                           \
    if (!(cond) && g_fail++ < 20) std::printf(__VA_ARGS__); \
  } while (0)

static void sweep(const std::vector<int64_t>& splits, int64_t C) {
  const int64_t E = (int64_t)splits.size();
  int64_t T = 0, Ptot = 0;
  for (int64_t k : splits) {
    T += k;
    Ptot += col_padded_rows(k);
  }
  CHECK(Ptot <= col_rows_bound(T, E), "rows bound: sum Kp %lld > bound %lld\n", (long long)Ptot,
        (long long)col_rows_bound(T, E));
  std::vector<uint8_t> seen(C * Ptot, 0), seen_b(C * Ptot / 2, 0), seen_s(C * Ptot / 32, 0),
      seen_pc(C * Ptot / 128, 0);
  int64_t P = 0;
  for (int64_t e = 0; e < E; ++e) {
    const int64_t kp = col_padded_rows(splits[e]);
    CHECK(kp % 128 == 0 && kp >= splits[e] && kp < splits[e] + 128, "padded rows %lld for k %lld\n", (long long)kp,
          (long long)splits[e]);
    for (int64_t c = 0; c < C; ++c) {
      for (int64_t t = 0; t < kp; ++t) {
        const int64_t i = col_elem(C, P, kp, c, t);
        CHECK(i >= C * P && i < C * (P + kp), "group %lld element outside its slice\n", (long long)e);
        if (i >= 0 && i < C * Ptot) {
          CHECK(!seen[i], "element %lld written twice\n", (long long)i);
          seen[i] = 1;
        }
        // the GEMM reader: group base + channel row + token, one code per byte
        CHECK(col_group_bytes(C, P, 1) + c * col_row_bytes(kp, 1) + t == i, "reader/writer mismatch (1 per byte)\n");
        // two codes per byte: byte i / 2 holds tokens 2j and 2j + 1 of one channel
        const int64_t b = col_group_bytes(C, P, 2) + c * col_row_bytes(kp, 2) + t / 2;
        CHECK(b == i / 2, "reader/writer mismatch (2 per byte)\n");
        if (t % 2 == 0 && b >= 0 && b < C * Ptot / 2) seen_b[b]++;
      }
      for (int64_t blk = 0; blk < kp / 32; ++blk) {
        const int64_t s = col_e8m0(C, P, blk, c);
        CHECK(s == col_e8m0_group(C, P) + blk * col_e8m0_block_stride(C) + c, "E8M0 reader/writer mismatch\n");
        if (s >= 0 && s < C * Ptot / 32) {
          CHECK(!seen_s[s], "E8M0 entry %lld written twice\n", (long long)s);
          seen_s[s] = 1;
        }
      }
      for (int64_t blk = 0; blk < kp / 128; ++blk) {
        const int64_t s = col_pc_scale(C, P, blk, c);
        CHECK(s == col_pc_scale_group(C, P) + blk * C + c, "fp32 scale reader/writer mismatch\n");
        if (s >= 0 && s < C * Ptot / 128) {
          CHECK(!seen_pc[s], "fp32 scale %lld written twice\n", (long long)s);
          seen_pc[s] = 1;
        }
      }
    }
    P += kp;
  }
  for (size_t i = 0; i < seen.size(); ++i) CHECK(seen[i], "element %zu never written\n", i);
  for (size_t i = 0; i < seen_b.size(); ++i) CHECK(seen_b[i] == 1, "byte %zu holds %d token pairs\n", i, seen_b[i]);
  for (size_t i = 0; i < seen_s.size(); ++i) CHECK(seen_s[i], "E8M0 entry %zu never written\n", i);
  for (size_t i = 0; i < seen_pc.size(); ++i) CHECK(seen_pc[i], "fp32 scale %zu never written\n", i);
}

// dgrad's weight view: E experts of n rows each quantized colwise (split sizes n, ..., n) is
// read as group e at byte e * col_group_bytes(k, Kp(n)), scales at e * col_e8m0_group(k, Kp(n)).
static void sweep_dgrad(int64_t E, int64_t n, int64_t k) {
  const int64_t np = col_padded_rows(n);
  int64_t P = 0;
  for (int64_t e = 0; e < E; ++e) {
    for (int epb = 1; epb <= 2; ++epb) {
      CHECK(col_group_bytes(k, P, epb) == e * col_group_bytes(k, np, epb), "dgrad weight group stride\n");
    }
    CHECK(col_e8m0_group(k, P) == e * col_e8m0_group(k, np), "dgrad weight scale group stride\n");
    P += np;
  }
}

int main() {
  std::mt19937_64 rng(2024);
  const std::vector<std::vector<int64_t>> fixed = {
      {0, 1, 31, 32, 33, 127, 128, 129, 256}, {256, 128, 128, 256}, {0}, {1}, {512}, {300, 0, 45, 1, 200},
      {0, 0, 0, 5}, {1000}, {8588, 0, 8600}};
  for (const auto& s : fixed)
    for (int64_t C : {32, 96, 256}) sweep(s, C);
  std::vector<int64_t> many(1024);
  for (auto& k : many) k = (int64_t)(rng() % 130);
  sweep(many, 32);
  for (int it = 0; it < 40; ++it) {
    std::vector<int64_t> s(1 + rng() % 16);
    for (auto& k : s) k = (rng() % 4 == 0) ? 0 : (int64_t)(rng() % 700);
    sweep(s, 32 * (1 + (int64_t)(rng() % 8)));
  }
  for (int64_t n : {32, 96, 128, 160, 2048})
    for (int64_t E : {1, 4, 128}) sweep_dgrad(E, n, 64);
  std::printf("group layout: %ld checks, %ld failures\n", g_checked, g_fail);
  return g_fail ? 1 : 0;
}

// Tile order of the grouped GEMMs on MI355X: 8 XCDs of 32 CUs, each XCD with its own L2.
//
// The hardware hands workgroup b to XCD b % 8, and each XCD takes its workgroups in increasing
// b.  xcd_logical() renumbers the launch so that the logical tiles go to the XCDs in runs of
// 32 (one per CU of an XCD), eight runs per round, one to each XCD (snake order over the
// rounds, below): the 32 workgroups running together on one XCD
// then read the same few A and B panels at the same K positions through that XCD's L2, and
// every XCD gets the same share of the tiles (also when the tile count is only an upper bound
// and the spare tiles at its end exit at once).  Shorter runs (kSkewRun) trade that sharing for
// balance when the tiles' lengths differ widely: the weight gradient over a skewed split uses
// them, so that the longest group's tiles spread over all eight XCDs instead of filling a few.
// The logical order packs tiles that share operand panels into those runs:
//   wgrad: per group, blocks of `gn` tile columns; inside a block, tile rows then columns
//          (TM x gn tiles with gn = 32 / TM share all A panels and gn B panels).
//   fprop: runs of `gm` m-tiles (rows of the groups' tokens) crossing the TN weight tiles in
//          blocks of `gn`; inside a block, m-tiles then weight tiles.
// Plain C++ for the host-side bijection test and for gfx950.
#pragma once

#include <stdint.h>

#include "tile_addr.hpp"  // BSFP8_HD

namespace bsfp8 {

constexpr int kXcds = 8;
constexpr int kCusPerXcd = 32;
constexpr int kSkewRun = 4;  // run length for a skewed weight-gradient split

// Launch size for `tiles` logical tiles: a whole number of rounds of 8 runs of 32.
BSFP8_HD int64_t xcd_launch_size(int64_t tiles) {
  const int64_t round = (int64_t)kXcds * kCusPerXcd;
  return (tiles + round - 1) / round * round;
}

// Logical tile of workgroup b (launch of xcd_launch_size() workgroups) for runs of `run` tiles
// (a divisor of 32): XCD x = b % 8 takes its j-th workgroup (j = b / 8) from run
// 8 q + (q even ? x : 7 - x) of round q = j / run, at position j % run.  The snake over the
// rounds balances the XCDs' totals when the runs get shorter along the order (the
// weight-gradient order puts the largest groups first when the split is skewed): XCD x takes
// the x-th longest run of one round and the (7-x)-th of the next.  Within an XCD the hardware
// hands the next workgroup to whichever CU frees first.
BSFP8_HD int64_t xcd_logical(int64_t b, int run = kCusPerXcd) {
  const int64_t x = b % kXcds, j = b / kXcds, q = j / run;
  const int64_t r = q * kXcds + ((q & 1) ? kXcds - 1 - x : x);
  return r * run + j % run;
}

// Columns per block of the wgrad order for a TM-row tile grid.
BSFP8_HD int wgrad_block_cols(int tm_count) {
  const int g = kCusPerXcd / tm_count;
  return g > 0 ? g : 1;
}

// wgrad: logical tile L < E * TM * TN -> (group e, tile row tm, tile column tn).
BSFP8_HD void wgrad_tile(int64_t L, int TM, int TN, int* e, int* tm, int* tn) {
  const int64_t per_group = (int64_t)TM * TN;
  *e = (int)(L / per_group);
  const int r = (int)(L % per_group);
  const int gn = wgrad_block_cols(TM);
  const int j = r / (TM * gn);                 // column block
  const int q = r - j * TM * gn;
  const int w = TN - j * gn < gn ? TN - j * gn : gn;  // width of this block
  *tm = q / w;
  *tn = j * gn + q % w;
}

// fprop: weight tiles per column block, and m-tiles per run, for TN weight tiles.  A run of gm
// m-tiles crosses the TN weight tiles in blocks of gn, so the 32 workgroups of an XCD share
// about gm A panels and gn B panels (4 + 8 for wide weights, rather than 1 + 32).
BSFP8_HD int fprop_block_cols(int tn_count) { return tn_count < 8 ? tn_count : 8; }

BSFP8_HD int fprop_run_mtiles(int tn_count) {
  const int g = kCusPerXcd / fprop_block_cols(tn_count);
  return g > 0 ? g : 1;
}

// fprop: logical tile L -> (global m-tile index mt, weight tile tn).
BSFP8_HD void fprop_tile(int64_t L, int TN, int64_t* mt, int* tn) {
  const int gn = fprop_block_cols(TN), gm = fprop_run_mtiles(TN);
  const int64_t run = L / ((int64_t)gm * TN);
  const int r = (int)(L % ((int64_t)gm * TN));
  const int jb = r / (gm * gn);                         // column block
  const int q = r - jb * gm * gn;
  const int w = TN - jb * gn < gn ? TN - jb * gn : gn;  // width of this block
  *mt = run * gm + q / w;
  *tn = jb * gn + q % w;
}

}  // namespace bsfp8

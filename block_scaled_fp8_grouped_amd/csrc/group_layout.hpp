// Per-group colwise layout of the quantized operands: the one definition that the quantize
// kernels (writers), the GEMM descriptors (readers), the dgrad weight view and the size queries
// use, and that a host-side test sweeps over ragged, empty and 1024-group splits.  Plain C++:
// compiles for the host and for gfx950.
//
// Group e holds k_e live rows of a [R][C] buffer.  Its rows are padded to Kp_e = 128 ceil(k_e /
// 128) and the groups are packed one after another along the token axis: P_e = sum_{f<e} Kp_f
// rows precede group e (the per-member strides of the grouped quantizer: TE PR #3224, Greptile
// summary; the K-major per-expert pack of DeepGEMM issue #365, reproducer).  Within a group
// each channel's Kp_e codes are contiguous (token axis fastest), so element (e, t, c) sits at
// element index C P_e + c Kp_e + t; pad lanes k_e <= t < Kp_e hold code 0.  Block scales follow
// the same packing with one entry per block of the token axis, block-major within a group:
// E8M0 bytes (32-row blocks) at C P_e / 32 + b C + c, per-channel fp32 scales (128-row blocks)
// at C P_e / 128 + b C + c.  A data recipe with two codes per byte (MXFP4) stores element index
// i as nibble i % 2 of byte i / 2.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define BSFP8_LAYOUT_HD __host__ __device__ __forceinline__
#else
#define BSFP8_LAYOUT_HD inline
#endif

namespace bsfp8 {

// Padded rows of a group of k live rows.
BSFP8_LAYOUT_HD int64_t col_padded_rows(int64_t k) { return (k + 127) / 128 * 128; }

// Element index of (t, c) in a group whose packed offset is P rows and padded size kp rows, in
// a buffer of C channels; divide by the codes per byte (epb) for the byte offset.
BSFP8_LAYOUT_HD int64_t col_elem(int64_t C, int64_t P, int64_t kp, int64_t c, int64_t t) {
  return C * P + c * kp + t;
}
// Byte offset of the group's first code, and the bytes of one channel's run within the group.
BSFP8_LAYOUT_HD int64_t col_group_bytes(int64_t C, int64_t P, int epb) { return C * P / epb; }
BSFP8_LAYOUT_HD int64_t col_row_bytes(int64_t kp, int epb) { return kp / epb; }

// E8M0 scale of 32-row block b of channel c (byte offset); the group's first scale byte and the
// bytes between consecutive blocks of one channel.
BSFP8_LAYOUT_HD int64_t col_e8m0(int64_t C, int64_t P, int64_t b, int64_t c) { return C * P / 32 + b * C + c; }
BSFP8_LAYOUT_HD int64_t col_e8m0_group(int64_t C, int64_t P) { return C * P / 32; }
BSFP8_LAYOUT_HD int64_t col_e8m0_block_stride(int64_t C) { return C; }

// Per-channel fp32 scale of 128-row block b of channel c (float index), and the group's first.
BSFP8_LAYOUT_HD int64_t col_pc_scale(int64_t C, int64_t P, int64_t b, int64_t c) { return C * P / 128 + b * C + c; }
BSFP8_LAYOUT_HD int64_t col_pc_scale_group(int64_t C, int64_t P) { return C * P / 128; }

// Packed rows any valid split of at most R rows into E groups can need: sum Kp_e <= R + 127 E,
// rounded down to whole 128-row blocks.
BSFP8_LAYOUT_HD int64_t col_rows_bound(int64_t R, int64_t E) { return 128 * ((R + 127 * E) / 128); }

}  // namespace bsfp8

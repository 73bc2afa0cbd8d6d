// Shared device helpers of the block-scaled FP8 grouped kernels (gfx950 / CDNA4).
//
//  * group_scan: every workgroup reads the device-resident split sizes and computes, in LDS,
//    the prefix sums that place its tile (group offsets off_e, padded offsets P_e and tile
//    prefixes), plus the validation of the sizes.  No host copy of the sizes is ever needed
//    (TE PR #3224 review: split sizes stay on the device), and nothing depends on the buffer's
//    capacity beyond the bound check, so one group, empty groups and 128-token groups take
//    the same code (TE #3484, bug description).
//  * e4m3 / E8M0 helpers: the hardware fp8 conversion rounds to nearest even on the OCP
//    E4M3FN grid; the E8M0 exponent is read off the fp32 bit pattern of the block amax.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bsfp8.h"
#include "group_layout.hpp"

namespace bsfp8 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kMaxGroups = BSFP8_MAX_GROUPS;

// ---------------------------------------------------------------------------------------------
// Scale rules
// ---------------------------------------------------------------------------------------------

// MXFP8 block exponent: smallest e with amax <= 448 * 2^e, clamped to [-127, 127].
// amax = 1.m * 2^u (u unbiased); 448 = 1.75 * 2^8, so e = u - 8 when 1.m <= 1.75, else u - 7.
// fp32 subnormals (and 0) are below 448 * 2^-127 and give -127.  For any finite amax the
// result is at most 120, so 2^-e is always a normal fp32.
__device__ __forceinline__ int e8m0_exponent(float amax) {
  const uint32_t bits = __float_as_uint(amax);
  const int ef = (int)((bits >> 23) & 0xffu);
  if (ef == 0) return -127;
  const int u = ef - 127;
  int e = u - 8 + ((bits & 0x7fffffu) > 0x600000u ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// MXFP4 block exponent: smallest e with amax <= 6 * 2^e, clamped to [-127, 127].
// amax = 1.m * 2^u; 6 = 1.5 * 2^2, so e = u - 2 when 1.m <= 1.5, else u - 1.  fp32 subnormals
// (and 0) give -127; for finite amax the result is at most 126.
__device__ __forceinline__ int e8m0_exponent_fp4(float amax) {
  const uint32_t bits = __float_as_uint(amax);
  const int ef = (int)((bits >> 23) & 0xffu);
  if (ef == 0) return -127;
  const int u = ef - 127;
  int e = u - 2 + ((bits & 0x7fffffu) > 0x400000u ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// 2^-e as an fp32 (exact; e in [-127, 126]).
__device__ __forceinline__ float exp2_neg(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }

// 1 / d rounded to nearest even, for d in [1, 2^126]: the hardware reciprocal (within 1 ulp)
// and one Newton step with fused multiply-adds, r + r (1 - d r).  On that domain it equals
// the IEEE division 1.0f / d for every fp32 d (checked exhaustively on the GPU through
// bsfp8_recip_check); above 2^126, where 1 / d is subnormal, it does not, and callers keep d
// within the domain.  Three instructions instead of the division's ten.
__device__ __forceinline__ float recip_rn(float d) {
  const float r = __builtin_amdgcn_rcpf(d);
  const float e = __builtin_fmaf(-d, r, 1.0f);
  return __builtin_fmaf(e, r, r);
}

// Two fp32 -> two e4m3 codes in the low 16 bits (round to nearest even, sign kept).
__device__ __forceinline__ uint32_t e4m3x2(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}
// Four fp32 -> four e4m3 codes packed little-endian in a dword.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Eight fp32 -> eight e2m1 codes packed in a dword, element i in bits 4i..4i+3 (round to
// nearest even, sign kept, magnitudes above 6 saturate; unit conversion scale).
__device__ __forceinline__ uint32_t e2m1x8(float a0, float a1, float a2, float a3, float a4, float a5, float a6,
                                           float a7) {
  uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a0, a1, 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a2, a3, 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a4, a5, 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a6, a7, 1.0f, 3);
  return w;
}

// bf16 halves of a dword -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, rounded to nearest even by the hardware conversion (v_cvt_pk_bf16_f32, one
// instruction): on every non-NaN fp32 it equals the integer round-to-nearest-even of the top 16
// bits, and a NaN stays a NaN (checked over all 2^32 patterns on the GPU: bsfp8_bf16_cvt_check
// in the probe library).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// ---------------------------------------------------------------------------------------------
// Group scan
// ---------------------------------------------------------------------------------------------

__device__ __forceinline__ int64_t wave_inclusive_scan(int64_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t u = __shfl_up(v, d, 64);
    if (lane >= d) v += u;
  }
  return v;
}

// Where a workgroup's tile sits: its group and the group's row extents.
struct GroupInfo {
  int64_t k;    // live rows of the group
  int64_t off;  // first row of the group in the token buffer
  int64_t kp;   // rows rounded up to 128
  int64_t p;    // sum of kp over earlier groups (colwise packed offset, in rows)
  int64_t tile; // first linear tile index of the group (tile_rows > 0 only)
  int32_t e;    // group index, or -1 when the workgroup has no tile
};

template <int NT>
struct GroupScanSmem {
  int64_t wave_tot[NT / 64][3];
  int64_t wave_aux[NT / 64][2];  // per wave: largest size, live groups
  int32_t tile_prefix[kMaxGroups + 1];  // the sizes, for the ranking
  int64_t info[5];
  int32_t sel;
  uint32_t flags;
};

// Size skew at which the weight-gradient GEMM takes its groups largest first: the largest group
// holds more than kSkewRatio times the mean size of the non-empty groups.  Each group's tiles
// run for as many K steps as it has padded rows, so with a skewed split the largest groups
// decide the kernel's end; started first, they finish beside the rest (longest-processing-time
// order).  Near-uniform splits keep index order.  Ranking is done for at most kRankMaxGroups
// groups (every workgroup ranks the sizes itself).
constexpr int kSkewRatio = 2;
constexpr int kRankMaxGroups = 256;

// Scans split_sizes[0..E) across the workgroup.  tile_rows > 0 makes each group own
// ceil(k_e / tile_rows) tiles, and the workgroup's linear tile `tile_index` is mapped to its
// group (binary search over the tile prefix).  tile_rows == 0 selects group g = pick(skewed)
// (pick is called with the same argument by every thread and must return the same value;
// g < 0: no group), where, with `by_size` and a skewed split (kSkewRatio), skewed is true and g
// is a size rank: groups ordered by decreasing size, equal sizes by index.  The rank and the
// skew depend on split_sizes only.  Returns the validation bits (BSFP8_STATUS_*); GroupInfo.e
// is -1 when there is no group to select (a tile beyond the last group's tiles, g < 0) or when
// the sizes are invalid.
template <int NT, class Pick>
__device__ uint32_t group_scan(const int32_t* __restrict__ splits, int E, int64_t capacity,
                               int tile_rows, int64_t tile_index, Pick pick,
                               GroupScanSmem<NT>& sm, GroupInfo& gi, bool by_size = false) {
  constexpr int kItems = (kMaxGroups + NT - 1) / NT;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  int64_t k[kItems], kp[kItems], tl[kItems];
  int64_t sk = 0, skp = 0, stl = 0, kmax = 0, nlive = 0;
  uint32_t bad = 0;
#pragma unroll
  for (int i = 0; i < kItems; ++i) {
    const int e = tid * kItems + i;
    const int64_t v = e < E ? (int64_t)splits[e] : 0;
    if (v < 0) bad |= BSFP8_STATUS_NEGATIVE_SPLIT;
    k[i] = v < 0 ? 0 : v;
    kp[i] = col_padded_rows(k[i]);
    tl[i] = tile_rows > 0 ? (k[i] + tile_rows - 1) / tile_rows : 0;
    sk += k[i];
    skp += kp[i];
    stl += tl[i];
    kmax = k[i] > kmax ? k[i] : kmax;
    nlive += k[i] > 0;
  }
  const bool rank = by_size && tile_rows == 0 && E <= kRankMaxGroups;
  // without ranking the selection is known now and is published by the prefix pass below
  const int group_index = tile_rows == 0 && !rank ? pick(false) : -1;
  if (rank) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      const int64_t m = __shfl_xor(kmax, d, 64), c = __shfl_xor(nlive, d, 64);
      kmax = m > kmax ? m : kmax;
      nlive += c;
    }
  }
  // exclusive prefix of the per-thread sums across the workgroup
  const int64_t ik = wave_inclusive_scan(sk), ikp = wave_inclusive_scan(skp), itl = wave_inclusive_scan(stl);
  if (tid == 0) {
    sm.flags = 0;
    // With tiles, no group may own tile_index, so the selection starts unset; a selection by
    // index or rank always writes it.  Only the tile kernels clear it: in the weight-gradient
    // kernel the same store left every result bit unchanged but its launches fetched 35 -> 59
    // GB from beyond L2 (measured A/B on the 128-expert shape; the cause was not found).
    if (tile_rows > 0) sm.sel = -1;
  }
  if (lane == 63) {
    sm.wave_tot[wave][0] = ik;
    sm.wave_tot[wave][1] = ikp;
    sm.wave_tot[wave][2] = itl;
  }
  if (rank) {
    if (lane == 0) {
      sm.wave_aux[wave][0] = kmax;
      sm.wave_aux[wave][1] = nlive;
    }
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      const int e = tid * kItems + i;
      if (e < E) sm.tile_prefix[e] = (int32_t)k[i];  // the sizes, for the ranking below
    }
  }
  __syncthreads();
  if (bad) atomicOr(&sm.flags, bad);
  int64_t bk = ik - sk, bkp = ikp - skp, btl = itl - stl, tot = 0;
  for (int w = 0; w < NT / 64; ++w) {
    if (w < wave) {
      bk += sm.wave_tot[w][0];
      bkp += sm.wave_tot[w][1];
      btl += sm.wave_tot[w][2];
    }
    tot += sm.wave_tot[w][0];
  }
  // per-entry exclusive prefixes; the selected group publishes its extents: with tiles, the one
  // whose tile range [otl, otl + tl) holds tile_index (none when it is past the last group's
  // tiles), else group group_index
  int64_t ok = bk, okp = bkp, otl = btl;
#pragma unroll
  for (int i = 0; i < kItems; ++i) {
    const int e = tid * kItems + i;
    const bool sel = tile_rows > 0 ? e < E && tile_index >= otl && tile_index < otl + tl[i]
                                   : e == group_index && e < E;
    if (sel) {
      sm.info[0] = k[i];
      sm.info[1] = ok;
      sm.info[2] = kp[i];
      sm.info[3] = okp;
      sm.info[4] = otl;
      sm.sel = e;
    }
    ok += k[i];
    okp += kp[i];
    otl += tl[i];
  }
  __syncthreads();
  uint32_t flags = sm.flags;
  if (tot > capacity) flags |= BSFP8_STATUS_EXCEEDS_CAPACITY;
  gi.e = -1;
  if (flags) return flags;
  if (tile_rows > 0) {
    if (sm.sel < 0) return 0;  // past the last group's tiles
    gi.e = sm.sel;
    gi.tile = sm.info[4];
  } else if (rank) {
    int64_t big = 0, live = 0;
    for (int w = 0; w < NT / 64; ++w) {
      big = sm.wave_aux[w][0] > big ? sm.wave_aux[w][0] : big;
      live += sm.wave_aux[w][1];
    }
    const bool skewed = big * live > (int64_t)kSkewRatio * tot;
    const int g = pick(skewed);
    if (g < 0) return 0;
    // the selected group (skewed: the one of size rank g; else group g) publishes its extents
    int64_t ok2 = bk, okp2 = bkp;
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      const int e = tid * kItems + i;
      if (e < E) {
        int r = e;
        if (skewed) {
          r = 0;
          for (int f = 0; f < E; ++f) {
            const int32_t kf = sm.tile_prefix[f];
            r += (kf > (int32_t)k[i]) || (kf == (int32_t)k[i] && f < e);
          }
        }
        if (r == g) {
          sm.info[0] = k[i];
          sm.info[1] = ok2;
          sm.info[2] = kp[i];
          sm.info[3] = okp2;
          sm.sel = e;
        }
      }
      ok2 += k[i];
      okp2 += kp[i];
    }
    __syncthreads();
    gi.e = sm.sel;
    gi.tile = 0;
  } else {
    if (group_index < 0) return 0;
    gi.e = group_index;
    gi.tile = 0;
  }
  gi.k = sm.info[0];
  gi.off = sm.info[1];
  gi.kp = sm.info[2];
  gi.p = sm.info[3];
  return 0;
}

// group_scan selecting a fixed group index (ignored when tile_rows > 0).
template <int NT>
__device__ uint32_t group_scan(const int32_t* __restrict__ splits, int E, int64_t capacity,
                               int tile_rows, int64_t tile_index, int group_index,
                               GroupScanSmem<NT>& sm, GroupInfo& gi, bool by_size = false) {
  return group_scan<NT>(splits, E, capacity, tile_rows, tile_index, [group_index](bool) { return group_index; }, sm,
                        gi, by_size);
}

// OR the validation bits into the caller's status word (one thread of workgroup 0 only).
__device__ __forceinline__ void report_status(uint32_t* status, uint32_t flags) {
  if (status != nullptr && flags != 0 && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0)
    atomicOr(status, flags);
}

}  // namespace bsfp8

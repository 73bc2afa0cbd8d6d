// Probe library (libbsfp8_peak.so).  The MFMA-only throughput probe: the rate the matrix cores
// sustain on this machine with nothing else in the loop, to set the grouped GEMMs against.  The
// precision probe: one 32 x 32 block-scaled e4m3 dot product through each candidate matrix
// instruction, which shows why the MXFP8 GEMMs run the bf16 MFMA on widened codes.  And the
// checks of the fast reciprocal that the fused SwiGLU uses against the IEEE division, and of the
// GEMMs' hardware fp32 -> bf16 conversion against an integer round-to-nearest-even.
//
// Each wave holds its A and B operands in registers (read once from the caller's pool) and
// issues 4 independent accumulator chains of one instruction per iteration; with 2 workgroups
// of 4 waves per CU the MFMA pipe of every SIMD always has an independent instruction ready.
// Optionally the first wave of each workgroup stamps the shader-clock counter and the
// constant-rate real-time counter around its loop, which gives the clock the chip held.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsfp8_peak.h"
#include "common.hpp"  // recip_rn, the reciprocal under test

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int int4v __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kChains = 4;

template <int KIND>
__global__ __launch_bounds__(BSFP8_PEAK_THREADS) void mfma_peak_kernel(const uint32_t* __restrict__ pool,
                                                                        float* __restrict__ out, int64_t iters,
                                                                        uint64_t* __restrict__ stamps) {
  const int64_t t = (int64_t)blockIdx.x * BSFP8_PEAK_THREADS + threadIdx.x;
  v8i a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (int)pool[(t * 16 + i) & (BSFP8_PEAK_POOL_WORDS - 1)];
    b[i] = (int)pool[(t * 16 + 8 + i) & (BSFP8_PEAK_POOL_WORDS - 1)];
  }
  v16f acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = v16f{};
  uint64_t clk0 = 0, rt0 = 0;
  if (stamps != nullptr && threadIdx.x == 0) {
    clk0 = __builtin_amdgcn_s_memtime();
    rt0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
      if constexpr (KIND == BSFP8_PEAK_BF16) {
        const v4i a4 = v4i{a[0], a[1], a[2], a[3]}, b4 = v4i{b[0], b[1], b[2], b[3]};
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a4), __builtin_bit_cast(v8bf, b4),
                                                         acc[c], 0, 0, 0);
      } else if constexpr (KIND == BSFP8_PEAK_FP8) {
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 0, 0, 0, 127, 0, 127);
      } else {
        const v8i a4 = v8i{a[0], a[1], a[2], a[3], 0, 0, 0, 0}, b4 = v8i{b[0], b[1], b[2], b[3], 0, 0, 0, 0};
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a4, b4, acc[c], 4, 4, 0, 127, 0, 127);
      }
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  if (stamps != nullptr && threadIdx.x == 0) {
    // the end stamps follow the sum of every accumulator, i.e. the wave's last MFMA result
    asm volatile("" ::"v"(s));
    const uint64_t clk1 = __builtin_amdgcn_s_memtime(), rt1 = __builtin_amdgcn_s_memrealtime();
    stamps[4 * blockIdx.x + 0] = clk0;
    stamps[4 * blockIdx.x + 1] = rt0;
    stamps[4 * blockIdx.x + 2] = clk1;
    stamps[4 * blockIdx.x + 3] = rt1;
  }
  out[t] = s;
}

// 64 consecutive bit patterns per thread from lo; mismatching patterns are counted and the
// lowest one kept.
__global__ __launch_bounds__(256) void recip_check_kernel(uint32_t lo, uint32_t count, unsigned long long* mism,
                                                          uint32_t* first) {
  const uint64_t base = ((uint64_t)blockIdx.x * 256 + threadIdx.x) * 64;
  unsigned long long local = 0;
  uint32_t low = 0xFFFFFFFFu;
  for (int i = 0; i < 64; ++i) {
    const uint64_t j = base + i;
    if (j >= count) break;
    const uint32_t bits = lo + (uint32_t)j;
    const float d = __uint_as_float(bits);
    if (__float_as_uint(bsfp8::recip_rn(d)) != __float_as_uint(1.0f / d)) {
      ++local;
      low = low < bits ? low : bits;
    }
  }
  if (local) {
    atomicAdd(mism, local);
    atomicMin(first, low);
  }
}

// The GEMMs' fp32 -> bf16 output conversion (the hardware one, bsfp8::f32_to_bf16) against an
// integer rounding of the fp32 bits written out here: mode 0 round to nearest even (carry
// 0x7fff plus the kept lowest bit into the top half), mode 1 truncation (a reference that
// must differ, so the check is seen to catch differences).  A NaN input must give a bf16 NaN;
// any other input the reference's bits.  64 consecutive patterns per thread from lo;
// mismatching patterns are counted and the lowest one kept.
__global__ __launch_bounds__(256) void bf16_cvt_check_kernel(uint32_t lo, uint32_t count, int mode,
                                                             unsigned long long* mism, uint32_t* first) {
  const uint64_t base = ((uint64_t)blockIdx.x * 256 + threadIdx.x) * 64;
  unsigned long long local = 0;
  uint32_t low = 0xFFFFFFFFu;
  for (int i = 0; i < 64; ++i) {
    const uint64_t j = base + i;
    if (j >= count) break;
    const uint32_t bits = lo + (uint32_t)j;
    const uint32_t got = bsfp8::f32_to_bf16(__uint_as_float(bits));
    const bool nan_in = (bits & 0x7f800000u) == 0x7f800000u && (bits & 0x007fffffu) != 0;
    bool bad;
    if (nan_in) {
      bad = (got & 0x7f80u) != 0x7f80u || (got & 0x007fu) == 0;
    } else {
      const uint32_t want = mode == 0 ? (bits + 0x7fffu + ((bits >> 16) & 1u)) >> 16 : bits >> 16;
      bad = got != (want & 0xffffu);
    }
    if (bad) {
      ++local;
      low = low < bits ? low : bits;
    }
  }
  if (local) {
    atomicAdd(mism, local);
    atomicMin(first, low);
  }
}

// Eight e4m3 codes -> eight bf16 values times `scale` (exact: 4 significant bits).
__device__ __forceinline__ v8bf widen8(v2i d, float scale) {
  const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)d[0], scale, false);
  const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)d[0], scale, true);
  const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)d[1], scale, false);
  const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)d[1], scale, true);
  return v8bf{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Two 16-byte pieces, `gap` bytes apart, as one 8-register operand.
__device__ __forceinline__ v8i halves(const uint8_t* p, int gap) {
  const v4i lo = *(const v4i*)p, hi = *(const v4i*)(p + gap);
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// One wave computes C[i][j] = sum_t A[i][t] B[j][t] for 32 x 32 outputs over k e4m3 values per row
// with one matrix instruction, each operand given as 32 rows of k codes and E8M0 scales per 32
// along k (block b of row r at b * 32 + r).  KIND picks the instruction (BSFP8_DOT_*):
//  - BF16: every code widened to bf16 with its block scale folded in (exact), then the bf16 MFMA
//    32x32x16; lane l supplies row l % 32 and the 8 values [k0 + 8 (l / 32), +8) of a K=16 step;
//  - FP8_32X32X64: the scaled MFMA with e4m3 operands.  Lane l = 32 h + r supplies row r of a K=64
//    step as two 16-code halves, [k0 + 16 h, +16) in its first four registers and
//    [k0 + 32 + 16 h, +16) in the last four, and the scale byte of block h of the step
//    ([k0 + 32 h, +32)): the codes of one scale block are split over the lane pair (r, r + 32).
//    (Measured: with each lane holding one whole block instead, blocks get each other's scales.)
//  - FP8_16X16X128: the same at 16 x 16 x 128: lane l = 16 q + r supplies row r as
//    [k0 + 16 q, +16) and [k0 + 64 + 16 q, +16), and the scale of block q; four output tiles;
//  - FP8_LEGACY: the unscaled fp8 MFMA 32x32x16 (lane l: row l % 32, codes [k0 + 8 (l / 32), +8));
//    the scales are not applied.
// A 32 x 32 fp32 result of the 32 x 32 forms: lane l holds column l % 32, its element r row
// 8 (r / 4) + 4 (l / 32) + r % 4; of the 16 x 16 form: column l % 16, element r row 4 (l / 16) + r.
template <int KIND>
__global__ __launch_bounds__(64) void mfma_dot_kernel(const uint8_t* __restrict__ a_q, const uint8_t* __restrict__ a_s,
                                                      const uint8_t* __restrict__ b_q, const uint8_t* __restrict__ b_s,
                                                      int k, float* __restrict__ out) {
  const int lane = threadIdx.x;
  if constexpr (KIND == BSFP8_DOT_FP8_16X16X128) {
    const int r = lane & 15, q = lane >> 4;
    v4f acc[2][2] = {};
    for (int k0 = 0; k0 < k; k0 += 128) {
      const int kk = k0 + 32 * q;
      v8i a[2], b[2];
      int sa[2], sb[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        a[t] = halves(a_q + (int64_t)(16 * t + r) * k + k0 + 16 * q, 64);
        b[t] = halves(b_q + (int64_t)(16 * t + r) * k + k0 + 16 * q, 64);
        sa[t] = a_s[(kk / 32) * 32 + 16 * t + r];
        sb[t] = b_s[(kk / 32) * 32 + 16 * t + r];
      }
#pragma unroll
      for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int tj = 0; tj < 2; ++tj)
          acc[ti][tj] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[ti], b[tj], acc[ti][tj], 0, 0, 0, sa[ti], 0,
                                                                         sb[tj]);
    }
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int tj = 0; tj < 2; ++tj)
#pragma unroll
        for (int e = 0; e < 4; ++e) out[(16 * ti + 4 * q + e) * 32 + 16 * tj + r] = acc[ti][tj][e];
  } else {
    const int r = lane & 31, h = lane >> 5;
    v16f acc = {};
    if constexpr (KIND == BSFP8_DOT_FP8_32X32X64) {
      for (int k0 = 0; k0 < k; k0 += 64) {
        const int kk = k0 + 32 * h;
        const v8i a = halves(a_q + (int64_t)r * k + k0 + 16 * h, 32);
        const v8i b = halves(b_q + (int64_t)r * k + k0 + 16 * h, 32);
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, 0, a_s[(kk / 32) * 32 + r], 0,
                                                              b_s[(kk / 32) * 32 + r]);
      }
    } else {
      for (int k0 = 0; k0 < k; k0 += 16) {
        const int kk = k0 + 8 * h;
        const v2i a = *(const v2i*)(a_q + (int64_t)r * k + kk), b = *(const v2i*)(b_q + (int64_t)r * k + kk);
        if constexpr (KIND == BSFP8_DOT_FP8_LEGACY) {
          acc = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(__builtin_bit_cast(long, a), __builtin_bit_cast(long, b),
                                                           acc, 0, 0, 0);
        } else {
          const float fa = __uint_as_float(max((uint32_t)a_s[(kk / 32) * 32 + r] << 23, 0x00400000u));
          const float fb = __uint_as_float(max((uint32_t)b_s[(kk / 32) * 32 + r] << 23, 0x00400000u));
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(widen8(a, fa), widen8(b, fb), acc, 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) out[(8 * (e / 4) + 4 * h + e % 4) * 32 + r] = acc[e];
  }
}

// Global -> LDS DMA throughput: workgroup b streams its source region (src + b * span, or src
// itself when `shared`) into LDS, each wave 8 KB per round as 8 buffer_load_dwordx4 ... lds of
// 64 lanes x 16 bytes into its own 8 KB of LDS, then waits for them and meets the other waves
// at a barrier; round r of wave w takes the region's bytes from offset
// (r * waves * 8 KB + w * 8 KB + u * 1 KB) mod span, instruction u.  After the last round every
// lane XORs the 8 dwords-x4 it moved in that round (read back from LDS) into out[b * 64 * waves
// + t], so the caller can check that the DMA delivered the bytes it names.
__device__ __forceinline__ int4v rsrc4(const void* base, uint32_t num_records) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return int4v{__builtin_amdgcn_readfirstlane((int)(uint32_t)a), __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffff)),
               __builtin_amdgcn_readfirstlane((int)num_records), 0x00020000};
}

__global__ __launch_bounds__(512) void lds_dma_kernel(const uint8_t* __restrict__ src, uint32_t span, int shared,
                                                      int rounds, uint32_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t sm[8 * 8192];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, nw = blockDim.x >> 6;
  const uint8_t* base = src + (shared ? 0 : (uint64_t)blockIdx.x * span);
  const int4v rs = rsrc4(base, span);
  const uint32_t lds0 =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)(sm + w * 8192));
  const uint32_t per_round = (uint32_t)nw * 8192u;
  for (int r = 0; r < rounds; ++r) {
    const uint32_t off = (uint32_t)r * per_round + (uint32_t)w * 8192u + (uint32_t)lane * 16u;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t o = (off + (uint32_t)u * 1024u) % span;
      asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(o), "s"(rs), "{m0}"(lds0 + u * 1024u)
                   : "memory");
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
  uint32_t x = 0;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int4v v = *(const int4v*)(sm + w * 8192 + u * 1024 + lane * 16);
    x ^= (uint32_t)(v[0] ^ v[1] ^ v[2] ^ v[3]);
  }
  out[(uint64_t)blockIdx.x * blockDim.x + t] = x;
}

double mfma_flops(int kind) {
  switch (kind) {
    case BSFP8_PEAK_BF16: return 2.0 * 32 * 32 * 16;
    case BSFP8_PEAK_FP8:
    case BSFP8_PEAK_FP4: return 2.0 * 32 * 32 * 64;
    default: return 0.0;
  }
}

}  // namespace

extern "C" int bsfp8_mfma_peak_probe(int kind, const uint32_t* pool, float* out, int64_t blocks, int64_t iters,
                                     uint64_t* stamps, void* stream) {
  if (pool == nullptr || out == nullptr) return -1;
  if (mfma_flops(kind) == 0.0) return -2;
  if (blocks < 1 || blocks > 65536 || iters < 1 || iters > (int64_t(1) << 31)) return -3;
  const dim3 grid((unsigned)blocks), block(BSFP8_PEAK_THREADS);
  hipStream_t s = (hipStream_t)stream;
  switch (kind) {
    case BSFP8_PEAK_BF16:
      hipLaunchKernelGGL(mfma_peak_kernel<BSFP8_PEAK_BF16>, grid, block, 0, s, pool, out, iters, stamps);
      break;
    case BSFP8_PEAK_FP8:
      hipLaunchKernelGGL(mfma_peak_kernel<BSFP8_PEAK_FP8>, grid, block, 0, s, pool, out, iters, stamps);
      break;
    default:
      hipLaunchKernelGGL(mfma_peak_kernel<BSFP8_PEAK_FP4>, grid, block, 0, s, pool, out, iters, stamps);
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" double bsfp8_mfma_peak_flops(int kind, int64_t blocks, int64_t iters) {
  return mfma_flops(kind) * (double)blocks * (BSFP8_PEAK_THREADS / 64) * (double)iters * kChains;
}

extern "C" int bsfp8_wall_clock_khz(int device) {
  int khz = 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, device) != hipSuccess) return -1;
  return khz;
}

extern "C" int bsfp8_mfma_dot_probe(int kind, const uint8_t* a_q, const uint8_t* a_s, const uint8_t* b_q,
                                    const uint8_t* b_s, int64_t k, float* out, void* stream) {
  if (a_q == nullptr || a_s == nullptr || b_q == nullptr || b_s == nullptr || out == nullptr) return -1;
  if (kind < BSFP8_DOT_BF16 || kind > BSFP8_DOT_FP8_LEGACY) return -2;
  if (k < 128 || k > 65536 || k % 128 != 0) return -3;
  if (((uintptr_t)a_q | (uintptr_t)b_q) % 32 != 0) return -5;
  hipStream_t s = (hipStream_t)stream;
  const int kk = (int)k;
  switch (kind) {
    case BSFP8_DOT_BF16:
      hipLaunchKernelGGL(mfma_dot_kernel<BSFP8_DOT_BF16>, dim3(1), dim3(64), 0, s, a_q, a_s, b_q, b_s, kk, out);
      break;
    case BSFP8_DOT_FP8_32X32X64:
      hipLaunchKernelGGL(mfma_dot_kernel<BSFP8_DOT_FP8_32X32X64>, dim3(1), dim3(64), 0, s, a_q, a_s, b_q, b_s, kk, out);
      break;
    case BSFP8_DOT_FP8_16X16X128:
      hipLaunchKernelGGL(mfma_dot_kernel<BSFP8_DOT_FP8_16X16X128>, dim3(1), dim3(64), 0, s, a_q, a_s, b_q, b_s, kk,
                         out);
      break;
    default:
      hipLaunchKernelGGL(mfma_dot_kernel<BSFP8_DOT_FP8_LEGACY>, dim3(1), dim3(64), 0, s, a_q, a_s, b_q, b_s, kk, out);
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int bsfp8_lds_dma_probe(const uint8_t* src, int64_t span, int shared, int64_t blocks, int waves,
                                   int64_t rounds, uint32_t* out, void* stream) {
  if (src == nullptr || out == nullptr) return -1;
  if (span < 8192 || span > (int64_t(1) << 31) || span % 1024 != 0) return -3;
  if (blocks < 1 || blocks > 4096 || waves < 1 || waves > 8 || rounds < 1 || rounds > 100000) return -3;
  hipLaunchKernelGGL(lds_dma_kernel, dim3((unsigned)blocks), dim3(64 * waves), 0, (hipStream_t)stream, src,
                     (uint32_t)span, shared ? 1 : 0, (int)rounds, out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int bsfp8_bf16_cvt_check(uint32_t lo_bits, uint32_t hi_bits, int mode, unsigned long long* mismatches,
                                    uint32_t* first_bits, void* stream) {
  if (mismatches == nullptr || first_bits == nullptr) return -1;
  if (mode != 0 && mode != 1) return -2;
  if (hi_bits <= lo_bits) return -3;
  const uint32_t count = hi_bits - lo_bits;
  const uint64_t blocks = ((uint64_t)count + 64 * 256 - 1) / (64 * 256);
  hipLaunchKernelGGL(bf16_cvt_check_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, lo_bits,
                     count, mode, mismatches, first_bits);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int bsfp8_recip_check(uint32_t lo_bits, uint32_t hi_bits, unsigned long long* mismatches,
                                 uint32_t* first_bits, void* stream) {
  if (mismatches == nullptr || first_bits == nullptr) return -1;
  if (hi_bits <= lo_bits) return -3;
  const uint32_t count = hi_bits - lo_bits;
  const uint64_t blocks = ((uint64_t)count + 64 * 256 - 1) / (64 * 256);
  hipLaunchKernelGGL(recip_check_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, lo_bits, count,
                     mismatches, first_bits);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

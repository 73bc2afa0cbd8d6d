// Probe library (libbsfp8_peak.so).  The MFMA-only throughput probe: the rate the matrix cores
// sustain on this machine with nothing else in the loop, to set the grouped GEMMs against.  And
// the check of the fast reciprocal that the fused SwiGLU uses against the IEEE division.
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
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

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

/*
 * A plain C caller of libbsfp8.so on the GPU, with no Python and no torch: it allocates device
 * buffers with the HIP runtime, sizes them with the library's size queries, runs the grouped
 * quantize (MXFP8 colwise) of dy and x and the k-grouped weight gradient through the C ABI
 * declared in include/bsfp8.h, and checks the results against the CPU oracle (liboracle.so):
 * quantized bytes and scales bit for bit, the gradient within a per-expert relative Frobenius
 * error of 1e-5.  Groups of 200, 0, 33 and 128 rows, 64 padding rows of garbage bf16 bits.
 *
 * Test infrastructure (it links the oracle); tests/test_gpu_c_abi.py builds and runs it.
 * Exit status 0 when every check passes.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "bsfp8.h"

/* the oracle's C entry points (oracle/oracle.c) */
int oracle_grouped_quantize(const uint16_t* in, int64_t R, int64_t C, const int32_t* splits, int32_t E, int recipe,
                            int which, float zero_amax_scale, uint8_t* row_q, uint8_t* row_s, uint8_t* col_q,
                            void* col_s);
int oracle_grouped_wgrad(const uint8_t* dy_q, const void* dy_s, int64_t n, const uint8_t* x_q, const void* x_s,
                         int64_t h, const int32_t* splits, int32_t E, int64_t R, int recipe, const int32_t* rows_sel,
                         int32_t n_sel, int accumulate, const float* mg_in, double* out);
int64_t oracle_padded_rows(const int32_t* splits, int32_t E);

#define CHECK_HIP(x)                                                              \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
      exit(2);                                                                    \
    }                                                                             \
  } while (0)
#define CHECK_LIB(x)                                                                    \
  do {                                                                                  \
    int r_ = (x);                                                                       \
    if (r_ != 0) {                                                                      \
      fprintf(stderr, "%s:%d: library error %d: %s\n", __FILE__, __LINE__, r_, bsfp8_strerror(r_)); \
      exit(2);                                                                          \
    }                                                                                   \
  } while (0)

/* splitmix64: the inputs' random bits */
static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static uint64_t next_u64(void) {
  uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}
/* a standard normal value (Box-Muller) rounded to bf16 (nearest even) */
static uint16_t randn_bf16(void) {
  const double u1 = ((next_u64() >> 11) + 1.0) / 9007199254740993.0, u2 = (next_u64() >> 11) / 9007199254740992.0;
  const float v = (float)(sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2));
  uint32_t b;
  memcpy(&b, &v, 4);
  b += 0x7fffu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

static void* dev_upload(const void* host, size_t bytes) {
  void* d = NULL;
  CHECK_HIP(hipMalloc(&d, bytes ? bytes : 16));
  if (bytes) CHECK_HIP(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
  return d;
}

int main(void) {
  const int32_t splits[] = {200, 0, 33, 128};
  const int32_t E = 4;
  const int64_t T = 361, R = T + 64, n = 64, h = 128;
  const int recipe = BSFP8_RECIPE_MX_1X32_E8M0;
  int failures = 0;

  uint16_t* dy = (uint16_t*)malloc(R * n * 2);
  uint16_t* x = (uint16_t*)malloc(R * h * 2);
  for (int64_t i = 0; i < R * n; ++i) dy[i] = i < T * n ? randn_bf16() : (uint16_t)next_u64(); /* garbage padding */
  for (int64_t i = 0; i < R * h; ++i) x[i] = i < T * h ? randn_bf16() : (uint16_t)next_u64();

  /* device side, sized by the library's queries */
  const size_t dq_bytes = bsfp8_colwise_data_bytes(R, n, E, recipe), ds_bytes = bsfp8_colwise_scale_bytes(R, n, E, recipe);
  const size_t xq_bytes = bsfp8_colwise_data_bytes(R, h, E, recipe), xs_bytes = bsfp8_colwise_scale_bytes(R, h, E, recipe);
  void* d_dy = dev_upload(dy, R * n * 2);
  void* d_x = dev_upload(x, R * h * 2);
  int32_t* d_splits = (int32_t*)dev_upload(splits, sizeof(splits));
  uint8_t *d_dq, *d_ds, *d_xq, *d_xs;
  float* d_out;
  uint32_t* d_status;
  CHECK_HIP(hipMalloc((void**)&d_dq, dq_bytes));
  CHECK_HIP(hipMalloc((void**)&d_ds, ds_bytes));
  CHECK_HIP(hipMalloc((void**)&d_xq, xq_bytes));
  CHECK_HIP(hipMalloc((void**)&d_xs, xs_bytes));
  CHECK_HIP(hipMalloc((void**)&d_out, E * n * h * 4));
  CHECK_HIP(hipMalloc((void**)&d_status, 4));
  CHECK_HIP(hipMemset(d_status, 0, 4));
  CHECK_HIP(hipMemset(d_out, 0xff, E * n * h * 4)); /* NaN bits: every output must be written */
  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));

  CHECK_LIB(bsfp8_grouped_quantize(d_dy, R, n, d_splits, E, recipe, BSFP8_COLWISE, 1e-30f, NULL, NULL, d_dq, d_ds, NULL,
                                   d_status, (void*)stream));
  CHECK_LIB(bsfp8_grouped_quantize(d_x, R, h, d_splits, E, recipe, BSFP8_COLWISE, 1e-30f, NULL, NULL, d_xq, d_xs, NULL,
                                   d_status, (void*)stream));
  CHECK_LIB(bsfp8_grouped_gemm_wgrad(d_dq, d_ds, n, d_xq, d_xs, h, d_splits, E, R, recipe, d_out, 0, d_status,
                                     (void*)stream));
  CHECK_HIP(hipStreamSynchronize(stream));

  uint32_t status = 0;
  CHECK_HIP(hipMemcpy(&status, d_status, 4, hipMemcpyDeviceToHost));
  if (status != 0) {
    fprintf(stderr, "device status %u\n", status);
    return 1;
  }

  /* the oracle on the host copies of the same inputs */
  const int64_t rows = oracle_padded_rows(splits, E);
  uint8_t* o_dq = (uint8_t*)calloc(n * rows, 1);
  uint8_t* o_ds = (uint8_t*)calloc(n * rows / 32, 1);
  uint8_t* o_xq = (uint8_t*)calloc(h * rows, 1);
  uint8_t* o_xs = (uint8_t*)calloc(h * rows / 32, 1);
  if (oracle_grouped_quantize(dy, R, n, splits, E, recipe, BSFP8_COLWISE, 1e-30f, NULL, NULL, o_dq, o_ds) ||
      oracle_grouped_quantize(x, R, h, splits, E, recipe, BSFP8_COLWISE, 1e-30f, NULL, NULL, o_xq, o_xs)) {
    fprintf(stderr, "oracle quantize failed\n");
    return 2;
  }
  uint8_t* g_dq = (uint8_t*)malloc(n * rows);
  uint8_t* g_ds = (uint8_t*)malloc(n * rows / 32);
  uint8_t* g_xq = (uint8_t*)malloc(h * rows);
  uint8_t* g_xs = (uint8_t*)malloc(h * rows / 32);
  CHECK_HIP(hipMemcpy(g_dq, d_dq, n * rows, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(g_ds, d_ds, n * rows / 32, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(g_xq, d_xq, h * rows, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(g_xs, d_xs, h * rows / 32, hipMemcpyDeviceToHost));
  if (memcmp(g_dq, o_dq, n * rows) || memcmp(g_ds, o_ds, n * rows / 32)) {
    fprintf(stderr, "dy: quantized bytes or scales differ from the oracle\n");
    ++failures;
  }
  if (memcmp(g_xq, o_xq, h * rows) || memcmp(g_xs, o_xs, h * rows / 32)) {
    fprintf(stderr, "x: quantized bytes or scales differ from the oracle\n");
    ++failures;
  }

  double* ref = (double*)malloc(E * n * h * sizeof(double));
  if (oracle_grouped_wgrad(o_dq, o_ds, n, o_xq, o_xs, h, splits, E, R, recipe, NULL, 0, 0, NULL, ref)) {
    fprintf(stderr, "oracle wgrad failed\n");
    return 2;
  }
  float* got = (float*)malloc(E * n * h * 4);
  CHECK_HIP(hipMemcpy(got, d_out, E * n * h * 4, hipMemcpyDeviceToHost));
  for (int32_t e = 0; e < E; ++e) {
    double num = 0, den = 0;
    for (int64_t i = 0; i < n * h; ++i) {
      const double d = (double)got[e * n * h + i] - ref[e * n * h + i];
      num += d * d;
      den += ref[e * n * h + i] * ref[e * n * h + i];
    }
    const int ok = den == 0 ? num == 0 : sqrt(num / den) <= 1e-5;
    printf("expert %d (%d rows): relative Frobenius error %.3e%s\n", e, splits[e], den == 0 ? sqrt(num) : sqrt(num / den),
           ok ? "" : "  FAIL");
    failures += !ok;
  }
  CHECK_HIP(hipStreamDestroy(stream));
  printf(failures ? "FAIL\n" : "PASS\n");
  return failures ? 1 : 0;
}

// C ABI of libbsfp8: argument validation, buffer-size queries and launches on the caller's
// stream.  Every host-checkable error is reported before any HIP call is made, so these
// checks run (and are tested) on machines without a GPU.  Nothing here allocates, and the
// library holds no mutable state.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/bsfp8.h"
#include "group_layout.hpp"

namespace bsfp8 {
int launch_grouped_quantize(const void* in, int64_t R, int64_t C, const int32_t* splits, int E, int recipe,
                            int which, float zas, uint8_t* row_q, uint8_t* row_s, uint8_t* col_q, void* col_s,
                            const float* noop_flag, uint32_t* status, hipStream_t stream);
int launch_grouped_act_quantize(int act, const void* h, const float* probs, const void* dy, int64_t R, int64_t C,
                                const int32_t* splits, int E, int recipe, int which, uint8_t* row_q, uint8_t* row_s,
                                uint8_t* col_q, void* col_s, uint32_t* status, hipStream_t stream);
int launch_grouped_gemm_wgrad(const uint8_t* dy_q, const void* dy_s, int64_t n, const uint8_t* x_q, const void* x_s,
                              int64_t h, const int32_t* splits, int E, int64_t R, int recipe, float* out,
                              int accumulate, uint32_t* status, hipStream_t stream);
int launch_grouped_gemm_fprop(const uint8_t* x_q, const uint8_t* x_s, int64_t R, int64_t K, const uint8_t* w_q,
                              const uint8_t* w_s, int64_t N, const int32_t* splits, int E, int recipe, void* out,
                              int out_dtype, uint32_t* status, hipStream_t stream);
int launch_grouped_gemm_dgrad(const uint8_t* dy_q, const uint8_t* dy_s, int64_t R, int64_t n, const uint8_t* w_q,
                              const void* w_s, int64_t k, const int32_t* splits, int E, int recipe, void* out,
                              int out_dtype, uint32_t* status, hipStream_t stream);
}  // namespace bsfp8

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }
bool valid_recipe(int r) {
  return r == BSFP8_RECIPE_MX_1X32_E8M0 || r == BSFP8_RECIPE_PER_CHANNEL_128_F32 || r == BSFP8_RECIPE_MXFP4_1X32_E8M0;
}
// recipes with E8M0 block scales (both layouts; the only ones the m-grouped GEMMs take)
bool mx_recipe(int r) { return r == BSFP8_RECIPE_MX_1X32_E8M0 || r == BSFP8_RECIPE_MXFP4_1X32_E8M0; }
// the recipe argument of the GEMM calls: a data recipe, or MXFP8 on the scaled fp8 MFMA
bool wgrad_recipe(int r) { return valid_recipe(r) || r == (BSFP8_RECIPE_MX_1X32_E8M0 | BSFP8_GEMM_FP8_MFMA); }
bool mgrouped_recipe(int r) { return mx_recipe(r) || r == (BSFP8_RECIPE_MX_1X32_E8M0 | BSFP8_GEMM_FP8_MFMA); }
// data elements per byte
int64_t per_byte(int r) { return r == BSFP8_RECIPE_MXFP4_1X32_E8M0 ? 2 : 1; }
bool valid_groups(int32_t e) { return e > 0 && e <= BSFP8_MAX_GROUPS; }
// dims must be positive multiples of 32 and small enough that byte offsets fit in int64
bool valid_dim(int64_t d) { return d > 0 && d % 32 == 0 && d <= (int64_t(1) << 40); }
// The GEMM kernels address a 256-row operand tile with 32-bit offsets: 256 * row length must
// stay below 2^32, i.e. a K extent (k for fprop, a group's padded rows for wgrad) below 2^24.
constexpr int64_t kMaxKExtent = (int64_t(1) << 24) - 128;
// The GEMM epilogues address a 128-row block of the output with 32-bit byte offsets and mark
// lanes past the last column with offsets from 2^31 up: 128 * 4 * (output row length) must stay
// below 2^31.
constexpr int64_t kMaxOutCols = int64_t(1) << 21;

}  // namespace

extern "C" {

int64_t bsfp8_colwise_rows_bound(int64_t capacity_rows, int32_t num_groups) {
  if (capacity_rows < 0 || !valid_groups(num_groups)) return 0;
  return bsfp8::col_rows_bound(capacity_rows, num_groups);
}

size_t bsfp8_colwise_data_bytes(int64_t capacity_rows, int64_t cols, int32_t num_groups, int recipe) {
  if (!valid_dim(cols) || !valid_recipe(recipe)) return 0;
  return (size_t)bsfp8_colwise_rows_bound(capacity_rows, num_groups) * (size_t)(cols / per_byte(recipe));
}

size_t bsfp8_colwise_scale_bytes(int64_t capacity_rows, int64_t cols, int32_t num_groups, int recipe) {
  if (!valid_dim(cols) || !valid_recipe(recipe)) return 0;
  const size_t rows = (size_t)bsfp8_colwise_rows_bound(capacity_rows, num_groups);
  if (mx_recipe(recipe)) return rows / 32 * (size_t)cols;
  return rows / 128 * (size_t)cols * sizeof(float);
}

size_t bsfp8_rowwise_data_bytes(int64_t rows, int64_t cols, int recipe) {
  if (rows < 0 || !valid_dim(cols) || !mx_recipe(recipe)) return 0;
  return (size_t)rows * (size_t)(cols / per_byte(recipe));
}

size_t bsfp8_rowwise_scale_bytes(int64_t rows, int64_t cols) {
  if (rows < 0 || !valid_dim(cols)) return 0;
  return (size_t)rows * (size_t)(cols / 32);
}

int bsfp8_grouped_quantize(const void* in_bf16, int64_t capacity_rows, int64_t cols, const int32_t* split_sizes,
                           int32_t num_groups, int recipe, int which, float zero_amax_scale, uint8_t* row_q,
                           uint8_t* row_s, uint8_t* col_q, void* col_s, const float* noop_flag, uint32_t* status,
                           void* stream) {
  if (!valid_recipe(recipe)) return BSFP8_ERR_RECIPE;
  if (which <= 0 || (which & ~(BSFP8_ROWWISE | BSFP8_COLWISE)) != 0) return BSFP8_ERR_ARGUMENT;
  if ((which & BSFP8_ROWWISE) && !mx_recipe(recipe)) return BSFP8_ERR_LAYOUT;
  if (capacity_rows < 0 || !valid_dim(cols)) return BSFP8_ERR_SHAPE;
  if (recipe == BSFP8_RECIPE_PER_CHANNEL_128_F32 && !(isfinite(zero_amax_scale) && zero_amax_scale >= 0.0f))
    return BSFP8_ERR_ARGUMENT;
  if (split_sizes == nullptr && (which & BSFP8_COLWISE)) return BSFP8_ERR_NULL_POINTER;
  if (split_sizes != nullptr && !valid_groups(num_groups)) return BSFP8_ERR_NUM_GROUPS;
  if (capacity_rows == 0) return BSFP8_OK;  // nothing to read or write
  if (in_bf16 == nullptr) return BSFP8_ERR_NULL_POINTER;
  if ((which & BSFP8_ROWWISE) && (row_q == nullptr || row_s == nullptr)) return BSFP8_ERR_NULL_POINTER;
  if ((which & BSFP8_COLWISE) && (col_q == nullptr || col_s == nullptr)) return BSFP8_ERR_NULL_POINTER;
  if (!aligned16(in_bf16) || !aligned4(split_sizes) || !aligned4(noop_flag) || !aligned4(status))
    return BSFP8_ERR_ALIGNMENT;
  if ((which & BSFP8_ROWWISE) && (!aligned16(row_q) || !aligned16(row_s))) return BSFP8_ERR_ALIGNMENT;
  if ((which & BSFP8_COLWISE) && (!aligned16(col_q) || !aligned16(col_s))) return BSFP8_ERR_ALIGNMENT;
  return bsfp8::launch_grouped_quantize(in_bf16, capacity_rows, cols, split_sizes, split_sizes ? num_groups : 0,
                                        recipe, which, zero_amax_scale, (which & BSFP8_ROWWISE) ? row_q : nullptr,
                                        (which & BSFP8_ROWWISE) ? row_s : nullptr,
                                        (which & BSFP8_COLWISE) ? col_q : nullptr,
                                        (which & BSFP8_COLWISE) ? col_s : nullptr, noop_flag, status,
                                        (hipStream_t)stream);
}

int bsfp8_grouped_act_quantize(int activation, const void* h_bf16, const float* probs, const void* dy_bf16,
                               int64_t capacity_rows, int64_t cols, const int32_t* split_sizes, int32_t num_groups,
                               int recipe, int which, uint8_t* row_q, uint8_t* row_s, uint8_t* col_q, void* col_s,
                               uint32_t* status, void* stream) {
  if (activation < BSFP8_ACT_SRELU || activation > BSFP8_ACT_SWIGLU_GRAD) return BSFP8_ERR_ARGUMENT;
  const bool grad = activation == BSFP8_ACT_SRELU_GRAD || activation == BSFP8_ACT_SWIGLU_GRAD;
  if (!valid_recipe(recipe)) return BSFP8_ERR_RECIPE;
  if (!mx_recipe(recipe)) return BSFP8_ERR_LAYOUT;
  if (which <= 0 || (which & ~(BSFP8_ROWWISE | BSFP8_COLWISE)) != 0) return BSFP8_ERR_ARGUMENT;
  if (capacity_rows < 0 || !valid_dim(cols)) return BSFP8_ERR_SHAPE;
  if (split_sizes == nullptr) return BSFP8_ERR_NULL_POINTER;
  if (!valid_groups(num_groups)) return BSFP8_ERR_NUM_GROUPS;
  if (capacity_rows == 0) return BSFP8_OK;  // nothing to read or write
  if (h_bf16 == nullptr || (grad && dy_bf16 == nullptr)) return BSFP8_ERR_NULL_POINTER;
  if ((which & BSFP8_ROWWISE) && (row_q == nullptr || row_s == nullptr)) return BSFP8_ERR_NULL_POINTER;
  if ((which & BSFP8_COLWISE) && (col_q == nullptr || col_s == nullptr)) return BSFP8_ERR_NULL_POINTER;
  if (!aligned16(h_bf16) || !aligned16(dy_bf16) || !aligned4(probs) || !aligned4(split_sizes) || !aligned4(status))
    return BSFP8_ERR_ALIGNMENT;
  if ((which & BSFP8_ROWWISE) && (!aligned16(row_q) || !aligned16(row_s))) return BSFP8_ERR_ALIGNMENT;
  if ((which & BSFP8_COLWISE) && (!aligned16(col_q) || !aligned16(col_s))) return BSFP8_ERR_ALIGNMENT;
  return bsfp8::launch_grouped_act_quantize(activation, h_bf16, probs, grad ? dy_bf16 : nullptr, capacity_rows,
                                            cols, split_sizes, num_groups, recipe, which,
                                            (which & BSFP8_ROWWISE) ? row_q : nullptr,
                                            (which & BSFP8_ROWWISE) ? row_s : nullptr,
                                            (which & BSFP8_COLWISE) ? col_q : nullptr,
                                            (which & BSFP8_COLWISE) ? col_s : nullptr, status, (hipStream_t)stream);
}

int bsfp8_grouped_gemm_wgrad(const uint8_t* dy_col_q, const void* dy_col_s, int64_t n, const uint8_t* x_col_q,
                             const void* x_col_s, int64_t h, const int32_t* split_sizes, int32_t num_groups,
                             int64_t capacity_rows, int recipe, float* out, int accumulate, uint32_t* status,
                             void* stream) {
  if (!wgrad_recipe(recipe)) return BSFP8_ERR_RECIPE;
  if (!valid_groups(num_groups)) return BSFP8_ERR_NUM_GROUPS;
  if (!valid_dim(n) || !valid_dim(h) || capacity_rows < 0) return BSFP8_ERR_SHAPE;
  if (capacity_rows + 127 > kMaxKExtent || h > kMaxOutCols) return BSFP8_ERR_SHAPE;
  if (accumulate != 0 && accumulate != 1) return BSFP8_ERR_ARGUMENT;
  if (split_sizes == nullptr || out == nullptr) return BSFP8_ERR_NULL_POINTER;
  // the operands are read only when some group is non-empty, which needs capacity_rows > 0
  if (capacity_rows > 0 && (dy_col_q == nullptr || dy_col_s == nullptr || x_col_q == nullptr || x_col_s == nullptr))
    return BSFP8_ERR_NULL_POINTER;
  if (!aligned16(dy_col_q) || !aligned16(x_col_q) || !aligned16(dy_col_s) || !aligned16(x_col_s) ||
      !aligned16(out) || !aligned4(split_sizes) || !aligned4(status))
    return BSFP8_ERR_ALIGNMENT;
  return bsfp8::launch_grouped_gemm_wgrad(dy_col_q, dy_col_s, n, x_col_q, x_col_s, h, split_sizes, num_groups,
                                          capacity_rows, recipe, out, accumulate, status, (hipStream_t)stream);
}

int bsfp8_grouped_gemm_fprop(const uint8_t* x_row_q, const uint8_t* x_row_s, int64_t capacity_rows, int64_t k,
                             const uint8_t* w_q, const uint8_t* w_s, int64_t n, const int32_t* split_sizes,
                             int32_t num_groups, int recipe, void* out, int out_dtype, uint32_t* status,
                             void* stream) {
  if (!mgrouped_recipe(recipe)) return BSFP8_ERR_RECIPE;
  if (!valid_groups(num_groups)) return BSFP8_ERR_NUM_GROUPS;
  if (!valid_dim(k) || !valid_dim(n) || capacity_rows < 0 || k > kMaxKExtent || n > kMaxOutCols)
    return BSFP8_ERR_SHAPE;
  if (out_dtype != BSFP8_OUT_F32 && out_dtype != BSFP8_OUT_BF16) return BSFP8_ERR_ARGUMENT;
  if (capacity_rows == 0) return BSFP8_OK;  // zero-row early return: nothing is dereferenced
  if (x_row_q == nullptr || x_row_s == nullptr || w_q == nullptr || w_s == nullptr || split_sizes == nullptr ||
      out == nullptr)
    return BSFP8_ERR_NULL_POINTER;
  if (!aligned16(x_row_q) || !aligned16(x_row_s) || !aligned16(w_q) || !aligned16(w_s) || !aligned16(out) ||
      !aligned4(split_sizes) || !aligned4(status))
    return BSFP8_ERR_ALIGNMENT;
  return bsfp8::launch_grouped_gemm_fprop(x_row_q, x_row_s, capacity_rows, k, w_q, w_s, n, split_sizes, num_groups,
                                          recipe, out, out_dtype, status, (hipStream_t)stream);
}

int bsfp8_grouped_gemm_dgrad(const uint8_t* dy_row_q, const uint8_t* dy_row_s, int64_t capacity_rows, int64_t n,
                             const uint8_t* w_col_q, const void* w_col_s, int64_t k, const int32_t* split_sizes,
                             int32_t num_groups, int recipe, void* out, int out_dtype, uint32_t* status,
                             void* stream) {
  if (!mgrouped_recipe(recipe)) return BSFP8_ERR_RECIPE;
  if (!valid_groups(num_groups)) return BSFP8_ERR_NUM_GROUPS;
  // the weight rows are n rounded up to 128: that padded length bounds the 32-bit tile offsets
  if (!valid_dim(n) || !valid_dim(k) || capacity_rows < 0 || n + 127 > kMaxKExtent || k > kMaxOutCols)
    return BSFP8_ERR_SHAPE;
  if (out_dtype != BSFP8_OUT_F32 && out_dtype != BSFP8_OUT_BF16) return BSFP8_ERR_ARGUMENT;
  if (capacity_rows == 0) return BSFP8_OK;  // zero-row early return: nothing is dereferenced
  if (dy_row_q == nullptr || dy_row_s == nullptr || w_col_q == nullptr || w_col_s == nullptr ||
      split_sizes == nullptr || out == nullptr)
    return BSFP8_ERR_NULL_POINTER;
  if (!aligned16(dy_row_q) || !aligned16(dy_row_s) || !aligned16(w_col_q) || !aligned16(w_col_s) || !aligned16(out) ||
      !aligned4(split_sizes) || !aligned4(status))
    return BSFP8_ERR_ALIGNMENT;
  return bsfp8::launch_grouped_gemm_dgrad(dy_row_q, dy_row_s, capacity_rows, n, w_col_q, w_col_s, k, split_sizes,
                                          num_groups, recipe, out, out_dtype, status, (hipStream_t)stream);
}

const char* bsfp8_strerror(int code) {
  switch (code) {
    case BSFP8_OK: return "success";
    case BSFP8_ERR_NULL_POINTER: return "a required pointer is NULL";
    case BSFP8_ERR_NUM_GROUPS: return "num_groups must be in [1, 1024]";
    case BSFP8_ERR_RECIPE: return "unknown recipe";
    case BSFP8_ERR_SHAPE: return "a dimension is negative, not a multiple of 32, or too large";
    case BSFP8_ERR_ALIGNMENT: return "a pointer is not 16-byte aligned";
    case BSFP8_ERR_LAYOUT: return "rowwise layout needs an MX 1x32 E8M0 recipe (MXFP8 or MXFP4)";
    case BSFP8_ERR_ARGUMENT: return "invalid argument";
    case BSFP8_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown error code";
  }
}

}  // extern "C"

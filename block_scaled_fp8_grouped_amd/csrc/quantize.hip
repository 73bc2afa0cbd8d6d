// Grouped quantize: bf16 -> e4m3 with MXFP8 1x32 E8M0 scales or per-channel 128-row fp32
// scales (DeepGEMM #365 reproducer: per-channel cast and K-major pack; TE #3484: MXFP8 block
// scaling over a padded token buffer; TE PR #3224: columnwise scales strided per group member),
// or bf16 -> e2m1 with MXFP4 1x32 E8M0 scales (TE #3484 additional context: the same gated
// grouped paths take a 4-bit block-scaled quantizer), two codes per byte along the contiguous
// axis.
//
// One workgroup (4 waves) walks 8 consecutive 128-row tiles of one 128-channel column: the
// split sizes are scanned once for the first tile and later tiles step forward through the
// groups; each tile is read once from HBM (16-byte loads, 256 contiguous bytes per row) into
// registers while the previous tile is being quantized, then staged in LDS; then
//   colwise: wave w takes tokens [32w, 32w + 32) of the tile and lane l the channel pair
//            (2l, 2l+1): one LDS dword per token, conflict-free, the block amax, the scale and
//            32 codes per channel, written as 32 contiguous bytes of the channel's K-major run;
//   rowwise: 4 lanes per 32-channel block of a row, amax by two lane exchanges, 8 codes per
//            lane; the tile's row scales are staged in LDS and written 128 rows at a time.
// Rows past the group's live rows are never read: they enter LDS as zeros, which leaves every
// block amax unchanged and makes the packed pad lanes 0x00.  Tiles are placed by the
// in-kernel scan of the split sizes (the grid is an upper bound; spare workgroups exit).
//
// With an activation fused in front (fc1's output -> activation -> quantize), each thread
// evaluates the activation once per element from the registers its loads landed in and stages
// the fp32 values in LDS (64 KB: two workgroups per CU); both layouts quantize those values.
// The GLU gradient's tile pairs 64 da columns with the 64 db columns of the same inputs, so one
// sigmoid serves both outputs.
#include <type_traits>

#include "common.hpp"
#include "group_layout.hpp"

namespace bsfp8 {

constexpr int kQThreads = 256;
constexpr int kQRows = 128;
constexpr int kQCols = 128;
constexpr int kQTilesPerWG = 8;  // most consecutive 128-row tiles one workgroup walks
// Tiles per workgroup for a launch of `tiles` 128 x 128 tiles: up to kQTilesPerWG on large
// inputs (one group scan and one prologue per run of tiles), fewer on small ones so that the
// launch still spreads over the chip (at least ~1024 workgroups when the input has them).
static inline int quantize_tiles_per_wg(int64_t tiles) {
  const int64_t t = tiles / 1024;
  return (int)(t < 1 ? 1 : t > kQTilesPerWG ? kQTilesPerWG : t);
}

// Where one 128-row tile of the token buffer lives.
struct QTile {
  int64_t row0;  // first token row
  int64_t jblk;  // 128-row block index inside its group
  int64_t p, kp; // the group's packed offset and padded length (colwise layout)
  int nlive;     // live rows of the tile (<= 128)
};

// Inputs of the activation fused in front of the quantizer (ACT != 0): the routing probability of
// each token row (NULL: 1), for the gradients the incoming bf16 gradient, and for the GLU
// activations their width F (fc1's output row holds a = [0, F) and b = [F, 2F)).
struct ActArgs {
  const float* probs;
  const uint16_t* dy;
  int64_t glu_f;
};

// 2^x in fp32 by a stated algorithm every IEEE fp32 machine reproduces bit for bit: x clamped to
// [-126, 126]; k = floor(x + 1/2), r = x - k (exact); the degree-7 Taylor polynomial of
// exp(r ln 2) (coefficients (ln 2)^n / n! in fp32, Horner order, no fused multiply-add) times 2^k.
__device__ __forceinline__ float exp2_stated(float x) {
  x = x > 126.0f ? 126.0f : (x < -126.0f ? -126.0f : x);
  const float kf = floorf(x + 0.5f);  // an integer in [-126, 126]: exact as fp32 and as int
  const int k = (int)kf;
  const float r = x - kf;
  float poly = 1.52527338e-05f;
  poly = poly * r + 0.000154035304f;
  poly = poly * r + 0.00133335581f;
  poly = poly * r + 0.00961812911f;
  poly = poly * r + 0.0555041087f;
  poly = poly * r + 0.240226507f;
  poly = poly * r + 0.693147182f;
  poly = poly * r + 1.0f;
  return ldexpf(poly, k);
}

// The activations between fc1 and fc2 (TE #3484: fc1 -> ScaledSReLU / ScaledSwiGLU -> fc2 with
// per-token probs), in fp32, each operation rounded in the order written:
//   ACT 1: r = max(h, 0) (+0 for h <= 0);  y = (r * r) * p
//   ACT 2: its gradient                     g = ((2 * r) * p) * dy
//   ACT 3: sg = 1 / (1 + 2^(-a log2 e)), s = a * sg;  y = (s * b) * p
// (the division correctly rounded: recip_rn equals it on the [1, 2^126] that 1 + 2^x spans here)
template <int ACT>
__device__ __forceinline__ float act_value(float h, float b, float p, float d) {
  if constexpr (ACT <= 2) {
    const float r = h > 0.0f ? h : 0.0f;
    if constexpr (ACT == 1) {
      const float r2 = r * r;
      return r2 * p;
    } else {
      const float tp = (2.0f * r) * p;
      return tp * d;
    }
  } else {
    const float t = exp2_stated(-h * 1.44269502f);
    const float den = 1.0f + t;  // in [1, 2^126]: t <= 2^126 after the clamp
    const float sg = recip_rn(den);
    const float sl = h * sg;
    const float sb = sl * b;
    return sb * p;
  }
}

//   ACT 4: the gradient of ACT 3, q = dy * p:  da = (q * b) * (sg * (1 + a * (1 - sg))),  db = q * s
// (sg and s shared by the two outputs of one element)
__device__ __forceinline__ void glu_grad(float a, float b, float p, float d, float& da, float& db) {
  const float t = exp2_stated(-a * 1.44269502f);
  const float den = 1.0f + t;  // in [1, 2^126]
  const float sg = recip_rn(den);
  const float sl = a * sg;
  const float q = d * p;
  db = q * sl;
  const float u = 1.0f - sg;
  const float v = a * u;
  const float w = 1.0f + v;
  const float ds = sg * w;
  const float qb = q * b;
  da = qb * ds;
}

template <int RECIPE, bool ROW, bool COL, int ACT = 0>
__global__ __launch_bounds__(kQThreads) void grouped_quantize_kernel(
    const uint16_t* __restrict__ in, int64_t R, int64_t C, const int32_t* __restrict__ splits, int E,
    float zero_amax_scale, uint8_t* __restrict__ row_q, uint8_t* __restrict__ row_s,
    uint8_t* __restrict__ col_q, void* __restrict__ col_s, const float* noop_flag, uint32_t* status,
    ActArgs act, int tpw) {
  static_assert(ACT == 0 || RECIPE != BSFP8_RECIPE_PER_CHANNEL_128_F32, "the fused activation takes MX recipes");
  // a set flag turns the whole call into a no-op: the outputs (and the status word) keep what
  // they hold, which lets a captured graph skip re-quantizing a cached weight
  if (noop_flag != nullptr && *noop_flag != 0.0f) return;
  __shared__ GroupScanSmem<kQThreads> gsm;
  // the tile: bf16 pairs, or with an activation its fp32 values (evaluated once per element)
  __shared__ __attribute__((aligned(16))) uint32_t tile[ACT == 0 ? kQRows : 1][kQCols / 2];
  __shared__ __attribute__((aligned(16))) float ytile[ACT != 0 ? kQRows : 1][ACT != 0 ? kQCols : 1];
  __shared__ float pc_amax[4][kQCols];
  __shared__ uint8_t rs_tile[kQCols / 32][kQRows];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  // workgroup -> (run of tpw row tiles, 128-channel tile), channel tiles fastest: the
  // workgroups in flight together read neighbouring pieces of the same rows
  const int64_t ctiles = (C + kQCols - 1) / kQCols;
  const int64_t rt0 = (int64_t)blockIdx.x / ctiles * tpw, ctile = (int64_t)blockIdx.x % ctiles;
  const int64_t c0 = ctile * kQCols;
  const int ncols = (int)((C - c0) < kQCols ? (C - c0) : kQCols);  // a multiple of 32
  // The GLU gradient pairs its outputs: tile columns [0, 64) are da at input columns
  // [c0h, c0h + gw) and [64, 128) db at the same input columns, so one evaluation of the sigmoid
  // serves both (C = 2F; gw, a multiple of 32, is the tile's live width of each half).
  constexpr int kHalf = kQCols / 2;
  const int64_t c0h = ctile * kHalf;
  const int gw = ACT == 4 ? (int)((act.glu_f - c0h) < kHalf ? (act.glu_f - c0h) : kHalf) : 0;
  auto out_col = [&](int lc) -> int64_t {  // output column of tile column lc
    if constexpr (ACT == 4) return (lc < kHalf ? c0h : act.glu_f + c0h - kHalf) + lc;
    return c0 + lc;
  };
  auto live_col = [&](int lc) -> bool {  // lc a multiple of 2 (colwise) or 8 (rowwise)
    if constexpr (ACT == 4) return (lc & (kHalf - 1)) < gw;
    return lc < ncols;
  };

  // group of the run's first tile from the scan of the split sizes; later tiles walk forward
  GroupInfo g{};
  if (splits != nullptr) {
    const uint32_t flags = group_scan<kQThreads>(splits, E, R, kQRows, rt0, 0, gsm, g);
    report_status(status, flags);
    if (g.e < 0) return;
  }
  auto place = [&](int64_t rt, QTile& q) -> bool {
    if (splits == nullptr) {
      q.row0 = rt * kQRows;
      if (q.row0 >= R) return false;
      q.nlive = (int)(R - q.row0 < kQRows ? R - q.row0 : kQRows);
      q.jblk = q.p = q.kp = 0;
      return true;
    }
    while (rt >= g.tile + (g.k + kQRows - 1) / kQRows) {  // past this group (or it is empty)
      g.tile += (g.k + kQRows - 1) / kQRows;
      g.off += g.k;
      g.p += g.kp;
      if (++g.e >= E) return false;
      g.k = splits[g.e];  // validated by the scan: 0 <= k, sum <= capacity
      g.kp = col_padded_rows(g.k);
    }
    q.jblk = rt - g.tile;
    q.row0 = g.off + kQRows * q.jblk;
    const int64_t left = g.k - kQRows * q.jblk;
    q.nlive = (int)(left < kQRows ? left : kQRows);
    q.p = g.p;
    q.kp = g.kp;
    return true;
  };

  // this thread's share of a tile: 16 lanes per row, 8 channels (16 bytes) each (the GLU
  // gradient: 8 lanes per row, 8 input columns of a, b and dy each)
  constexpr int kLanesPerRow = ACT == 4 ? 8 : 16;
  constexpr int kPasses = kQRows * kLanesPerRow / kQThreads;
  v4i pre[kPasses];
  v4i pre2[ACT >= 2 ? kPasses : 1];  // dy (ACT 2) or b (ACT 3, 4)
  v4i pre3[ACT == 4 ? kPasses : 1];  // dy of the GLU gradient
  float pre_p[ACT != 0 ? kPasses : 1];
  auto load_tile = [&](const QTile& q) {
#pragma unroll
    for (int pass = 0; pass < kPasses; ++pass) {
      const int r = pass * (kQThreads / kLanesPerRow) + tid / kLanesPerRow;
      const int ch = tid % kLanesPerRow;
      pre[pass] = v4i{0, 0, 0, 0};
      if constexpr (ACT >= 2) pre2[pass] = v4i{0, 0, 0, 0};
      if constexpr (ACT == 4) pre3[pass] = v4i{0, 0, 0, 0};
      if constexpr (ACT != 0) pre_p[pass] = 0.0f;
      if (r < q.nlive && live_col(ch * 8)) {
        if constexpr (ACT <= 2) {
          pre[pass] = *(const v4i*)(in + (q.row0 + r) * C + c0 + ch * 8);
          if constexpr (ACT == 2) pre2[pass] = *(const v4i*)(act.dy + (q.row0 + r) * C + c0 + ch * 8);
        } else {
          // a and b at input column j of the two halves of the [2F] row
          const int64_t F = act.glu_f, j = (ACT == 4 ? c0h : c0) + ch * 8;
          const uint16_t* hr = in + (q.row0 + r) * 2 * F;
          pre[pass] = *(const v4i*)(hr + j);
          pre2[pass] = *(const v4i*)(hr + F + j);
          if constexpr (ACT == 4) pre3[pass] = *(const v4i*)(act.dy + (q.row0 + r) * F + j);
        }
        if constexpr (ACT != 0) pre_p[pass] = act.probs != nullptr ? act.probs[q.row0 + r] : 1.0f;
      }
    }
  };
  // with an activation: its fp32 values into the LDS tile, once per element (rows and columns
  // past the live ones hold zero inputs and p = 0, which give +0)
  auto commit_act = [&]() {
#pragma unroll
    for (int pass = 0; pass < kPasses; ++pass) {
      const int r = pass * (kQThreads / kLanesPerRow) + tid / kLanesPerRow;
      const int ch = tid % kLanesPerRow;
      const float p = pre_p[pass];
      float y[8], z[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t hw = (uint32_t)pre[pass][i];
        const uint32_t w2 = ACT >= 2 ? (uint32_t)pre2[pass][i] : 0u;
        if constexpr (ACT == 4) {
          const uint32_t w3 = (uint32_t)pre3[pass][i];
          glu_grad(bf16_lo(hw), bf16_lo(w2), p, bf16_lo(w3), y[2 * i], z[2 * i]);
          glu_grad(bf16_hi(hw), bf16_hi(w2), p, bf16_hi(w3), y[2 * i + 1], z[2 * i + 1]);
        } else {
          // ACT 2 takes w2 as its dy, ACT 3 as b
          y[2 * i] = act_value<ACT>(bf16_lo(hw), bf16_lo(w2), p, bf16_lo(w2));
          y[2 * i + 1] = act_value<ACT>(bf16_hi(hw), bf16_hi(w2), p, bf16_hi(w2));
        }
      }
      *(float4*)&ytile[r][ch * 8] = make_float4(y[0], y[1], y[2], y[3]);
      *(float4*)&ytile[r][ch * 8 + 4] = make_float4(y[4], y[5], y[6], y[7]);
      if constexpr (ACT == 4) {
        *(float4*)&ytile[r][kHalf + ch * 8] = make_float4(z[0], z[1], z[2], z[3]);
        *(float4*)&ytile[r][kHalf + ch * 8 + 4] = make_float4(z[4], z[5], z[6], z[7]);
      }
    }
  };

  QTile cur;
  if (!place(rt0, cur)) return;
  load_tile(cur);
  for (int t = 0; t < tpw; ++t) {
    if constexpr (ACT != 0) {
      commit_act();
    } else {
#pragma unroll
      for (int pass = 0; pass < kPasses; ++pass) *(v4i*)&tile[pass * 16 + (tid >> 4)][(tid & 15) * 4] = pre[pass];
    }
    __syncthreads();
    // the next tile's loads are in flight while this one is quantized
    QTile nxt;
    const bool more = t + 1 < tpw && place(rt0 + t + 1, nxt);
    if (more) load_tile(nxt);
    const int64_t row0 = cur.row0, P = cur.p, kp = cur.kp, jblk = cur.jblk;
    const int nlive = cur.nlive;

    if constexpr (COL && ACT != 0) {
      // ---- colwise with the activation: the same split, on the fp32 activation values ----
      constexpr bool F4 = RECIPE == BSFP8_RECIPE_MXFP4_1X32_E8M0;
      const int c = 2 * lane;
      float y0[32], y1[32];
      uint32_t m0 = 0, m1 = 0;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const float2 yy = *(const float2*)&ytile[wave * 32 + i][c];
        y0[i] = yy.x;
        y1[i] = yy.y;
        m0 = max(m0, __float_as_uint(y0[i]) & 0x7fffffffu);
        m1 = max(m1, __float_as_uint(y1[i]) & 0x7fffffffu);
      }
      const int e0 = F4 ? e8m0_exponent_fp4(__uint_as_float(m0)) : e8m0_exponent(__uint_as_float(m0));
      const int e1 = F4 ? e8m0_exponent_fp4(__uint_as_float(m1)) : e8m0_exponent(__uint_as_float(m1));
      const float s0 = exp2_neg(e0), s1 = exp2_neg(e1);
      const uint32_t sbits = (uint32_t)(e0 + 127) | ((uint32_t)(e1 + 127) << 8);
      if (live_col(c)) {
        const int64_t oc = out_col(c);
        if constexpr (F4) {
          v4i q0, q1;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float* a = y0 + 8 * i;
            const float* b = y1 + 8 * i;
            q0[i] = (int)e2m1x8(a[0] * s0, a[1] * s0, a[2] * s0, a[3] * s0, a[4] * s0, a[5] * s0, a[6] * s0, a[7] * s0);
            q1[i] = (int)e2m1x8(b[0] * s1, b[1] * s1, b[2] * s1, b[3] * s1, b[4] * s1, b[5] * s1, b[6] * s1, b[7] * s1);
          }
          uint8_t* dst = col_q + col_elem(C, P, kp, oc, kQRows * jblk + 32 * wave) / 2;
          *(v4i*)dst = q0;
          *(v4i*)(dst + kp / 2) = q1;
        } else {
          v4i q0[2], q1[2];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            q0[i >> 2][i & 3] = (int)e4m3x4(y0[4 * i] * s0, y0[4 * i + 1] * s0, y0[4 * i + 2] * s0, y0[4 * i + 3] * s0);
            q1[i >> 2][i & 3] = (int)e4m3x4(y1[4 * i] * s1, y1[4 * i + 1] * s1, y1[4 * i + 2] * s1, y1[4 * i + 3] * s1);
          }
          uint8_t* dst = col_q + col_elem(C, P, kp, oc, kQRows * jblk + 32 * wave);
          *(v4i*)dst = q0[0];
          *(v4i*)(dst + 16) = q0[1];
          *(v4i*)(dst + kp) = q1[0];
          *(v4i*)(dst + kp + 16) = q1[1];
        }
        *(uint16_t*)((uint8_t*)col_s + col_e8m0(C, P, 4 * jblk + wave, oc)) = (uint16_t)sbits;
      }
    } else if constexpr (COL) {
      // ---- colwise: wave -> 32 tokens, lane -> channel pair ----
      const int c = 2 * lane;
      uint32_t w[32];
      uint32_t m0 = 0, m1 = 0;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        w[i] = tile[wave * 32 + i][lane];
        m0 = max(m0, w[i] & 0x7fffu);
        m1 = max(m1, (w[i] >> 16) & 0x7fffu);
      }
      float s0, s1;
      uint32_t sbits = 0;
      if constexpr (RECIPE != BSFP8_RECIPE_PER_CHANNEL_128_F32) {
        constexpr bool F4 = RECIPE == BSFP8_RECIPE_MXFP4_1X32_E8M0;
        const float a0 = __uint_as_float(m0 << 16), a1 = __uint_as_float(m1 << 16);
        const int e0 = F4 ? e8m0_exponent_fp4(a0) : e8m0_exponent(a0);
        const int e1 = F4 ? e8m0_exponent_fp4(a1) : e8m0_exponent(a1);
        s0 = exp2_neg(e0);
        s1 = exp2_neg(e1);
        sbits = (uint32_t)(e0 + 127) | ((uint32_t)(e1 + 127) << 8);
      } else {
        pc_amax[wave][c] = __uint_as_float(m0 << 16);
        pc_amax[wave][c + 1] = __uint_as_float(m1 << 16);
        __syncthreads();
        float a0 = pc_amax[0][c], a1 = pc_amax[0][c + 1];
#pragma unroll
        for (int q = 1; q < 4; ++q) {
          a0 = fmaxf(a0, pc_amax[q][c]);
          a1 = fmaxf(a1, pc_amax[q][c + 1]);
        }
        float sf0 = a0 / 448.0f, sf1 = a1 / 448.0f;
        if (sf0 == 0.0f) sf0 = zero_amax_scale;
        if (sf1 == 0.0f) sf1 = zero_amax_scale;
        if (sf0 < 1e-30f) sf0 = 1e-30f;
        if (sf1 < 1e-30f) sf1 = 1e-30f;
        s0 = 1.0f / sf0;
        s1 = 1.0f / sf1;
        if (wave == 0 && c0 + c < C) {
          float2 sv;
          sv.x = sf0;
          sv.y = sf1;
          *(float2*)((float*)col_s + col_pc_scale(C, P, jblk, c0 + c)) = sv;
        }
      }
      if constexpr (RECIPE == BSFP8_RECIPE_MXFP4_1X32_E8M0) {
        // 32 tokens of each channel -> 16 bytes, token 2j in the low nibble of byte j
        v4i q0, q1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t* wi = w + 8 * i;
          q0[i] = (int)e2m1x8(bf16_lo(wi[0]) * s0, bf16_lo(wi[1]) * s0, bf16_lo(wi[2]) * s0, bf16_lo(wi[3]) * s0,
                              bf16_lo(wi[4]) * s0, bf16_lo(wi[5]) * s0, bf16_lo(wi[6]) * s0, bf16_lo(wi[7]) * s0);
          q1[i] = (int)e2m1x8(bf16_hi(wi[0]) * s1, bf16_hi(wi[1]) * s1, bf16_hi(wi[2]) * s1, bf16_hi(wi[3]) * s1,
                              bf16_hi(wi[4]) * s1, bf16_hi(wi[5]) * s1, bf16_hi(wi[6]) * s1, bf16_hi(wi[7]) * s1);
        }
        if (c0 + c < C) {
          uint8_t* dst = col_q + col_elem(C, P, kp, c0 + c, kQRows * jblk + 32 * wave) / 2;
          *(v4i*)dst = q0;
          *(v4i*)(dst + kp / 2) = q1;
          *(uint16_t*)((uint8_t*)col_s + col_e8m0(C, P, 4 * jblk + wave, c0 + c)) = (uint16_t)sbits;
        }
      } else {
        v4i q0[2], q1[2];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t lo = e4m3x4(bf16_lo(w[4 * i]) * s0, bf16_lo(w[4 * i + 1]) * s0, bf16_lo(w[4 * i + 2]) * s0,
                                     bf16_lo(w[4 * i + 3]) * s0);
          const uint32_t hi = e4m3x4(bf16_hi(w[4 * i]) * s1, bf16_hi(w[4 * i + 1]) * s1, bf16_hi(w[4 * i + 2]) * s1,
                                     bf16_hi(w[4 * i + 3]) * s1);
          q0[i >> 2][i & 3] = (int)lo;
          q1[i >> 2][i & 3] = (int)hi;
        }
        if (c0 + c < C) {
          uint8_t* dst = col_q + col_elem(C, P, kp, c0 + c, kQRows * jblk + 32 * wave);
          *(v4i*)dst = q0[0];
          *(v4i*)(dst + 16) = q0[1];
          *(v4i*)(dst + kp) = q1[0];
          *(v4i*)(dst + kp + 16) = q1[1];
          if constexpr (RECIPE == BSFP8_RECIPE_MX_1X32_E8M0) {
            *(uint16_t*)((uint8_t*)col_s + col_e8m0(C, P, 4 * jblk + wave, c0 + c)) = (uint16_t)sbits;
          }
        }
      }
    }

    if constexpr (ROW) {
      // ---- rowwise: 16 lanes per row (8 channels each), 4 lanes per 32-channel block ----
#pragma unroll
      for (int pass = 0; pass < kQRows / 16; ++pass) {
        const int r = pass * 16 + (tid >> 4);
        const int ch = tid & 15;
        uint32_t m = 0;
        float yv[8];  // the values this lane quantizes (bf16 inputs, or the activation's fp32 values)
        if constexpr (ACT != 0) {
          const float4 ya = *(const float4*)&ytile[r][ch * 8], yb = *(const float4*)&ytile[r][ch * 8 + 4];
          yv[0] = ya.x, yv[1] = ya.y, yv[2] = ya.z, yv[3] = ya.w;
          yv[4] = yb.x, yv[5] = yb.y, yv[6] = yb.z, yv[7] = yb.w;
#pragma unroll
          for (int i = 0; i < 8; ++i) m = max(m, __float_as_uint(yv[i]) & 0x7fffffffu);
        } else {
          const v4i v = *(const v4i*)&tile[r][ch * 4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            yv[2 * i] = bf16_lo((uint32_t)v[i]);
            yv[2 * i + 1] = bf16_hi((uint32_t)v[i]);
            m = max(m, max((uint32_t)v[i] & 0x7fffu, ((uint32_t)v[i] >> 16) & 0x7fffu));
          }
          m <<= 16;  // the bf16 magnitude's fp32 bits
        }
        m = max(m, (uint32_t)__shfl_xor((int)m, 1, 64));
        m = max(m, (uint32_t)__shfl_xor((int)m, 2, 64));
        const float amax = __uint_as_float(m);
        const int e = RECIPE == BSFP8_RECIPE_MXFP4_1X32_E8M0 ? e8m0_exponent_fp4(amax) : e8m0_exponent(amax);
        const float s = exp2_neg(e);
        if (r < nlive && live_col(ch * 8)) {
          if constexpr (RECIPE == BSFP8_RECIPE_MXFP4_1X32_E8M0) {  // 8 codes -> 4 bytes
            *(uint32_t*)(row_q + ((row0 + r) * C + out_col(ch * 8)) / 2) = e2m1x8(
                yv[0] * s, yv[1] * s, yv[2] * s, yv[3] * s, yv[4] * s, yv[5] * s, yv[6] * s, yv[7] * s);
          } else {
            v2i q;
            q[0] = (int)e4m3x4(yv[0] * s, yv[1] * s, yv[2] * s, yv[3] * s);
            q[1] = (int)e4m3x4(yv[4] * s, yv[5] * s, yv[6] * s, yv[7] * s);
            *(v2i*)(row_q + (row0 + r) * C + out_col(ch * 8)) = q;
          }
        }
        if ((ch & 3) == 0) rs_tile[ch >> 2][r] = (uint8_t)(e + 127);
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < (kQCols / 32) * kQRows / kQThreads; ++i) {
        const int idx = tid + i * kQThreads;
        const int b = idx / kQRows, r = idx % kQRows;
        if (r < nlive && live_col(b * 32)) row_s[(out_col(b * 32) / 32) * R + row0 + r] = rs_tile[b][r];
      }
    }
    __syncthreads();  // the LDS tile and row scales are free for the next tile
    if (!more) break;
    cur = nxt;
  }
}

// Upper bound of the number of 128-row tiles over all groups: sum ceil(k_e / 128) <=
// floor((R + 127 E) / 128) for any valid sizes.
static inline int64_t quantize_row_tiles(int64_t R, int E, bool grouped) {
  return grouped ? (R + 127 * (int64_t)E) / kQRows : (R + kQRows - 1) / kQRows;
}

int launch_grouped_quantize(const void* in, int64_t R, int64_t C, const int32_t* splits, int E, int recipe,
                            int which, float zas, uint8_t* row_q, uint8_t* row_s, uint8_t* col_q, void* col_s,
                            const float* noop_flag, uint32_t* status, hipStream_t stream) {
  const int64_t rtiles = quantize_row_tiles(R, E, splits != nullptr), gy = (C + kQCols - 1) / kQCols;
  const int tpw = quantize_tiles_per_wg(rtiles * gy);
  const int64_t gx = (rtiles + tpw - 1) / tpw;
  if (gx <= 0 || gy <= 0) return BSFP8_OK;
  if (gx * gy > 0x7fffffff) return BSFP8_ERR_SHAPE;
  dim3 grid((unsigned)(gx * gy)), block(kQThreads);
  const uint16_t* x = (const uint16_t*)in;
  const bool row = (which & BSFP8_ROWWISE) != 0, col = (which & BSFP8_COLWISE) != 0;
  const ActArgs none{nullptr, nullptr, 0};
  if (recipe == BSFP8_RECIPE_MX_1X32_E8M0) {
    if (row && col)
      hipLaunchKernelGGL((grouped_quantize_kernel<BSFP8_RECIPE_MX_1X32_E8M0, true, true>), grid, block, 0, stream, x,
                         R, C, splits, E, zas, row_q, row_s, col_q, col_s, noop_flag, status, none, tpw);
    else if (row)
      hipLaunchKernelGGL((grouped_quantize_kernel<BSFP8_RECIPE_MX_1X32_E8M0, true, false>), grid, block, 0, stream,
                         x, R, C, splits, E, zas, row_q, row_s, col_q, col_s, noop_flag, status, none, tpw);
    else
      hipLaunchKernelGGL((grouped_quantize_kernel<BSFP8_RECIPE_MX_1X32_E8M0, false, true>), grid, block, 0, stream,
                         x, R, C, splits, E, zas, row_q, row_s, col_q, col_s, noop_flag, status, none, tpw);
  } else if (recipe == BSFP8_RECIPE_MXFP4_1X32_E8M0) {
    if (row && col)
      hipLaunchKernelGGL((grouped_quantize_kernel<BSFP8_RECIPE_MXFP4_1X32_E8M0, true, true>), grid, block, 0, stream,
                         x, R, C, splits, E, zas, row_q, row_s, col_q, col_s, noop_flag, status, none, tpw);
    else if (row)
      hipLaunchKernelGGL((grouped_quantize_kernel<BSFP8_RECIPE_MXFP4_1X32_E8M0, true, false>), grid, block, 0, stream,
                         x, R, C, splits, E, zas, row_q, row_s, col_q, col_s, noop_flag, status, none, tpw);
    else
      hipLaunchKernelGGL((grouped_quantize_kernel<BSFP8_RECIPE_MXFP4_1X32_E8M0, false, true>), grid, block, 0, stream,
                         x, R, C, splits, E, zas, row_q, row_s, col_q, col_s, noop_flag, status, none, tpw);
  } else {
    hipLaunchKernelGGL((grouped_quantize_kernel<BSFP8_RECIPE_PER_CHANNEL_128_F32, false, true>), grid, block, 0,
                       stream, x, R, C, splits, E, zas, row_q, row_s, col_q, col_s, noop_flag, status, none, tpw);
  }
  return hipGetLastError() == hipSuccess ? BSFP8_OK : BSFP8_ERR_LAUNCH;
}

template <int RECIPE, int ACT>
static void launch_act(dim3 grid, dim3 block, hipStream_t stream, bool row, bool col, const uint16_t* x, int64_t R,
                       int64_t C, const int32_t* splits, int E, uint8_t* row_q, uint8_t* row_s, uint8_t* col_q,
                       void* col_s, uint32_t* status, ActArgs a, int tpw) {
  if (row && col)
    hipLaunchKernelGGL((grouped_quantize_kernel<RECIPE, true, true, ACT>), grid, block, 0, stream, x, R, C, splits, E,
                       0.0f, row_q, row_s, col_q, col_s, nullptr, status, a, tpw);
  else if (row)
    hipLaunchKernelGGL((grouped_quantize_kernel<RECIPE, true, false, ACT>), grid, block, 0, stream, x, R, C, splits, E,
                       0.0f, row_q, row_s, col_q, col_s, nullptr, status, a, tpw);
  else
    hipLaunchKernelGGL((grouped_quantize_kernel<RECIPE, false, true, ACT>), grid, block, 0, stream, x, R, C, splits, E,
                       0.0f, row_q, row_s, col_q, col_s, nullptr, status, a, tpw);
}

int launch_grouped_act_quantize(int act, const void* h, const float* probs, const void* dy, int64_t R, int64_t cols,
                                const int32_t* splits, int E, int recipe, int which, uint8_t* row_q, uint8_t* row_s,
                                uint8_t* col_q, void* col_s, uint32_t* status, hipStream_t stream) {
  // output columns: cols, or 2 cols for the GLU gradient (da | db)
  const int64_t C = act == BSFP8_ACT_SWIGLU_GRAD ? 2 * cols : cols;
  const int64_t rtiles = quantize_row_tiles(R, E, true), gy = (C + kQCols - 1) / kQCols;
  const int tpw = quantize_tiles_per_wg(rtiles * gy);
  const int64_t gx = (rtiles + tpw - 1) / tpw;
  if (gx <= 0 || gy <= 0) return BSFP8_OK;
  if (gx * gy > 0x7fffffff) return BSFP8_ERR_SHAPE;
  dim3 grid((unsigned)(gx * gy)), block(kQThreads);
  const uint16_t* x = (const uint16_t*)h;
  const bool row = (which & BSFP8_ROWWISE) != 0, col = (which & BSFP8_COLWISE) != 0;
  const ActArgs a{probs, (const uint16_t*)dy, cols};
  auto go = [&](auto recipe_tag) {
    constexpr int RC = decltype(recipe_tag)::value;
    switch (act) {
      case BSFP8_ACT_SRELU:
        launch_act<RC, 1>(grid, block, stream, row, col, x, R, C, splits, E, row_q, row_s, col_q, col_s, status, a,
                          tpw);
        break;
      case BSFP8_ACT_SRELU_GRAD:
        launch_act<RC, 2>(grid, block, stream, row, col, x, R, C, splits, E, row_q, row_s, col_q, col_s, status, a,
                          tpw);
        break;
      case BSFP8_ACT_SWIGLU:
        launch_act<RC, 3>(grid, block, stream, row, col, x, R, C, splits, E, row_q, row_s, col_q, col_s, status, a,
                          tpw);
        break;
      default:
        launch_act<RC, 4>(grid, block, stream, row, col, x, R, C, splits, E, row_q, row_s, col_q, col_s, status, a,
                          tpw);
    }
  };
  if (recipe == BSFP8_RECIPE_MX_1X32_E8M0)
    go(std::integral_constant<int, BSFP8_RECIPE_MX_1X32_E8M0>());
  else
    go(std::integral_constant<int, BSFP8_RECIPE_MXFP4_1X32_E8M0>());
  return hipGetLastError() == hipSuccess ? BSFP8_OK : BSFP8_ERR_LAUNCH;
}

}  // namespace bsfp8

/*
 * oracle.c -- plain, slow CPU reference for block-scaled FP8 grouped quantize / GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may load or call this file: only the
 * tests, the smoke check and the benchmark's CPU-baseline leg use it.  It shares no code,
 * header, table or constant with the HIP library; both sides only receive the same seeded
 * inputs.  Arithmetic is IEEE fp32 where the method is defined in fp32 (the per-channel cast)
 * and fp64 everywhere else.  Build flags: -O2 -fno-fast-math -ffp-contract=off (no FMA
 * contraction, no reassociation); OpenMP is used only across independent outputs.
 *
 * Sources (cited by page title and section):
 *  [DG365]  DeepGEMM issue #365, "Non-deterministic numerical problem of
 *           k_grouped_fp8_gemm_nt_contiguous": reproducer (per-channel cast, K-major pack,
 *           reference wgrad, stress test).
 *  [TE3484] TransformerEngine issue #3484, "NaN expert weight gradients at num_groups == 1 with
 *           a padded token buffer for SReLU": bug description, reproducer, expected behaviour,
 *           additional context (scope).
 *  [TE3224] TransformerEngine PR #3224, "Improve device-init grouped linear module with single
 *           grouped weight support": summary (MXFP8 kernel fix, zero-row early return).
 *
 * Readings where the pages are silent (each is listed with its reason in the design notes):
 *  - e4m3 is OCP FP8 E4M3FN; rounding is to nearest, ties to the even code; magnitudes >= 448
 *    saturate to 448 (never reached by either recipe for finite input); the sign is kept.
 *  - MXFP8 1x32 scale: the smallest power of two 2^e, e in [-127, 127], with amax <= 448 * 2^e;
 *    amax == 0 gives e = -127 (byte 0).  Stored as the E8M0 byte e + 127.
 *  - MXFP4 (the 4-bit member of the same block-scaled family, next to MXFP8): e2m1 is OCP FP4
 *    E2M1 (values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives); rounding to nearest, ties to
 *    the even code; the scale is the smallest 2^e, e in [-127, 127], with amax <= 6 * 2^e.  Two
 *    codes share a byte along the contiguous axis: element 2i in bits 3..0, 2i+1 in bits 7..4.
 *  - Scale blocks restart at every group start; a partial block takes its amax over live rows.
 *  - Rows at or past sum(split_sizes) are outside every group and are never read.
 *
 * Layouts produced (the same byte layout the library documents, derived here on its own):
 *  group e: k_e = split_sizes[e], off_e = sum_{f<e} k_f, Kp_e = 128 * ceil(k_e / 128),
 *           P_e = sum_{f<e} Kp_f.
 *  colwise data   : byte (e, t, c)  at C*P_e + c*Kp_e + t,   t < Kp_e (t >= k_e holds 0x00)
 *  colwise MX     : E8M0 (e, b, c)  at C*P_e/32 + b*C + c,   b < Kp_e/32
 *  colwise PC128  : fp32 (e, b, c)  at C*P_e/128 + b*C + c,  b < Kp_e/128
 *  rowwise data   : byte (r, c)     at r*C + c
 *  rowwise MX     : E8M0 (r, b)     at b*R + r,              b < C/32
 *  MXFP4          : the same element indices as MXFP8; element i of a data buffer is nibble
 *                   i % 2 of byte i / 2 (so every data buffer has half the bytes)
 *
 * Parity unpinned: none of the functions below; every function has at least one test that pins
 * it to a value fixed by the pages, a library routine, exact arithmetic or brute force.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_ENOMEM (-2)

#define RECIPE_MX 1  /* MXFP8: one E8M0 power-of-two scale per 32 elements */
#define RECIPE_PC 2  /* per channel, one fp32 scale per 128 rows (the DeepGEMM reproducer's cast) */
#define RECIPE_MX4 3 /* MXFP4: e2m1 elements, one E8M0 power-of-two scale per 32 elements */
#define WHICH_ROW 1
#define WHICH_COL 2

/* Number of OpenMP threads the parallel loops below use (1 without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------------------------ */
/* OCP FP8 E4M3FN codec.                                                                       */
/* ------------------------------------------------------------------------------------------ */

/* Value of an e4m3 code: sign bit 7, exponent bits 6..3 with bias 7, mantissa bits 2..0.
 * Exponent field 0 is subnormal (m * 2^-9); pattern S.1111.111 is NaN; there is no infinity. */
double oracle_e4m3_decode(uint8_t q) {
  int sign = (q >> 7) & 1;
  int ef = (q >> 3) & 15;
  int mf = q & 7;
  double mag;
  if (ef == 15 && mf == 7) return NAN;
  if (ef == 0)
    mag = ldexp((double)mf, -9);
  else
    mag = ldexp(1.0 + mf / 8.0, ef - 7);
  return sign ? -mag : mag;
}

/* Nearest e4m3 code to v.  The 127 non-negative finite magnitudes (codes 0..126) are taken in
 * increasing order; v's magnitude is placed between two neighbours and the closer one wins,
 * a tie going to the code whose mantissa LSB (= code LSB) is 0.  Magnitudes >= 448 give 448. */
uint8_t oracle_e4m3_encode(float v) {
  uint8_t sign = signbit(v) ? 0x80 : 0x00;
  double a = fabs((double)v);
  int lo, hi;
  double dlo, dhi;
  if (isnan(v)) return sign | 0x7F;
  if (a >= 448.0) return sign | 126;
  lo = 0;   /* invariant: mag(lo) <= a < mag(hi) */
  hi = 126;
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (oracle_e4m3_decode((uint8_t)mid) <= a)
      lo = mid;
    else
      hi = mid;
  }
  dlo = a - oracle_e4m3_decode((uint8_t)lo);
  dhi = oracle_e4m3_decode((uint8_t)hi) - a;
  if (dlo < dhi) return sign | (uint8_t)lo;
  if (dhi < dlo) return sign | (uint8_t)hi;
  return sign | (uint8_t)((lo & 1) ? hi : lo);
}

void oracle_e4m3_encode_array(const float* v, uint8_t* out, int64_t n) {
  int64_t i;
#pragma omp parallel for schedule(static)
  for (i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(v[i]);
}

void oracle_e4m3_decode_array(const uint8_t* q, double* out, int64_t n) {
  int64_t i;
  for (i = 0; i < n; ++i) out[i] = oracle_e4m3_decode(q[i]);
}

/* MXFP8 scale exponent: smallest e in [-127, 127] with amax <= 448 * 2^e (amax == 0 -> -127).
 * The predicate is monotone in e, so a bisection over the integer range finds it. */
int oracle_e8m0_exponent(float amax) {
  int lo = -127, hi = 127;
  if (!(amax > 0.0f)) return -127;
  if ((double)amax <= ldexp(448.0, lo)) return lo;
  if (!((double)amax <= ldexp(448.0, hi))) return hi; /* unreachable for finite bf16 input */
  /* invariant: predicate false at lo, true at hi */
  while (hi - lo > 1) {
    int mid = lo + (hi - lo) / 2;
    if ((double)amax <= ldexp(448.0, mid))
      hi = mid;
    else
      lo = mid;
  }
  return hi;
}

void oracle_e8m0_exponent_array(const float* amax, int32_t* out, int64_t n) {
  int64_t i;
#pragma omp parallel for schedule(static)
  for (i = 0; i < n; ++i) out[i] = oracle_e8m0_exponent(amax[i]);
}

/* ------------------------------------------------------------------------------------------ */
/* OCP FP4 E2M1 codec and the MXFP4 scale exponent.                                            */
/* ------------------------------------------------------------------------------------------ */

/* Value of an e2m1 code (low 4 bits of q): sign bit 3, exponent bits 2..1 with bias 1, mantissa
 * bit 0.  Exponent field 0 is subnormal (m * 2^-1); every code is finite. */
double oracle_e2m1_decode(uint8_t q) {
  int sign = (q >> 3) & 1;
  int ef = (q >> 1) & 3;
  int mf = q & 1;
  double mag = ef == 0 ? 0.5 * mf : ldexp(1.0 + mf / 2.0, ef - 1);
  return sign ? -mag : mag;
}

/* Nearest e2m1 code to v, by the same placement rule as the e4m3 encoder over the 8
 * non-negative magnitudes (codes 0..7): closer neighbour wins, a tie goes to the code whose
 * mantissa bit is 0; magnitudes >= 6 give 6 (the MXFP4 recipe never exceeds 6). */
uint8_t oracle_e2m1_encode(float v) {
  uint8_t sign = signbit(v) ? 0x8 : 0x0;
  double a = fabs((double)v), dlo, dhi;
  int lo, hi;
  if (a >= 6.0) return sign | 7;
  lo = 0;  /* invariant: mag(lo) <= a < mag(hi) */
  hi = 7;
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (oracle_e2m1_decode((uint8_t)mid) <= a)
      lo = mid;
    else
      hi = mid;
  }
  dlo = a - oracle_e2m1_decode((uint8_t)lo);
  dhi = oracle_e2m1_decode((uint8_t)hi) - a;
  if (dlo < dhi) return sign | (uint8_t)lo;
  if (dhi < dlo) return sign | (uint8_t)hi;
  return sign | (uint8_t)((lo & 1) ? hi : lo);
}

void oracle_e2m1_encode_array(const float* v, uint8_t* out, int64_t n) {
  int64_t i;
  for (i = 0; i < n; ++i) out[i] = oracle_e2m1_encode(v[i]);
}

/* MXFP4 scale exponent: smallest e in [-127, 127] with amax <= 6 * 2^e (amax == 0 -> -127);
 * the same bisection as the MXFP8 rule with the e2m1 maximum. */
int oracle_e8m0_exponent_fp4(float amax) {
  int lo = -127, hi = 127;
  if (!(amax > 0.0f)) return -127;
  if ((double)amax <= ldexp(6.0, lo)) return lo;
  if (!((double)amax <= ldexp(6.0, hi))) return hi; /* unreachable for finite bf16 input */
  while (hi - lo > 1) {
    int mid = lo + (hi - lo) / 2;
    if ((double)amax <= ldexp(6.0, mid))
      hi = mid;
    else
      lo = mid;
  }
  return hi;
}

void oracle_e8m0_exponent_fp4_array(const float* amax, int32_t* out, int64_t n) {
  int64_t i;
  for (i = 0; i < n; ++i) out[i] = oracle_e8m0_exponent_fp4(amax[i]);
}

/* Element i of a data buffer: an e4m3 byte, or nibble i % 2 of byte i / 2 for MXFP4. */
static double elem_value(const uint8_t* q, int64_t i, int recipe) {
  if (recipe == RECIPE_MX4) return oracle_e2m1_decode((uint8_t)((q[i / 2] >> (4 * (i % 2))) & 15));
  return oracle_e4m3_decode(q[i]);
}

/* Stores code c (a byte, or a nibble for MXFP4) as element i of a data buffer. */
static void elem_store(uint8_t* q, int64_t i, uint8_t c, int recipe) {
  if (recipe == RECIPE_MX4) {
    int sh = 4 * (int)(i % 2);
    q[i / 2] = (uint8_t)((q[i / 2] & ~(15 << sh)) | ((c & 15) << sh));
  } else {
    q[i] = c;
  }
}

/* bf16 bit pattern -> fp32 (exact: bf16 is the top half of an fp32). */
static float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* ------------------------------------------------------------------------------------------ */
/* Group layout, derived from a host copy of split_sizes.                                      */
/* ------------------------------------------------------------------------------------------ */

typedef struct {
  int64_t k, off, kp, p;
} group_t;

/* Fills g[0..E) and returns 0, or ORACLE_EINVAL if a size is negative or the sum exceeds R. */
static int group_layout(const int32_t* splits, int32_t E, int64_t R, group_t* g) {
  int64_t off = 0, p = 0;
  int32_t e;
  for (e = 0; e < E; ++e) {
    int64_t k = splits[e];
    if (k < 0) return ORACLE_EINVAL;
    g[e].k = k;
    g[e].off = off;
    g[e].kp = 128 * ((k + 127) / 128);
    g[e].p = p;
    off += k;
    p += g[e].kp;
  }
  if (off > R) return ORACLE_EINVAL;
  return ORACLE_OK;
}

/* Total padded rows sum_e Kp_e (the colwise buffers hold C times this many bytes). */
int64_t oracle_padded_rows(const int32_t* splits, int32_t E) {
  int64_t s = 0;
  int32_t e;
  for (e = 0; e < E; ++e) s += 128 * (((int64_t)splits[e] + 127) / 128);
  return s;
}

/* ------------------------------------------------------------------------------------------ */
/* Grouped quantize.                                                                           */
/* ------------------------------------------------------------------------------------------ */

/* Per-channel cast of one 128-row block of one channel, as the DeepGEMM reproducer defines it:
 * amax in fp32; sf = amax / 448 (fp32 divide); a zero sf is replaced by zero_amax_scale; sf is
 * then clamped from below at 1e-30; each element is multiplied (fp32) by the fp32 reciprocal
 * 1 / sf and converted to e4m3.  vals[0..nlive) are the live elements, q gets nlive codes. */
static float pc_block(const float* vals, int64_t nlive, float zero_amax_scale, uint8_t* q) {
  float amax = 0.0f, sf, r;
  int64_t i;
  for (i = 0; i < nlive; ++i) {
    float a = fabsf(vals[i]);
    if (a > amax) amax = a;
  }
  sf = amax / 448.0f;
  if (sf == 0.0f) sf = zero_amax_scale;
  if (sf < 1e-30f) sf = 1e-30f;
  r = 1.0f / sf;
  for (i = 0; i < nlive; ++i) {
    float v = vals[i] * r;
    q[i] = oracle_e4m3_encode(v);
  }
  return sf;
}

/* MXFP8 / MXFP4 cast of one block of up to 32 live elements: E8M0 exponent from the block
 * amax, each element scaled by 2^-e (exact) and converted to e4m3 or e2m1.  Returns e. */
static int mx_block(const float* vals, int64_t nlive, int recipe, uint8_t* q) {
  float amax = 0.0f;
  int64_t i;
  int e;
  for (i = 0; i < nlive; ++i) {
    float a = fabsf(vals[i]);
    if (a > amax) amax = a;
  }
  e = recipe == RECIPE_MX4 ? oracle_e8m0_exponent_fp4(amax) : oracle_e8m0_exponent(amax);
  for (i = 0; i < nlive; ++i) {
    double v = ldexp((double)vals[i], -e); /* exact power-of-two scaling */
    q[i] = recipe == RECIPE_MX4 ? oracle_e2m1_encode((float)v) : oracle_e4m3_encode((float)v);
  }
  return e;
}

/*
 * in      : bf16 [R][C] row-major (bit patterns); rows >= sum(split_sizes) are never read.
 * splits  : host array of E group sizes, or NULL (rowwise only: all R rows live).
 * row_q   : [R][C] e4m3 (rowwise, MX only; MXFP4: [R][C/2] packed e2m1);  row_s : E8M0 [C/32][R]
 * col_q   : C * sum(Kp_e) bytes (MXFP4: half);  col_s : E8M0 C*sum(Kp_e)/32 bytes (MX, MXFP4)
 *           or fp32 C*sum(Kp_e)/128 (per-channel)
 * Only live rows are written for the rowwise outputs; the colwise outputs are written in full.
 */
/* Element (r, c) of the quantizer's input: a bf16 buffer, or fp32 values computed beforehand. */
static float in_value(const uint16_t* in_bf16, const float* in_f32, int64_t C, int64_t r, int64_t c) {
  return in_f32 ? in_f32[r * C + c] : bf16_to_f32(in_bf16[r * C + c]);
}

static int quantize_values(const uint16_t* in, const float* in_f32, int64_t R, int64_t C,
                           const int32_t* splits, int32_t E, int recipe, int which,
                           float zero_amax_scale, uint8_t* row_q, uint8_t* row_s, uint8_t* col_q,
                           void* col_s) {
  group_t* g;
  group_t all;
  int32_t ng, e;
  if (C <= 0 || C % 32 != 0 || R < 0) return ORACLE_EINVAL;
  if (recipe != RECIPE_MX && recipe != RECIPE_PC && recipe != RECIPE_MX4) return ORACLE_EINVAL;
  if ((which & WHICH_ROW) && recipe == RECIPE_PC) return ORACLE_EINVAL;
  if (splits == NULL) {
    if (which & WHICH_COL) return ORACLE_EINVAL;
    all.k = R; all.off = 0; all.kp = 128 * ((R + 127) / 128); all.p = 0;
    g = &all;
    ng = 1;
  } else {
    if (E <= 0) return ORACLE_EINVAL;
    g = (group_t*)malloc(sizeof(group_t) * (size_t)E);
    if (!g) return ORACLE_ENOMEM;
    if (group_layout(splits, E, R, g) != ORACLE_OK) { free(g); return ORACLE_EINVAL; }
    ng = E;
  }

  /* Rowwise: each live row independently, 32-channel blocks along the row. */
  if (which & WHICH_ROW) {
    for (e = 0; e < ng; ++e) {
      int64_t t;
#pragma omp parallel for schedule(static)
      for (t = 0; t < g[e].k; ++t) {
        int64_t r = g[e].off + t, b;
        float vals[32];
        uint8_t q[32];
        for (b = 0; b < C / 32; ++b) {
          int i, ex;
          for (i = 0; i < 32; ++i) vals[i] = in_value(in, in_f32, C, r, b * 32 + i);
          ex = mx_block(vals, 32, recipe, q);
          for (i = 0; i < 32; ++i) elem_store(row_q, r * C + b * 32 + i, q[i], recipe);
          row_s[b * R + r] = (uint8_t)(ex + 127);
        }
      }
    }
  }

  /* Colwise: per group, per channel, blocks of 32 (MX) or 128 (PC) rows starting at the group
   * start; written K-major (the token index contiguous) into the group's packed slot. */
  if (which & WHICH_COL) {
    int64_t blk = recipe == RECIPE_PC ? 128 : 32;
    for (e = 0; e < ng; ++e) {
      int64_t c;
      int64_t k = g[e].k, kp = g[e].kp, P = g[e].p, off = g[e].off;
#pragma omp parallel for schedule(static)
      for (c = 0; c < C; ++c) {
        int64_t b, t;
        float vals[128];
        uint8_t q[128];
        int64_t base = C * P + c * kp; /* element index of the channel's first row */
        for (b = 0; b < kp / blk; ++b) {
          int64_t t0 = b * blk;
          int64_t nlive = k - t0;
          if (nlive > blk) nlive = blk;
          if (nlive < 0) nlive = 0;
          for (t = 0; t < nlive; ++t) vals[t] = in_value(in, in_f32, C, off + t0 + t, c);
          if (recipe == RECIPE_PC) {
            float sf = pc_block(vals, nlive, zero_amax_scale, q);
            ((float*)col_s)[C * P / 128 + b * C + c] = sf;
          } else {
            int ex = mx_block(vals, nlive, recipe, q);
            ((uint8_t*)col_s)[C * P / 32 + b * C + c] = (uint8_t)(ex + 127);
          }
          for (t = 0; t < blk; ++t) elem_store(col_q, base + t0 + t, t < nlive ? q[t] : 0x00, recipe);
        }
      }
    }
  }
  if (splits != NULL) free(g);
  return ORACLE_OK;
}

int oracle_grouped_quantize(const uint16_t* in, int64_t R, int64_t C, const int32_t* splits,
                            int32_t E, int recipe, int which, float zero_amax_scale,
                            uint8_t* row_q, uint8_t* row_s, uint8_t* col_q, void* col_s) {
  return quantize_values(in, NULL, R, C, splits, E, recipe, which, zero_amax_scale, row_q, row_s, col_q, col_s);
}

/* ------------------------------------------------------------------------------------------ */
/* Activation fused with the quantize: the ScaledSReLU step between fc1 and fc2 of the         */
/* TransformerEngine #3484 reproducer (fc1 -> ScaledSReLU -> fc2, per-token probs).            */
/* ------------------------------------------------------------------------------------------ */

/*
 * Squared ReLU scaled by the token's routing probability, and its gradient, in fp32 (each
 * product rounded to fp32, in this order; r is +0 for h <= 0, including -0):
 *   act 1 (forward)  : r = max(h, 0);  y = (r * r) * p
 *   act 2 (backward) : r = max(h, 0);  g = ((2 * r) * p) * dy
 * h and dy are bf16 [R][C]; probs fp32 [R] (NULL means p = 1).  The fp32 values of the live rows
 * are then quantized exactly like a bf16 input (MX recipes; per-channel is not offered).
 */
static float act_value(int act, float hv, float p, float d) {
  float r = hv > 0.0f ? hv : 0.0f;
  if (act == 1) {
    float r2 = r * r;
    return r2 * p;
  } else {
    float tp = (2.0f * r) * p;
    return tp * d;
  }
}

/* 2^x in fp32 by a stated algorithm, so that any IEEE fp32 machine reproduces it bit for bit:
 * x is clamped to [-126, 126]; k = floor(x + 0.5) and r = x - k (exact, |r| <= 0.5); 2^r is the
 * degree-7 Taylor polynomial of exp(r ln 2), coefficients (ln 2)^n / n! rounded to fp32, in
 * Horner form with every operation rounded to fp32; the result is scaled by 2^k exactly.
 * Relative error below 2e-7 (the truncated series term is below 1.5e-8). */
float oracle_exp2_spec(float x) {
  static const float c[8] = {1.0f, 0.693147182f, 0.240226507f, 0.0555041087f, 0.00961812911f,
                             0.00133335581f, 0.000154035304f, 1.52527338e-05f};
  float r, poly;
  int k, n;
  if (x > 126.0f) x = 126.0f;
  if (x < -126.0f) x = -126.0f;
  k = (int)floorf(x + 0.5f);
  r = x - (float)k;
  poly = c[7];
  for (n = 6; n >= 0; --n) poly = poly * r + c[n];
  return ldexpf(poly, k);
}

/* SwiGLU scaled by the token's probability, and its gradient, in fp32 with the stated exp:
 *   sg = 1 / (1 + exp2_spec(-a * log2(e)));  s = a * sg                  (silu(a))
 *   act 3 (forward) : y = (s * b) * p
 *   act 4 (backward): q = dy * p;  da = (q * b) * (sg * (1 + a * (1 - sg)));  db = q * s
 * with a, b the two halves of fc1's output row (a the first). */
static void glu_values(float a, float b, float p, float d, float* y, float* da, float* db) {
  const float log2e = 1.44269502f;
  float t = oracle_exp2_spec(-a * log2e);
  float den = 1.0f + t;
  float sg = 1.0f / den;
  float sl = a * sg;
  if (y) {
    float sb = sl * b;
    *y = sb * p;
  }
  if (da) {
    float q = d * p;
    float u = 1.0f - sg;
    float v = a * u;
    float w = 1.0f + v;
    float ds = sg * w;
    float qb = q * b;
    *da = qb * ds;
    *db = q * sl;
  }
}

/* The GLU values element by element: a, b, dy bf16 and p fp32 per element; act 3 writes y to
 * out0, act 4 writes da to out0 and db to out1. */
void oracle_glu_values(int act, const uint16_t* a, const uint16_t* b, const float* p, const uint16_t* dy, int64_t n,
                       float* out0, float* out1) {
  int64_t i;
  for (i = 0; i < n; ++i) {
    if (act == 3)
      glu_values(bf16_to_f32(a[i]), bf16_to_f32(b[i]), p[i], 0.0f, &out0[i], NULL, NULL);
    else
      glu_values(bf16_to_f32(a[i]), bf16_to_f32(b[i]), p[i], bf16_to_f32(dy[i]), NULL, &out0[i], &out1[i]);
  }
}

/* The activation values themselves, element by element (h, dy bf16; p fp32 per element). */
void oracle_act_values(int act, const uint16_t* h, const float* p, const uint16_t* dy, int64_t n, float* out) {
  int64_t i;
  for (i = 0; i < n; ++i) out[i] = act_value(act, bf16_to_f32(h[i]), p[i], dy ? bf16_to_f32(dy[i]) : 0.0f);
}

/*
 * acts 1, 2: h [R][C] (and dy [R][C]); the quantized output is [R][C].
 * acts 3, 4 (SwiGLU): C is the GLU width F; h is [R][2F] (a = columns [0, F), b = [F, 2F));
 *   act 3 quantizes y [R][F]; act 4 takes dy [R][F] and quantizes (da | db) as [R][2F].
 */
int oracle_grouped_act_quantize(int act, const uint16_t* h, const float* probs, const uint16_t* dy,
                                int64_t R, int64_t C, const int32_t* splits, int32_t E, int recipe,
                                int which, uint8_t* row_q, uint8_t* row_s, uint8_t* col_q, void* col_s) {
  float* y;
  group_t* g;
  int32_t e;
  int rc;
  int64_t Cout = act == 4 ? 2 * C : C;
  if (act < 1 || act > 4 || ((act == 2 || act == 4) && dy == NULL) || recipe == RECIPE_PC) return ORACLE_EINVAL;
  if (C <= 0 || C % 32 != 0 || R < 0 || splits == NULL || E <= 0) return ORACLE_EINVAL;
  g = (group_t*)malloc(sizeof(group_t) * (size_t)E);
  y = (float*)calloc((size_t)(R > 0 ? R : 1) * (size_t)Cout, sizeof(float));
  if (!g || !y) { free(g); free(y); return ORACLE_ENOMEM; }
  if (group_layout(splits, E, R, g) != ORACLE_OK) { free(g); free(y); return ORACLE_EINVAL; }
  for (e = 0; e < E; ++e) {
    int64_t t, c;
    for (t = g[e].off; t < g[e].off + g[e].k; ++t) { /* live rows only */
      float p = probs ? probs[t] : 1.0f;
      if (act <= 2) {
        for (c = 0; c < C; ++c)
          y[t * C + c] = act_value(act, bf16_to_f32(h[t * C + c]), p, act == 2 ? bf16_to_f32(dy[t * C + c]) : 0.0f);
      } else {
        for (c = 0; c < C; ++c) {
          float a = bf16_to_f32(h[t * 2 * C + c]), b = bf16_to_f32(h[t * 2 * C + C + c]);
          if (act == 3)
            glu_values(a, b, p, 0.0f, &y[t * C + c], NULL, NULL);
          else
            glu_values(a, b, p, bf16_to_f32(dy[t * C + c]), NULL, &y[t * 2 * C + c], &y[t * 2 * C + C + c]);
        }
      }
    }
  }
  rc = quantize_values(NULL, y, R, Cout, splits, E, recipe, which, 0.0f, row_q, row_s, col_q, col_s);
  free(g);
  free(y);
  return rc;
}

/* ------------------------------------------------------------------------------------------ */
/* Dequantization helpers.                                                                     */
/* ------------------------------------------------------------------------------------------ */

/* Dequantized colwise element (e, t, c): dec(q) times its block scale. */
static double col_value(const uint8_t* q, const void* s, int recipe, int64_t C, const group_t* ge,
                        int64_t t, int64_t c) {
  double d = elem_value(q, C * ge->p + c * ge->kp + t, recipe);
  if (recipe != RECIPE_PC) {
    int byte = ((const uint8_t*)s)[C * ge->p / 32 + (t / 32) * C + c];
    return d * ldexp(1.0, byte - 127);
  }
  return d * (double)((const float*)s)[C * ge->p / 128 + (t / 128) * C + c];
}

/* ------------------------------------------------------------------------------------------ */
/* k-grouped weight gradient: dW[e][i][j] = sum_{t < k_e} dy_e[t][i] * x_e[t][j] in fp64,       */
/* t ascending, over the dequantized colwise operands.                                         */
/* ------------------------------------------------------------------------------------------ */

/*
 * rows_sel : NULL for all n rows, else n_sel row indices i (each in [0, n)).
 * out      : fp64 [E][n_sel][h].
 * accumulate = 0: out = sum (0 for an empty group).
 * accumulate = 1: out = mg_in + sum, with mg_in fp32 [E][n][h] (selected rows read); an empty
 *                 group leaves out = mg_in (main_grad untouched).
 */
int oracle_grouped_wgrad(const uint8_t* dy_q, const void* dy_s, int64_t n, const uint8_t* x_q,
                         const void* x_s, int64_t h, const int32_t* splits, int32_t E,
                         int64_t R, int recipe, const int32_t* rows_sel, int32_t n_sel,
                         int accumulate, const float* mg_in, double* out) {
  group_t* g;
  int32_t e;
  int64_t ns = rows_sel ? n_sel : n;
  if (E <= 0 || n <= 0 || h <= 0 || (recipe != RECIPE_MX && recipe != RECIPE_PC && recipe != RECIPE_MX4))
    return ORACLE_EINVAL;
  if (accumulate && !mg_in) return ORACLE_EINVAL;
  g = (group_t*)malloc(sizeof(group_t) * (size_t)E);
  if (!g) return ORACLE_ENOMEM;
  if (group_layout(splits, E, R, g) != ORACLE_OK) { free(g); return ORACLE_EINVAL; }
  for (e = 0; e < E; ++e) {
    int64_t k = g[e].k, ii;
    double *a = NULL, *bm = NULL;
    if (k > 0) {
      int64_t t, j;
      /* dequantize the group's operands: a[ii][t] for the selected dy channels, bm[j][t] */
      a = (double*)malloc(sizeof(double) * (size_t)(ns * k));
      bm = (double*)malloc(sizeof(double) * (size_t)(h * k));
      if (!a || !bm) { free(a); free(bm); free(g); return ORACLE_ENOMEM; }
      for (ii = 0; ii < ns; ++ii) {
        int64_t i = rows_sel ? rows_sel[ii] : ii;
        for (t = 0; t < k; ++t) a[ii * k + t] = col_value(dy_q, dy_s, recipe, n, &g[e], t, i);
      }
#pragma omp parallel for schedule(static) private(t)
      for (j = 0; j < h; ++j)
        for (t = 0; t < k; ++t) bm[j * k + t] = col_value(x_q, x_s, recipe, h, &g[e], t, j);
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (ii = 0; ii < ns; ++ii) {
      int64_t i = rows_sel ? rows_sel[ii] : ii, j, t;
      for (j = 0; j < h; ++j) {
        double s = 0.0;
        double* o = &out[((int64_t)e * ns + ii) * h + j];
        for (t = 0; t < k; ++t) s += a[ii * k + t] * bm[j * k + t];
        if (accumulate)
          *o = (double)mg_in[((int64_t)e * n + i) * h + j] + (k > 0 ? s : 0.0);
        else
          *o = s;
      }
    }
    free(a);
    free(bm);
  }
  free(g);
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* m-grouped forward: out[off_e + t][j] = sum_k x[off_e + t][k] * W[e][j][k] in fp64, k         */
/* ascending, over the dequantized rowwise operands.  Rows >= sum(split_sizes) are not written. */
/* ------------------------------------------------------------------------------------------ */

/*
 * x_q [R][K], x_s E8M0 [K/32][R]; w_q [E*N][K], w_s E8M0 [K/32][E*N] (recipe MX or MXFP4; the
 * data element indices are those of the [R][K] / [E*N][K] matrices).
 * cols_sel : NULL for all N columns, else n_sel column indices j.  out : fp64 [R][n_sel].
 */
int oracle_grouped_fprop(const uint8_t* x_q, const uint8_t* x_s, int64_t R, int64_t K,
                         const uint8_t* w_q, const uint8_t* w_s, int64_t N,
                         const int32_t* splits, int32_t E, int recipe, const int32_t* cols_sel,
                         int32_t n_sel, double* out) {
  group_t* g;
  int32_t e;
  int64_t ns = cols_sel ? n_sel : N;
  int64_t WR = (int64_t)E * N; /* rows of the weight buffer */
  if (E <= 0 || K <= 0 || K % 32 != 0 || N <= 0 || (recipe != RECIPE_MX && recipe != RECIPE_MX4))
    return ORACLE_EINVAL;
  g = (group_t*)malloc(sizeof(group_t) * (size_t)E);
  if (!g) return ORACLE_ENOMEM;
  if (group_layout(splits, E, R, g) != ORACLE_OK) { free(g); return ORACLE_EINVAL; }
  for (e = 0; e < E; ++e) {
    int64_t jj, t, kk;
    double* w;
    if (g[e].k == 0) continue;
    w = (double*)malloc(sizeof(double) * (size_t)(ns * K));
    if (!w) { free(g); return ORACLE_ENOMEM; }
    for (jj = 0; jj < ns; ++jj) {
      int64_t wr = (int64_t)e * N + (cols_sel ? cols_sel[jj] : jj);
      for (kk = 0; kk < K; ++kk)
        w[jj * K + kk] = elem_value(w_q, wr * K + kk, recipe) * ldexp(1.0, (int)w_s[(kk / 32) * WR + wr] - 127);
    }
#pragma omp parallel private(jj, kk)
    {
      double* xr = (double*)malloc(sizeof(double) * (size_t)K); /* one dequantized x row */
#pragma omp for schedule(static)
      for (t = 0; t < g[e].k; ++t) {
        int64_t r = g[e].off + t;
        if (!xr) continue;
        for (kk = 0; kk < K; ++kk)
          xr[kk] = elem_value(x_q, r * K + kk, recipe) * ldexp(1.0, (int)x_s[(kk / 32) * R + r] - 127);
        for (jj = 0; jj < ns; ++jj) {
          double s = 0.0;
          for (kk = 0; kk < K; ++kk) s += xr[kk] * w[jj * K + kk];
          out[r * ns + jj] = s;
        }
      }
      free(xr);
    }
    free(w);
  }
  free(g);
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* m-grouped data gradient: out[off_e + t][j] = sum_c dy[off_e + t][c] * W[e][c][j] in fp64, c  */
/* ascending, over the dequantized rowwise dy and the weight quantized colwise (32-blocks along */
/* c inside each expert).  The token axis is a free dimension here as in the forward GEMM.     */
/* Rows >= sum(split_sizes) are not written.                                                  */
/* ------------------------------------------------------------------------------------------ */

/*
 * dy_q [R][n], dy_s E8M0 [n/32][R] (rowwise).  w_q / w_s: the colwise output for the weight seen
 * as E groups of n rows [E*n][k]: group e has P_e = e*np rows packed (np = 128 * ceil(n/128)), so
 * its byte (c, j) -- row c of the group, channel j -- sits at k*np*e + j*np + c and its E8M0
 * scale (b = c/32, j) at k*np*e/32 + b*k + j (the colwise layout above with C = k).
 * Recipe MX or MXFP4 (element indices as above; MXFP4 packs two per byte).
 * cols_sel : NULL for all k columns, else n_sel column indices j.  out : fp64 [R][n_sel].
 */
int oracle_grouped_dgrad(const uint8_t* dy_q, const uint8_t* dy_s, int64_t R, int64_t n,
                         const uint8_t* w_q, const uint8_t* w_s, int64_t k,
                         const int32_t* splits, int32_t E, int recipe, const int32_t* cols_sel,
                         int32_t n_sel, double* out) {
  group_t* g;
  int32_t e;
  int64_t ns = cols_sel ? n_sel : k;
  int64_t np = 128 * ((n + 127) / 128);
  if (E <= 0 || n <= 0 || n % 32 != 0 || k <= 0 || k % 32 != 0 || (recipe != RECIPE_MX && recipe != RECIPE_MX4))
    return ORACLE_EINVAL;
  g = (group_t*)malloc(sizeof(group_t) * (size_t)E);
  if (!g) return ORACLE_ENOMEM;
  if (group_layout(splits, E, R, g) != ORACLE_OK) { free(g); return ORACLE_EINVAL; }
  for (e = 0; e < E; ++e) {
    int64_t jj, t, c;
    double* w; /* w[jj][c] = W[e][c][j] dequantized */
    if (g[e].k == 0) continue;
    w = (double*)malloc(sizeof(double) * (size_t)(ns * n));
    if (!w) { free(g); return ORACLE_ENOMEM; }
    for (jj = 0; jj < ns; ++jj) {
      int64_t j = cols_sel ? cols_sel[jj] : jj;
      for (c = 0; c < n; ++c)
        w[jj * n + c] = elem_value(w_q, k * np * e + j * np + c, recipe) *
                        ldexp(1.0, (int)w_s[k * np * e / 32 + (c / 32) * k + j] - 127);
    }
#pragma omp parallel private(jj, c)
    {
      double* yr = (double*)malloc(sizeof(double) * (size_t)n); /* one dequantized dy row */
#pragma omp for schedule(static)
      for (t = 0; t < g[e].k; ++t) {
        int64_t r = g[e].off + t;
        if (!yr) continue;
        for (c = 0; c < n; ++c)
          yr[c] = elem_value(dy_q, r * n + c, recipe) * ldexp(1.0, (int)dy_s[(c / 32) * R + r] - 127);
        for (jj = 0; jj < ns; ++jj) {
          double s = 0.0;
          for (c = 0; c < n; ++c) s += yr[c] * w[jj * n + c];
          out[r * ns + jj] = s;
        }
      }
      free(yr);
    }
    free(w);
  }
  free(g);
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* Unquantized brute force (tiny inputs): sum_t dy[off_e+t][i] * x[off_e+t][j] in fp64 from the */
/* bf16 values, as the DeepGEMM reproducer's reference wgrad does in fp32.                     */
/* ------------------------------------------------------------------------------------------ */

int oracle_wgrad_unquantized(const uint16_t* dy, int64_t n, const uint16_t* x, int64_t h,
                             const int32_t* splits, int32_t E, int64_t R, double* out) {
  group_t* g;
  int32_t e;
  if (E <= 0) return ORACLE_EINVAL;
  g = (group_t*)malloc(sizeof(group_t) * (size_t)E);
  if (!g) return ORACLE_ENOMEM;
  if (group_layout(splits, E, R, g) != ORACLE_OK) { free(g); return ORACLE_EINVAL; }
  for (e = 0; e < E; ++e) {
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i) {
      int64_t j, t;
      for (j = 0; j < h; ++j) {
        double s = 0.0;
        for (t = 0; t < g[e].k; ++t) {
          int64_t r = g[e].off + t;
          s += (double)bf16_to_f32(dy[r * n + i]) * (double)bf16_to_f32(x[r * h + j]);
        }
        out[((int64_t)e * n + i) * h + j] = s;
      }
    }
  }
  free(g);
  return ORACLE_OK;
}

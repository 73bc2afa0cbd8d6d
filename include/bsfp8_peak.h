/*
 * bsfp8_peak.h — probes for MI355X (gfx950), built as libbsfp8_peak.so: the MFMA-only
 * throughput probe, the matrix-instruction precision probe, the global -> LDS DMA throughput
 * probe, and the exhaustive checks of the reciprocal the fused SwiGLU uses and of the GEMMs'
 * fp32 -> bf16 output conversion.
 *
 * Not part of the quantize / GEMM path.  The grouped-GEMM throughput is quoted as a fraction of
 * the matrix-core peak; the published dense peaks assume the full engine clock, which a chip
 * running dense MFMA work on random operands need not hold.  This probe measures what the
 * matrix cores sustain on this machine when they do nothing else: every wave of the grid
 * issues independent chains of one MFMA instruction on operands read once from a caller pool,
 * with no memory traffic inside the loop, so the GEMM kernels can be set against it.
 *
 * All pointers are device pointers owned by the caller; nothing is allocated.  Calls are
 * asynchronous on `stream` (a hipStream_t, NULL = the default stream).
 */
#ifndef BSFP8_PEAK_H
#define BSFP8_PEAK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Instruction of a probe launch. */
#define BSFP8_PEAK_BF16 1 /* v_mfma_f32_32x32x16_bf16: the instruction of the MXFP8 GEMMs */
#define BSFP8_PEAK_FP8 2  /* v_mfma_scale_f32_32x32x64_f8f6f4, e4m3 x e4m3, unit scales */
#define BSFP8_PEAK_FP4 3  /* the same, e2m1 x e2m1: the instruction of the MXFP4 GEMMs */

#define BSFP8_PEAK_POOL_WORDS 8192  /* uint32 words of the operand pool */
#define BSFP8_PEAK_THREADS 256      /* threads per workgroup (4 waves) */

/*
 * Run `blocks` workgroups of 4 waves; each wave issues iters x 4 MFMAs of `kind` (4 independent
 * accumulator chains).  Lane t of the grid takes its A and B operand words from the pool at
 * words [16 t, 16 t + 16) modulo BSFP8_PEAK_POOL_WORDS (bf16: 4 words each; fp8: 8 words;
 * fp4: the first 4 of 8), so the operands are whatever the caller put there (random values
 * give the switching activity of real data).  out (fp32 [blocks * 256]) receives one sum of
 * each lane's accumulators, which keeps the work live (all-ones operands make it exactly
 * 4 * 16 * K * iters, K = 16 for bf16 and 64 for fp8 / fp4).
 * stamps (nullable, uint64 [blocks][4]): the first wave of workgroup b writes the shader-clock
 * counter and the real-time counter before its loop and after its last MFMA result,
 * (clk0, rt0, clk1, rt1); (clk1 - clk0) / (rt1 - rt0) times the real-time rate
 * (bsfp8_wall_clock_khz) is the shader clock the chip held meanwhile.
 * Returns 0, or a negative code: -1 NULL pool or out, -2 kind, -3 blocks or iters out of range
 * (1 <= blocks <= 65536, 1 <= iters <= 2^31), -4 the launch failed.
 */
int bsfp8_mfma_peak_probe(int kind, const uint32_t* pool, float* out, int64_t blocks, int64_t iters,
                          uint64_t* stamps, void* stream);

/* Instruction of a precision-probe launch (bsfp8_mfma_dot_probe). */
#define BSFP8_DOT_BF16 1           /* codes widened to bf16 with the block scale, v_mfma_f32_32x32x16_bf16 */
#define BSFP8_DOT_FP8_32X32X64 2   /* v_mfma_scale_f32_32x32x64_f8f6f4, e4m3, E8M0 scales in the instruction */
#define BSFP8_DOT_FP8_16X16X128 3  /* v_mfma_scale_f32_16x16x128_f8f6f4, e4m3, E8M0 scales in the instruction */
#define BSFP8_DOT_FP8_LEGACY 4     /* v_mfma_f32_32x32x16_fp8_fp8 (unscaled; the scales are ignored) */

/*
 * Precision probe: the block-scaled e4m3 product C[i][j] = sum_t deq(A)[i][t] deq(B)[j][t] for
 * i, j < 32, computed by one wave with the instruction `kind` and fp32 accumulation across
 * instructions.  It exists to measure how exactly each matrix instruction sums products
 * (MXFP8 block scaling: TransformerEngine issue #3484, "NaN expert weight gradients at
 * num_groups == 1 with a padded token buffer for SReLU", reproducer; the FP8 k-grouped GEMM
 * of DeepGEMM issue #365, "Non-deterministic numerical problem of
 * k_grouped_fp8_gemm_nt_contiguous", reproducer call).
 *   a_q, b_q  e4m3 codes [32][k] row-major (32-byte aligned device pointers);
 *   a_s, b_s  E8M0 scale bytes [k / 32][32]: block b of row r at b * 32 + r (the rowwise scale
 *             layout of bsfp8_grouped_quantize for 32 rows); kind FP8_LEGACY ignores them;
 *   k         values per row, a multiple of 128 in [128, 65536];
 *   out       fp32 [32][32] row-major, C[i][j] at i * 32 + j.
 * One workgroup of one wave, asynchronous on `stream`.  Returns 0, or -1 NULL pointer, -2 kind,
 * -3 k out of range, -4 the launch failed, -5 a code pointer not 32-byte aligned.
 */
int bsfp8_mfma_dot_probe(int kind, const uint8_t* a_q, const uint8_t* a_s, const uint8_t* b_q, const uint8_t* b_s,
                         int64_t k, float* out, void* stream);

/*
 * Global -> LDS DMA throughput probe: the path the grouped GEMMs stage their operand tiles by
 * (buffer_load_dwordx4 with the lds flag, 16 bytes per lane).  `blocks` workgroups of `waves`
 * waves; workgroup b streams its source region (src + b * span bytes, or src itself for every
 * workgroup when `shared` is nonzero) into LDS, each wave 8 KB per round (8 instructions of
 * 1 KB into its own 8 KB of LDS), waits for its loads, then meets the workgroup at a barrier.
 * Round r of wave w moves the bytes at offsets (r * waves * 8192 + w * 8192 + u * 1024 + 16 l)
 * mod span (instruction u, lane l), each 16 bytes long.  With span * blocks below the L2 the
 * sources stay in it; far above it they stream from HBM.  out (uint32 [blocks * 64 * waves]):
 * thread t = 64 w + l of workgroup b writes, at b * 64 * waves + t, the XOR of the 8 x 4 words
 * it moved in the last round, as read back from LDS.
 * Constraints: span a multiple of 1024 in [8192, 2^31]; the source spans blocks * span bytes
 * (span if shared); 1 <= blocks <= 4096, 1 <= waves <= 8, 1 <= rounds <= 100000.  Returns 0, or
 * -1 NULL pointer, -3 an argument out of range, -4 the launch failed.  The caller times it.
 */
int bsfp8_lds_dma_probe(const uint8_t* src, int64_t span, int shared, int64_t blocks, int waves, int64_t rounds,
                        uint32_t* out, void* stream);

/* Rate of the real-time counter of `device` in kHz (HIP's wall-clock rate), or -1. */
int bsfp8_wall_clock_khz(int device);

/*
 * Check of the fast reciprocal the fused SwiGLU quantize uses (hardware reciprocal and one
 * fused-multiply-add Newton step) against the IEEE-rounded division 1.0f / d, for every fp32
 * bit pattern d in [lo_bits, hi_bits).  *mismatches (device uint64, zeroed by the caller) is
 * increased by the number of patterns that differ; *first_bits (device uint32, set to
 * 0xFFFFFFFF by the caller) is lowered to the smallest differing pattern.
 * Returns 0, -1 NULL pointer, -3 empty range, -4 the launch failed.
 */
int bsfp8_recip_check(uint32_t lo_bits, uint32_t hi_bits, unsigned long long* mismatches, uint32_t* first_bits,
                      void* stream);

/*
 * Check of the fp32 -> bf16 conversion that the GEMMs' bf16 outputs go through (the hardware
 * round-to-nearest-even conversion) for every fp32 bit pattern in [lo_bits, hi_bits): against
 * an integer round-to-nearest-even of the fp32 bits (mode 0), or against truncation (mode 1, a
 * reference that differs, to show the check sees differences).  A NaN must give a bf16 NaN.
 * *mismatches (device uint64, zeroed by the caller) is increased by the number of patterns
 * that differ; *first_bits (device uint32, set to 0xFFFFFFFF by the caller) is lowered to the
 * smallest differing pattern.
 * Returns 0, -1 NULL pointer, -2 unknown mode, -3 empty range, -4 the launch failed.
 */
int bsfp8_bf16_cvt_check(uint32_t lo_bits, uint32_t hi_bits, int mode, unsigned long long* mismatches,
                         uint32_t* first_bits, void* stream);

/* Dense FLOPs one probe launch performs (2 M N K per MFMA), or 0 for an invalid kind. */
double bsfp8_mfma_peak_flops(int kind, int64_t blocks, int64_t iters);

#ifdef __cplusplus
}
#endif

#endif /* BSFP8_PEAK_H */

// Grouped block-scaled FP8 GEMMs on gfx950.
//
//  wgrad (k-grouped; DeepGEMM #365, k_grouped_fp8_gemm_nt_contiguous; TE #3484, the weight
//         gradient contracts over the token axis):  dW[e] (=|+=) dy_e^T x_e over the group's
//         k_e live tokens.  Both operands are the colwise (K-major per group) buffers; K is the
//         group's padded extent Kp_e, a multiple of 128 whose pad lanes hold zeros.
//  fprop (m-grouped; TE PR #3224, grouped GEMM over a single grouped weight; the token axis is
//         a free dimension): out[off_e + t] = x[off_e + t] W_e^T for t < k_e.
//  dgrad (m-grouped, TE #3484 scope: the token axis is free in everything but wgrad): the fprop
//         kernel with the colwise-quantized weight as B, out[off_e + t] = dy[off_e + t] W_e.
//
// Arithmetic.  The operands stay e4m3 (one byte) in HBM and LDS.  In registers every e4m3 value
// is widened to bf16 with its block scale folded in (exact: e4m3 has 4 significant bits and a
// power-of-two scale only moves the exponent), and the products are accumulated by the bf16
// MFMA (v_mfma_f32_32x32x16_bf16) in fp32.  The scaled FP8 MFMA is not used: measured on
// gfx950 it sums each group of 8 products in a ~14-bit window under the group's largest product
// (smaller products are truncated), which leaves about 1.5e-5 relative error on Gaussian data
// and cannot meet a 1e-5 bound; the bf16 MFMA on the same values is within fp32 rounding.
// Per-channel recipe (fp32 scales per 128 rows): unit-scale widening, one partial sum p per
// 128-row K step, folded as acc = fma(p, sa_i * sb_j, acc) in K order.
// MXFP4 recipe (e2m1, two per byte; TE #3484 additional context: a 4-bit block-scaled quantizer
// on the same grouped paths): the operands go to the scaled MFMA as they are
// (v_mfma_scale_f32_32x32x64_f8f6f4 in its fp4 x fp4 form, the E8M0 block scales applied by the
// instruction).  A lane's 16-byte chunk is exactly one 32-element scale block, and every partial
// sum of e2m1 products inside a block is a small multiple of 1/4, so the instruction's inner
// sums are exact and the result is fp32-accumulated like the bf16 path.
//
// Tiling.  Workgroup tile BM x BN, K step of 128 bytes per row, each wave owning a WM x WN
// block of 32 x 32 fragments.  MX recipes: 256 x 256 with 8 waves of 128 x 64 (two waves per
// SIMD, 128 fp32 accumulators each, so one wave's MFMAs run while the other waits on LDS or the
// barrier); per-channel recipe: 128 x 128 with 4 waves of 64 x 64.  Per K step the A and B
// tiles (rows of 128 bytes) and their scales are moved straight from HBM into LDS by LDS DMA
// (buffer loads with the lds flag, 16 bytes per lane, no staging registers), double-buffered;
// the 16-byte chunks of each row are XOR-swizzled so that the fragment reads of consecutive
// rows spread over all banks.  A lane of a 32 x 32 fragment owns row (lane % 32) and reads, for
// the K half s of the step, chunks 4s + h and 4s + 2 + h (h = lane / 32): for MXFP8 the first
// lies in 32-block 2s, the second in 2s + 1, so each half-fragment has a single block scale.
// The next step's loads are issued once the first K half's fragments are read and overlap the
// step's MFMAs.
//
// Determinism: one workgroup per output tile, fixed instruction order, no atomics, no split-K.
// Rows past a group's live rows lie outside the buffer range of the tile's loads, so they read
// as zeros (nothing beyond the live rows is fetched), and their results are not stored.
#include "common.hpp"
#include "group_layout.hpp"
#include "tile_addr.hpp"
#include "tile_sched.hpp"

namespace bsfp8 {

enum { kModeWgrad = 0, kModeFprop = 1 };
// Arithmetic of an MX GEMM: kFmtBf16 widens e4m3 codes to bf16 with the block scale folded in and
// runs the bf16 MFMA (also the per-channel recipe's path); kFmtF4 and kFmtF8 hand e2m1 / e4m3
// codes and their E8M0 bytes to the scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4).
enum { kFmtBf16 = 0, kFmtF4 = 1, kFmtF8 = 2 };

struct GemmArgs {
  const uint8_t* a_q;  // wgrad: dy colwise   fprop: x rowwise
  const void* a_s;
  const uint8_t* b_q;  // wgrad: x colwise    fprop: W rowwise
  const void* b_s;
  int64_t M;           // wgrad: n (dy channels)   fprop: unused (group rows)
  int64_t N;           // wgrad: h (x channels)    fprop: n (weight rows per expert)
  int64_t K;           // fprop / dgrad: reduction length in bytes of a row
  int64_t R;           // capacity rows
  // m-grouped B operand (fprop: the rowwise weight; dgrad: the colwise-quantized weight):
  int64_t b_ld;        // bytes per B row
  int64_t b_estride;   // bytes of B data per group
  int64_t bs_estride;  // B scale bytes per group (offset of the group's first scale)
  int64_t bs_bstride;  // B scale bytes between consecutive 32-blocks along K
  const int32_t* splits;
  int E;
  int tiles_m, tiles_n;  // wgrad: per-group tile grid; fprop: tiles_n only
  int64_t tiles;         // logical tiles (fprop: an upper bound; spare ones exit)
  void* out;
  uint32_t* status;
};

// 16 bytes per lane from a buffer resource straight into LDS (lane l -> lds + 16 l); lanes whose
// offset lies past the resource's range receive zeros.  (A plain __device__ wrapper: the host
// pass of the kernel templates must not see the builtin.)
__device__ __forceinline__ void buffer_dma16(__amdgpu_buffer_rsrc_t rs, uint8_t* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

// The scaled-MFMA loops (MXFP4, MXFP8 on the fp8 MFMA) issue their DMAs as inline assembly (M0 =
// the wave-uniform LDS byte address, one wait state between setting M0 and its use).  Issued through the builtins, the compiler
// cannot tell the DMA into the next LDS stage from the reads of the current one and makes the
// step's later fragment reads wait for it, which leaves the DMA no time to hide behind; the
// kernel waits for its DMAs itself (s_waitcnt vmcnt(0) before a stage is read), and any wait
// the compiler places for its own loads only waits longer, as loads complete in order.
__device__ __forceinline__ void asm_dma16(v4i rsrc, uint32_t lds, uint32_t voff) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voff), "s"(rsrc), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void asm_dma16g(const void* g, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "{m0}"(lds) : "memory");
}
// The four words of a raw buffer resource (base, stride 0, num_records bytes, the flags word
// passed to __builtin_amdgcn_make_buffer_rsrc elsewhere), wave-uniform.
__device__ __forceinline__ v4i rsrc_words(const void* base, uint32_t num_records) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return v4i{__builtin_amdgcn_readfirstlane((int)(uint32_t)a), __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffff)),
             __builtin_amdgcn_readfirstlane((int)num_records), 0x00020000};
}

template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// fp32 value 2^(byte - 127) of an E8M0 scale byte: the exponent field is the byte itself; byte 0
// is the fp32 subnormal 2^-127 (0x00400000, below every byte << 23 for byte >= 1).
__device__ __forceinline__ float e8m0_value(uint32_t byte) { return __uint_as_float(max(byte << 23, 0x00400000u)); }

// Eight e4m3 codes (two dwords) -> eight bf16 values times `scale`.
__device__ __forceinline__ v8bf widen8(int d0, int d1, float scale) {
  const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)d0, scale, false);
  const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)d0, scale, true);
  const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)d1, scale, false);
  const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)d1, scale, true);
  return v8bf{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

template <int MODE, bool PC, int FMT, int BM, int BN, int WM, int WN>
struct GemmShape {
  static constexpr int BK = 128;                    // bytes of a row per K step
  static constexpr int SBLK = FMT == kFmtF4 ? 8 : 4;  // E8M0 scale blocks per K step (MX recipes)
  static constexpr int BLK_BYTES = BK / SBLK;       // bytes of one scale block
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  static constexpr int NW = WAVES_M * WAVES_N, NT = NW * 64;
  static constexpr int FM = WM / 32, FN = WN / 32;
  // LDS stage: A rows, B rows, then scales (the scaled-MFMA paths: [SBLK blocks][rows] E8M0 bytes
  // as they arrive; the widened MXFP8 path: fp32 [4 blocks][rows], decoded from E8M0 words the
  // waves load into registers; PC: one fp32 per row)
  static constexpr bool E8_LDS = !PC && FMT != kFmtBf16;
  static constexpr int A_OFF = 0, B_OFF = BM * BK, SA_OFF = (BM + BN) * BK;
  static constexpr int SB_OFF = SA_OFF + (PC ? BM * 4 : E8_LDS ? SBLK * BM : 0);
  static constexpr int SAF_OFF = SB_OFF + (PC ? BN * 4 : E8_LDS ? SBLK * BN : 0), SBF_OFF = SAF_OFF + 16 * BM;
  static constexpr int STAGE = (PC || FMT != kFmtBf16) ? SAF_OFF : SBF_OFF + 16 * BN;
  static constexpr int A_INS = BM / 8 / NW, B_INS = BN / 8 / NW;  // 1 KB DMA instructions per wave
  static_assert(BM % WM == 0 && BN % WN == 0 && WM % 32 == 0 && WN % 32 == 0, "tile shape");
  static_assert(A_INS * 8 * NW == BM && B_INS * 8 * NW == BN, "DMA loader shape");
  static_assert(2 * STAGE + (int)sizeof(GroupScanSmem<NT>) <= 160 * 1024, "LDS budget");
};

// KTAIL (widened MXFP8 fprop only): K is not a multiple of 128, so the last K step runs past it.
// The scaled-MFMA paths (SC: MXFP4, and MXFP8 on the fp8 MFMA) decide per group at run time
// whether their last K step is such a tail step.
template <int MODE, bool PC, int FMT, int BM, int BN, int WM, int WN, bool ACCUM, int OUT, bool KTAIL>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void grouped_gemm_kernel(GemmArgs args) {
  using S = GemmShape<MODE, PC, FMT, BM, BN, WM, WN>;
  constexpr int NT = S::NT, NW = S::NW, BK = S::BK, FM = S::FM, FN = S::FN;
  constexpr int SBLK = S::SBLK, BLK_BYTES = S::BLK_BYTES;
  constexpr bool F4 = FMT == kFmtF4, F8 = FMT == kFmtF8, SC = F4 || F8;
  constexpr int EPB = F4 ? 2 : 1;  // elements per data byte
  static_assert(!(PC && SC) && !(KTAIL && SC), "recipe flags");
  __shared__ GroupScanSmem<NT> gsm;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * S::STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int wm = wave % S::WAVES_M, wn = wave / S::WAVES_M;

  // ---------------- tile placement (device scheduler) ----------------
  GroupInfo gi;
  int e, tm, tn;
  // workgroup -> logical tile in the XCD-aware order; workgroup 0 always has tile 0 and is
  // the one that reports the status bits
  if constexpr (MODE == kModeWgrad) {
    // e is the group's place in the order: its index, or, when the split is skewed, its size
    // rank (largest groups first; see group_scan), the tiles then dealt to the XCDs in short
    // runs (kSkewRun).  The scan decides the skew before the tile is placed.
    const uint32_t flags = group_scan<NT>(
        args.splits, args.E, args.R, 0, 0,
        [&](bool skewed) {
          const int64_t L = xcd_logical(blockIdx.x, skewed ? kSkewRun : kCusPerXcd);
          if (L >= args.tiles) return -1;
          wgrad_tile(L, args.tiles_m, args.tiles_n, &e, &tm, &tn);
          return e;
        },
        gsm, gi, true);
    report_status(args.status, flags);
    if (gi.e < 0) return;
    e = gi.e;
  } else {
    const int64_t L = xcd_logical(blockIdx.x);
    if (L >= args.tiles) return;
    int64_t mt;
    fprop_tile(L, args.tiles_n, &mt, &tn);
    const uint32_t flags = group_scan<NT>(args.splits, args.E, args.R, BM, mt, 0, gsm, gi);
    report_status(args.status, flags);
    if (gi.e < 0) return;
    e = gi.e;
    tm = (int)(mt - gi.tile);
  }

  // ---------------- operand descriptors ----------------
  const uint8_t *a_data, *b_data, *a_sc, *b_sc;
  int64_t lda, ldb, a_sld, b_sld, a_valid, b_valid, kext;
  const int64_t a_row0 = (int64_t)tm * BM, b_row0 = (int64_t)tn * BN;
  if constexpr (MODE == kModeWgrad) {
    if (gi.k == 0) {
      if constexpr (!ACCUM) {  // an empty group's gradient is zero
        float* o = (float*)args.out + ((int64_t)e * args.M + a_row0) * args.N + b_row0;
        for (int idx = tid; idx < BM * BN / 4; idx += NT) {
          const int r = idx / (BN / 4), c = (idx % (BN / 4)) * 4;
          if (a_row0 + r < args.M && b_row0 + c < args.N) *(float4*)(o + (int64_t)r * args.N + c) = float4{0, 0, 0, 0};
        }
      }
      return;
    }
    // the group's slice of the colwise buffers (group_layout.hpp): M (resp. N) channel rows of
    // Kp codes each, scales block-major with M (N) entries per block
    lda = ldb = col_row_bytes(gi.kp, EPB);
    kext = col_row_bytes(gi.kp, EPB);
    a_data = args.a_q + col_group_bytes(args.M, gi.p, EPB);
    b_data = args.b_q + col_group_bytes(args.N, gi.p, EPB);
    a_valid = args.M;
    b_valid = args.N;
    if constexpr (PC) {
      a_sc = (const uint8_t*)((const float*)args.a_s + col_pc_scale_group(args.M, gi.p));
      b_sc = (const uint8_t*)((const float*)args.b_s + col_pc_scale_group(args.N, gi.p));
    } else {
      a_sc = (const uint8_t*)args.a_s + col_e8m0_group(args.M, gi.p);
      b_sc = (const uint8_t*)args.b_s + col_e8m0_group(args.N, gi.p);
    }
    a_sld = col_e8m0_block_stride(args.M);
    b_sld = col_e8m0_block_stride(args.N);
  } else {
    lda = args.K;
    ldb = args.b_ld;
    kext = args.K;
    a_data = args.a_q + gi.off * args.K;
    b_data = args.b_q + (int64_t)e * args.b_estride;
    a_sc = (const uint8_t*)args.a_s + gi.off;
    b_sc = (const uint8_t*)args.b_s + (int64_t)e * args.bs_estride;
    a_sld = args.R;
    b_sld = args.bs_bstride;
    a_valid = gi.k;
    b_valid = args.N;
  }
  const int nk = (int)((kext + BK - 1) / BK);
  const int64_t nblk = (kext + BLK_BYTES - 1) / BLK_BYTES;  // scale blocks along K

  // ---------------- loads of one K step, straight into LDS ----------------
  // One DMA instruction moves 64 lanes x 16 bytes = 8 rows x 128 bytes; lane l fills LDS slot
  // l of the region, i.e. row 8g + l/8, swizzled chunk l%8, which holds K chunk (l%8) ^ swz(row).
  // The operand tiles are read through buffer resources that end with the tile's last valid
  // row: rows past it come back as zeros from the hardware range check (and are never stored),
  // so no lane needs a clamp.  A K chunk past kext (fprop tail step only) holds bytes of the
  // next row; the tail step masks it when reading fragments.  Each lane keeps its step-0 offset
  // in 32 bits (the host bounds 256 * ld + 128 by 2^32) and adds k0.
  const int a_last = (int)(a_valid - 1 - a_row0), b_last = (int)(b_valid - 1 - b_row0);  // >= 0
  const __amdgpu_buffer_rsrc_t a_rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a_data + a_row0 * lda), (short)0, (int)tile_range(a_valid - a_row0, lda), 0x00020000);
  const __amdgpu_buffer_rsrc_t b_rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(b_data + b_row0 * ldb), (short)0, (int)tile_range(b_valid - b_row0, ldb), 0x00020000);
  // LDS byte address of a place in smem (the assembly DMAs take it in M0)
  const uint32_t smem_lds =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)smem);
  auto lds_of = [&](const uint8_t* p) { return smem_lds + (uint32_t)(p - smem); };
  auto dma4 = [&](const void* g, uint8_t* l) {  // the per-channel recipe's fp32 scales
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)l, 4, 0, 0);
  };
  const v4i a_rw = rsrc_words(a_data + a_row0 * lda, (uint32_t)tile_range(a_valid - a_row0, lda));
  const v4i b_rw = rsrc_words(b_data + b_row0 * ldb, (uint32_t)tile_range(b_valid - b_row0, ldb));
  constexpr int FA_ROWS = SBLK * BM / NT;  // fprop: A-scale bytes (rows) each thread stages per K step
  uint8_t fa_b[FA_ROWS];                 // fprop: those bytes, held in registers until settle
  uint32_t a_off[S::A_INS], b_off[S::B_INS];
  // widened MX recipe: this wave's E8M0 scale words of the step whose loads are in flight
  uint32_t sc_w[(PC || SC) ? 1 : (SBLK * BM / 256 + SBLK * BN / 256) / NW];
#pragma unroll
  for (int u = 0; u < S::A_INS; ++u) a_off[u] = tile_dma_voffset(wave * S::A_INS + u, lane, (uint32_t)lda, 0);
#pragma unroll
  for (int u = 0; u < S::B_INS; ++u) b_off[u] = tile_dma_voffset(wave * S::B_INS + u, lane, (uint32_t)ldb, 0);
  // parts [p0, p1) of the step's loads: part 0 the fprop A scales, parts u < A_INS the A data
  // DMAs, then B_INS of B data, then the scale DMAs
  auto issue = [&](int kk, uint8_t* __restrict__ base, int p0 = 0, int p1 = 1 << 20) {
    const uint32_t k0 = (uint32_t)kk * BK;
    if (MODE == kModeFprop && p0 == 0) {
      // A scales first: waiting for these register loads (in settle) then does not wait for
      // the DMAs behind them.  Thread t -> block t / (NT / SBLK) of this K step, rows
      // FA_ROWS * (t % (NT / SBLK)) and the next FA_ROWS - 1 (t / (NT / SBLK) = wave / (NW / SBLK),
      // t % (NT / SBLK) = (wave % (NW / SBLK)) * 64 + lane: the block index comes from the scalar
      // wave index, so the buffer resource below is wave-uniform).
      static_assert((FA_ROWS == 2 || FA_ROWS == 4) && NW % SBLK == 0, "fprop A-scale staging shape");
      const int blk = wave / (NW / SBLK), r0 = FA_ROWS * ((wave % (NW / SBLK)) * 64 + lane);
      const int64_t kb = (int64_t)kk * SBLK + blk;
      if constexpr (SC) {
        // no branch: a block past kext loads the last valid one; settle() puts unit scales there
        const int64_t kbc = kb < nblk ? kb : nblk - 1;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(a_sc + kbc * a_sld + a_row0), (short)0, a_last + 1, 0x00020000);
#pragma unroll
        for (int i = 0; i < FA_ROWS; ++i) fa_b[i] = __builtin_amdgcn_raw_buffer_load_b8(rs, r0 + i, 0, 0);
      } else if (kb * BLK_BYTES < kext) {
        // the group's scale bytes of this block through a buffer resource spanning its valid
        // rows: rows past them read as 0 (their products are never stored)
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(a_sc + kb * a_sld + a_row0), (short)0, a_last + 1, 0x00020000);
#pragma unroll
        for (int i = 0; i < FA_ROWS; ++i) fa_b[i] = __builtin_amdgcn_raw_buffer_load_b8(rs, r0 + i, 0, 0);
      } else {
#pragma unroll
        for (int i = 0; i < FA_ROWS; ++i) fa_b[i] = 0x7f;  // past K: unit scales over zero data
      }
    }
#pragma unroll
    for (int u = 0; u < S::A_INS; ++u) {
      if (u < p0 || u >= p1) continue;
      const int g = wave * S::A_INS + u;
      if constexpr (SC) asm_dma16(a_rw, lds_of(base + S::A_OFF + g * 1024), a_off[u] + k0);
      else buffer_dma16(a_rs, base + S::A_OFF + g * 1024, a_off[u] + k0);
    }
#pragma unroll
    for (int u = 0; u < S::B_INS; ++u) {
      if (S::A_INS + u < p0 || S::A_INS + u >= p1) continue;
      const int g = wave * S::B_INS + u;
      if constexpr (SC) asm_dma16(b_rw, lds_of(base + S::B_OFF + g * 1024), b_off[u] + k0);
      else buffer_dma16(b_rs, base + S::B_OFF + g * 1024, b_off[u] + k0);
    }
    if (S::A_INS + S::B_INS < p0 || S::A_INS + S::B_INS >= p1) return;
    if constexpr (PC) {
      // one fp32 per row: BM + BN dwords, 64 per instruction
      constexpr int S_INS = (BM + BN) / 64;
      static_assert(S_INS % NW == 0, "PC scale loader shape");
#pragma unroll
      for (int u = 0; u < S_INS / NW; ++u) {
        const int v = wave * (S_INS / NW) + u;
        const int row = v * 64 + lane;
        if (v * 64 < BM) {
          dma4((const float*)a_sc + (int64_t)kk * a_sld + a_row0 + min(row, a_last), base + S::SA_OFF + v * 256);
        } else {
          dma4((const float*)b_sc + (int64_t)kk * b_sld + b_row0 + min(row - BM, b_last), base + S::SA_OFF + v * 256);
        }
      }
    } else if constexpr (SC) {
      // E8M0 block rows [blk][row], 16 bytes per lane: one instruction moves four whole 256-row
      // blocks (1 KB, contiguous in LDS), a quarter of the instructions 4-byte loads take (1-3%
      // on every scaled GEMM).  wgrad loads the A and B blocks, the m-grouped kernels the B
      // (weight) blocks; their token rows' A scales go through registers (part 0 above).  The
      // waves take the instructions in turn and waves past their number repeat one, writing the
      // same bytes to the same place: no branch in the step.  A lane past the tile's valid rows
      // reloads the last valid 16 bytes (valid rows are a multiple of 32), and a block past kext
      // reloads the last valid block: every source byte lies in the group's scale rows, and the
      // finite scales of a block past kext multiply the chunks settle() zeroes.
      static_assert(BM == 256 && BN == 256, "16-byte scale loader shape");
      constexpr int NA = MODE == kModeWgrad ? SBLK * BM / 1024 : 0, NI = NA + SBLK * BN / 1024;
      const int v = wave % NI;
      const bool is_a = v < NA;
      const int vv = is_a ? v : v - NA;
      const int blk = 4 * vv + (lane >> 4);
      const int r = scale_dma16_row(lane, is_a ? a_last : b_last);
      const int64_t kb = (int64_t)kk * SBLK + blk;
      const int64_t kbc = kb < nblk ? kb : nblk - 1;
      const uint8_t* src = (is_a ? a_sc + a_row0 : b_sc + b_row0) + kbc * (is_a ? a_sld : b_sld) + r;
      asm_dma16g(src, lds_of(base + (is_a ? S::SA_OFF : S::SB_OFF) + 4 * vv * 256));
    } else {
      // the widened path: E8M0 block rows [blk][row], 4 rows of 4 bytes per lane into registers
      constexpr int SA_INS = SBLK * BM / 256, SB_INS = SBLK * BN / 256;
      static_assert((SA_INS + SB_INS) % NW == 0, "MX scale loader shape");
#pragma unroll
      for (int u = 0; u < (SA_INS + SB_INS) / NW; ++u) {
        const int v = wave * ((SA_INS + SB_INS) / NW) + u;
        const bool is_a = v < SA_INS;
        const int vv = is_a ? v : v - SA_INS;
        // the 256 bytes [vv * 256, +256) of the [blk][rows] block rows: 4 rows per lane (a
        // 128-row tile: lanes 0-31 one block, lanes 32-63 the next)
        int blk, part, plane;  // scale rows part * 256 + 4 * plane ..
        if constexpr (BM >= 256 && BN >= 256) {
          const int per = (is_a ? BM : BN) / 256;
          blk = vv / per;
          part = vv % per;
          plane = lane;
        } else {
          const int rows = is_a ? BM : BN, flat = vv * 256 + 4 * lane;
          blk = flat / rows;
          part = 0;
          plane = (flat % rows) >> 2;
        }
        const int64_t kb = (int64_t)kk * SBLK + blk;
        if (MODE == kModeFprop && is_a) {
          // rows of a group start anywhere: single-byte loads per thread instead (above)
        } else if (MODE == kModeFprop && kb * BLK_BYTES >= kext) {
          sc_w[u] = 0x7f7f7f7fu;  // past K: unit scales over zero data
        } else {
          // valid rows are a multiple of 32 here, so a group of 4 is all valid or all past.  The
          // word goes to a register: settle() decodes it from there after the step's wait, with
          // no LDS round trip between that wait and the barrier (1-1.5% on every widened GEMM
          // against landing the bytes in LDS by DMA and reading them back)
          const int r4 = scale_dma_row(part, plane, is_a ? a_last : b_last);
          sc_w[u] = *(const uint32_t*)((is_a ? a_sc + a_row0 : b_sc + b_row0) + kb * (is_a ? a_sld : b_sld) + r4);
        }
      }
    }
  };
  // After the step's loads have landed: decode its E8M0 scales once into the stage's fp32 area,
  // so the fragment reads take fp32 scales with no per-read decode.  Each wave decodes the 256
  // bytes of scale words it loaded into registers (sc_w), and the fprop A scales come from the
  // register-staged bytes (fa_b).  (The scaled-MFMA paths take the E8M0 bytes from LDS as they
  // are; their settle() only places the fprop A scales and fixes up a tail step.)
  auto settle = [&](uint8_t* base, int kk) {
    if constexpr (SC) {
      // The scaled MFMA takes the E8M0 bytes as they are.  The fprop A scales, staged in
      // registers, are written to their [blk][row] place (unit scales for blocks past kext).
      if constexpr (MODE == kModeFprop) {
        const int blk = wave / (NW / SBLK);
        const bool valid = ((int64_t)kk * SBLK + blk) * BLK_BYTES < kext;
        uint8_t* f = base + S::SA_OFF + blk * BM + FA_ROWS * ((wave % (NW / SBLK)) * 64 + lane);
#pragma unroll
        for (int i = 0; i < FA_ROWS; ++i) f[i] = valid ? fa_b[i] : (uint8_t)0x7f;
      }
      // The scale blocks the DMA loaded past kext hold the last valid block's finite scales
      // (several waves may load the same bytes, so no wave rewrites them); they multiply the
      // chunks zeroed here.  A tail step: the 16-byte chunks this wave's data DMA put past kext (bytes of the next
      // row, or zeros past the operand) become zeros, so the step needs no masking
      const int64_t k0 = (int64_t)kk * BK;
      if (k0 + BK > kext) {
#pragma unroll
        for (int u = 0; u < S::A_INS; ++u) {
          const int g = wave * S::A_INS + u;
          if (k0 + dma_chunk(g, lane) >= kext) *(v4i*)(base + S::A_OFF + g * 1024 + 16 * lane) = v4i{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < S::B_INS; ++u) {
          const int g = wave * S::B_INS + u;
          if (k0 + dma_chunk(g, lane) >= kext) *(v4i*)(base + S::B_OFF + g * 1024 + 16 * lane) = v4i{0, 0, 0, 0};
        }
      }
    } else if constexpr (!PC) {
      constexpr int SA_INS = SBLK * BM / 256, SB_INS = SBLK * BN / 256, PER = (SA_INS + SB_INS) / NW;
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int v = wave * PER + u;
        const bool is_a = v < SA_INS;
        if (MODE == kModeFprop && is_a) continue;
        const int vv = is_a ? v : v - SA_INS;
        int idx;  // first of the lane's 4 rows in [blk][rows]
        if constexpr (BM >= 256 && BN >= 256) {
          const int per = (is_a ? BM : BN) / 256;
          idx = (is_a ? (vv / per) * BM : (vv / per) * BN) + (vv % per) * 256 + 4 * lane;
        } else {
          idx = vv * 256 + 4 * lane;
        }
        const uint32_t w4 = sc_w[u];
        float* f = (float*)(base + (is_a ? S::SAF_OFF : S::SBF_OFF)) + idx;
        *(v4f*)f = v4f{e8m0_value(w4 & 0xffu), e8m0_value((w4 >> 8) & 0xffu), e8m0_value((w4 >> 16) & 0xffu),
                       e8m0_value(w4 >> 24)};
      }
      if constexpr (MODE == kModeFprop) {
        float* f = (float*)(base + S::SAF_OFF) + (wave / (NW / 4)) * BM + FA_ROWS * ((wave % (NW / 4)) * 64 + lane);
#pragma unroll
        for (int i = 0; i < FA_ROWS; ++i) f[i] = e8m0_value(fa_b[i]);
      }
    }
  };
  auto wait_dma = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  v16f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // One K step.  `cur` (read) and `nxt` (DMA target) are distinct LDS stages; passing them as
  // restrict pointers lets the compiler see that the fragment reads of `cur` need not wait for
  // the DMA into `nxt`, so the loads overlap this step's MFMAs.
  auto step = [&](auto tail_tag, int kk, const uint8_t* __restrict__ cur, uint8_t* __restrict__ nxt) {
    // the fprop step that runs past kext: chunks at or past it read as zeros
    constexpr bool TAIL = decltype(tail_tag)::value;
    const int64_t k0 = (int64_t)kk * BK;
    auto chunk = [&](const uint8_t* p, int c) {
      const v4i v = *(const v4i*)p;
      if constexpr (TAIL) return k0 + 16 * c < kext ? v : v4i{0, 0, 0, 0};
      else return v;
    };
    v16f part[FM][FN];
    if constexpr (PC) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) part[i][j][r] = 0.0f;
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      // this K half's fp8 fragments and block scales -> registers
      v8i af[FM], bf[FN];
      float as[FM][2], bs[FN][2];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int row = wm * WM + i * 32 + l32;
        const v4i lo = chunk(cur + S::A_OFF + row * BK + (((4 * s + h) ^ swz(row)) << 4), 4 * s + h);
        const v4i hi = chunk(cur + S::A_OFF + row * BK + (((4 * s + 2 + h) ^ swz(row)) << 4), 4 * s + 2 + h);
        af[i] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        if constexpr (!PC) {
          as[i][0] = ((const float*)(cur + S::SAF_OFF))[(2 * s) * BM + row];
          as[i][1] = ((const float*)(cur + S::SAF_OFF))[(2 * s + 1) * BM + row];
        }
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int row = wn * WN + j * 32 + l32;
        const v4i lo = chunk(cur + S::B_OFF + row * BK + (((4 * s + h) ^ swz(row)) << 4), 4 * s + h);
        const v4i hi = chunk(cur + S::B_OFF + row * BK + (((4 * s + 2 + h) ^ swz(row)) << 4), 4 * s + 2 + h);
        bf[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        if constexpr (!PC) {
          bs[j][0] = ((const float*)(cur + S::SBF_OFF))[(2 * s) * BN + row];
          bs[j][1] = ((const float*)(cur + S::SBF_OFF))[(2 * s + 1) * BN + row];
        }
      }
      // the next step's loads go out after this half's reads are issued (issued before the first
      // read of `cur`, the compiler would make every read of the step wait for them), spread in
      // four parts over this half's MFMA groups, below: issued together, all of every wave's
      // loads queue at once behind the texture unit and hold back the MFMAs (spread, wgrad and
      // fprop run 2-3% faster; spread over both halves, 5% slower: the last ones land too late)
      // widen and multiply: 4 bf16 MFMAs (K = 16 each) per fragment pair
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        v8bf aw[FM], bw[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) aw[i] = widen8(af[i][2 * t], af[i][2 * t + 1], PC ? 1.0f : as[i][t >> 1]);
#pragma unroll
        for (int j = 0; j < FN; ++j) bw[j] = widen8(bf[j][2 * t], bf[j][2 * t + 1], PC ? 1.0f : bs[j][t >> 1]);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            if constexpr (PC) part[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw[i], bw[j], part[i][j], 0, 0, 0);
            else acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw[i], bw[j], acc[i][j], 0, 0, 0);
          }
        if (s == 0 && kk + 1 < nk) {
          constexpr int NP = S::A_INS + S::B_INS + 1;
          issue(kk + 1, nxt, t * NP / 4, t == 3 ? (1 << 20) : (t + 1) * NP / 4);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    if constexpr (PC) {
      // fold this 128-row block: acc = fma(p, sa_i * sb_j, acc)
      const float* fsa = (const float*)(cur + S::SA_OFF);
      const float* fsb = fsa + BM;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const float bsc = fsb[wn * WN + j * 32 + l32];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = wm * WM + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            acc[i][j][r] = __builtin_fmaf(part[i][j][r], fsa[row] * bsc, acc[i][j][r]);
          }
        }
    }
  };

  // MXFP4 K step: the same chunks as above go to the scaled MFMA without widening.  MFMA u of the
  // step (K elements [64u, 64u + 64), chunks 2u and 2u + 1) takes chunk 2u + h of each lane's row,
  // one whole E8M0 block, with that block's scale byte; for the half s = u / 2 these are the
  // chunks 4s + h and 4s + 2 + h read above.
  // Per-fragment LDS bases of the MXFP4 step.  Chunk c = 4s + 2u + h of a row sits at
  // row * BK + ((c ^ swz(row)) << 4) = base ^ ((4s + 2u) << 4) with base = row * BK + ((h ^ swz(row))
  // << 4) (4s + 2u is even and row * BK has no bits below 128); its E8M0 byte at
  // SA_OFF + (h * BM + row) + (4s + 2u) * BM.  Six bases per operand stay live, not 24 addresses.
  uint32_t a4b[FM], a4s[FM], b4b[FN], b4s[FN];
  if constexpr (SC) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int row = wm * WM + i * 32 + l32;
      a4b[i] = (uint32_t)(S::A_OFF + row * BK + ((h ^ swz(row)) << 4));
      a4s[i] = (uint32_t)(S::SA_OFF + h * BM + row);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int row = wn * WN + j * 32 + l32;
      b4b[j] = (uint32_t)(S::B_OFF + row * BK + ((h ^ swz(row)) << 4));
      b4s[j] = (uint32_t)(S::SB_OFF + h * BN + row);
    }
  }
  // The step is one basic block with no branch: it always issues the next step's loads (after
  // the last step they fetch clamped, in-range addresses into the idle stage and are waited for
  // before the epilogue), and a tail step needs no masking because settle() zeroed its chunks
  // past kext.  So the scheduler can interleave each chunk group's reads with the MFMAs of the
  // group before.
  auto step4 = [&](int kk, const uint8_t* __restrict__ cur, uint8_t* __restrict__ nxt) {
    auto chunk = [&](uint32_t off, int) { return *(const v4i*)(cur + off); };
    auto op = [](v4i v) { return __builtin_shufflevector(v, v, 0, 1, 2, 3, -1, -1, -1, -1); };
    // opaque per step: the chunk addresses are formed where they are used (one XOR each)
    // instead of being hoisted out of the K loop into 24 live registers
#pragma unroll
    for (int i = 0; i < FM; ++i) asm volatile("" : "+v"(a4b[i]), "+v"(a4s[i]));
#pragma unroll
    for (int j = 0; j < FN; ++j) asm volatile("" : "+v"(b4b[j]), "+v"(b4s[j]));
    // chunk group g = 2s + u (chunk 4s + 2u + h of each row): its fragments and scale bytes
    v4i af[2][FM], bf[2][FN];
    int as[2][FM], bs[2][FN];
    auto rd = [&](int g, int buf) {
      const int ce = 2 * g;  // the chunk index without h
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        af[buf][i] = chunk(a4b[i] ^ (uint32_t)(ce << 4), ce + h);
        as[buf][i] = cur[a4s[i] + ce * BM];
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        bf[buf][j] = chunk(b4b[j] ^ (uint32_t)(ce << 4), ce + h);
        bs[buf][j] = cur[b4s[j] + ce * BN];
      }
    };
    auto mm = [&](int buf) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(op(af[buf][i]), op(bf[buf][j]), acc[i][j], 4, 4,
                                                                       0, as[buf][i], 0, bs[buf][j]);
    };
    // software pipeline over the 4 groups: group g + 1's reads go out beside group g's MFMAs;
    // the scheduling fences keep each phase's reads from being hoisted further up (two groups'
    // fragments fit beside the accumulators, four do not)
    // wgrad spreads the next step's loads in three parts over the first three groups (2% faster,
    // as in the bf16 step above); the forward issues them together (spread, its A-scale
    // registers no longer fit beside the fragments and spill)
    constexpr int NP = S::A_INS + S::B_INS + 1;
    constexpr int P1 = MODE == kModeWgrad ? NP / 3 : NP, P2 = MODE == kModeWgrad ? 2 * NP / 3 : NP;
    rd(0, 0);
    issue(kk + 1, nxt, 0, P1);
    __builtin_amdgcn_sched_barrier(0);
    rd(1, 1);
    mm(0);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (P1 < NP) issue(kk + 1, nxt, P1, P2);
    __builtin_amdgcn_sched_barrier(0);
    rd(2, 0);
    mm(1);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (P2 < NP) issue(kk + 1, nxt, P2);
    __builtin_amdgcn_sched_barrier(0);
    rd(3, 1);
    mm(0);
    __builtin_amdgcn_sched_barrier(0);
    mm(1);
    // the MFMAs stay in this step: sunk below the DMA wait and barrier that follow, they would
    // keep all four groups' fragments live at once
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) asm volatile("" : "+v"(acc[i][j]));
  };
  // MXFP8 K step on the scaled fp8 MFMA.  MFMA m of the step (K bytes [64 m, 64 m + 64)) takes
  // from lane (row, h) the two 16-byte chunks 4 m + h and 4 m + 2 + h of its row, in its first and
  // last four registers, and the E8M0 byte of block 2 m + h: the instruction pairs the chunks
  // of one scale block over the lanes (row, 0) and (row, 1) (measured on the GPU; the precision
  // probe of the probe library pins this layout).  These are the chunks the widened path reads
  // for its K half m.  Same structure as the MXFP4 step: branch-free, the next step's loads
  // always issued (here first: measured 2% faster than after the first reads), the second
  // MFMA's reads beside the first's MFMAs.
  auto step8f = [&](int kk, const uint8_t* __restrict__ cur, uint8_t* __restrict__ nxt) {
    auto chunk = [&](uint32_t off) { return *(const v4i*)(cur + off); };
#pragma unroll
    for (int i = 0; i < FM; ++i) asm volatile("" : "+v"(a4b[i]), "+v"(a4s[i]));
#pragma unroll
    for (int j = 0; j < FN; ++j) asm volatile("" : "+v"(b4b[j]), "+v"(b4s[j]));
    v8i af[2][FM], bf[2][FN];
    int as[2][FM], bs[2][FN];
    auto rd = [&](int m, int buf) {
      const uint32_t lo = (uint32_t)(4 * m) << 4, hi = (uint32_t)(4 * m + 2) << 4;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const v4i a = chunk(a4b[i] ^ lo), b = chunk(a4b[i] ^ hi);
        af[buf][i] = v8i{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        as[buf][i] = cur[a4s[i] + 2 * m * BM];
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const v4i a = chunk(b4b[j] ^ lo), b = chunk(b4b[j] ^ hi);
        bf[buf][j] = v8i{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        bs[buf][j] = cur[b4s[j] + 2 * m * BN];
      }
    };
    auto mm = [&](int buf) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[buf][i], bf[buf][j], acc[i][j], 0, 0, 0,
                                                                       as[buf][i], 0, bs[buf][j]);
    };
    issue(kk + 1, nxt);
    __builtin_amdgcn_sched_barrier(0);
    rd(0, 0);
    __builtin_amdgcn_sched_barrier(0);
    rd(1, 1);
    mm(0);
    __builtin_amdgcn_sched_barrier(0);
    mm(1);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) asm volatile("" : "+v"(acc[i][j]));
  };
  issue(0, smem);
  wait_dma();
  settle(smem, 0);
  __syncthreads();
  // the last step runs past kext (MXFP8 fprop with K not a multiple of 128; MXFP4 when the
  // group's K bytes are not a multiple of 128): it is the tail step
  static_assert(!KTAIL || MODE == kModeFprop, "only fprop has a static K tail");
  if constexpr (SC) {
    for (int kk = 0; kk < nk; ++kk) {
      uint8_t* cur = smem + (kk & 1) * S::STAGE;
      uint8_t* nxt = smem + ((kk & 1) ^ 1) * S::STAGE;
      if constexpr (F4) step4(kk, cur, nxt);
      else step8f(kk, cur, nxt);
      wait_dma();  // after the last step: the surplus loads have landed before LDS is reused
      if (kk + 1 < nk) settle(nxt, kk + 1);
      __syncthreads();
    }
  } else {
    const int nfull = KTAIL ? nk - 1 : nk;
    for (int kk = 0; kk < nfull; ++kk) {
      uint8_t* cur = smem + (kk & 1) * S::STAGE;
      uint8_t* nxt = smem + ((kk & 1) ^ 1) * S::STAGE;
      step(BoolC<false>(), kk, cur, nxt);
      if (kk + 1 < nk) {
        wait_dma();
        settle(nxt, kk + 1);
      }
      __syncthreads();
    }
    if constexpr (KTAIL) {  // the tail step (its loads were issued by the step before)
      step(BoolC<true>(), nfull, smem + (nfull & 1) * S::STAGE, smem + ((nfull & 1) ^ 1) * S::STAGE);
      __syncthreads();
    }
  }

  // ---------------- epilogue ----------------
  // Each wave stores its own WM x WN block straight from its accumulator registers: element r of
  // fragment (i, j) of lane (h, l32) is row i*32 + 8(r/4) + 4h + r%4, column j*32 + l32 of the
  // block, so one store instruction writes two row segments of 32 outputs (whole 128-byte lines
  // for fp32; the two halves of a bf16 line come from the fragments j and j + 1 and meet in
  // L2).  No LDS and no wave waits for another.  With accumulation the main_grad values of the
  // next fragment row are in flight while this one is added and stored.  (Staging each fragment
  // row through LDS into 16-byte runs of whole rows was as fast on the 128-expert shapes and
  // 10% slower on the 32-expert Zipf wgrad, whose short tiles make the epilogue a larger share.)
  // Global accesses go through a buffer resource that spans exactly the block's valid rows
  // (from its first column to the end of its last valid row); lanes past the last column get
  // an offset beyond that range.  The hardware drops out-of-range stores and returns zeros for
  // out-of-range loads, so every access is issued unconditionally.
  {
    constexpr int ES = (MODE == kModeFprop && OUT == BSFP8_OUT_BF16) ? 2 : 4;  // output element bytes
    const int64_t row0 = a_row0 + wm * WM;  // first row of this wave's block within the group
    const int64_t col0 = b_row0 + wn * WN;  // first column of the block
    const int64_t left = (MODE == kModeWgrad ? args.M : (int64_t)gi.k) - row0;
    const int vrows = left < 0 ? 0 : (left > WM ? WM : (int)left);  // valid rows of the block
    const int64_t org = (MODE == kModeWgrad ? (int64_t)e * args.M + row0 : gi.off + row0) * args.N + col0;
    const uint32_t nbytes =
        vrows > 0 && col0 < args.N ? (uint32_t)(((int64_t)(vrows - 1) * args.N + args.N - col0) * ES) : 0u;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((uint8_t*)args.out + org * ES, (short)0, (int)nbytes, 0x00020000);
    // byte offsets below WM * N * ES < 2^31 (host bound on N); a lane past the last column starts
    // at 2^31, so all its offsets stay at or above 2^31 > nbytes (and below 2^32)
    uint32_t loff[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j)
      loff[j] = (uint32_t)((4 * h) * args.N + j * 32 + l32) * (uint32_t)ES |
                (col0 + j * 32 + l32 < args.N ? 0u : 0x80000000u);
    auto voff = [&](int i, int j, int r) {
      return loff[j] + (uint32_t)((i * 32 + 8 * (r >> 2) + (r & 3)) * args.N) * (uint32_t)ES;
    };
    auto put = [&](float v, int i, int j, int r) {
      if constexpr (ES == 4) __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(v), rs, (int)voff(i, j, r), 0, 0);
      else __builtin_amdgcn_raw_buffer_store_b16((short)f32_to_bf16(v), rs, (int)voff(i, j, r), 0, 0);
    };
    if constexpr (MODE == kModeWgrad && ACCUM) {
      v16f m[2][FN];
      auto load = [&](int i, v16f* d) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            d[j][r] = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (int)voff(i, j, r), 0, 0));
      };
      load(0, m[0]);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if (i + 1 < FM) load(i + 1, m[(i + 1) & 1]);
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) put(m[i & 1][j][r] + acc[i][j][r], i, j, r);
      }
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) put(acc[i][j][r], i, j, r);
    }
  }
}

// ------------------------------------------------------------------------------------------
// Launchers
// ------------------------------------------------------------------------------------------

template <int MODE, bool PC, int FMT, int BM, int BN, int WM, int WN, bool ACCUM, int OUT, bool KTAIL = false>
static int launch(const GemmArgs& a, dim3 grid, hipStream_t stream) {
  using S = GemmShape<MODE, PC, FMT, BM, BN, WM, WN>;
  hipLaunchKernelGGL((grouped_gemm_kernel<MODE, PC, FMT, BM, BN, WM, WN, ACCUM, OUT, KTAIL>), grid, dim3(S::NT), 0,
                     stream, a);
  return hipGetLastError() == hipSuccess ? BSFP8_OK : BSFP8_ERR_LAUNCH;
}

// Weight-gradient launches with fewer 256 x 256 tiles than this (half the CUs) take 128 x 128
// tiles on the widened MXFP8 path.
constexpr int64_t kSmallWgradTiles = 128;

int launch_grouped_gemm_wgrad(const uint8_t* dy_q, const void* dy_s, int64_t n, const uint8_t* x_q, const void* x_s,
                              int64_t h, const int32_t* splits, int E, int64_t R, int recipe, float* out,
                              int accumulate, uint32_t* status, hipStream_t stream) {
  GemmArgs a{};
  a.a_q = dy_q;
  a.a_s = dy_s;
  a.b_q = x_q;
  a.b_s = x_s;
  a.M = n;
  a.N = h;
  a.R = R;
  a.splits = splits;
  a.E = E;
  a.out = out;
  a.status = status;
  const bool f8 = (recipe & BSFP8_GEMM_FP8_MFMA) != 0;  // MXFP8 on the scaled fp8 MFMA
  recipe &= ~BSFP8_GEMM_FP8_MFMA;
  if (recipe == BSFP8_RECIPE_MX_1X32_E8M0 && !f8 &&
      (int64_t)E * ((n + 255) / 256) * ((h + 255) / 256) < kSmallWgradTiles) {
    // A launch too small to give every CU a 256 x 256 tile (the single-group shape of TE #3484's
    // reproducer has 16) takes 128 x 128 tiles of 4 waves instead: four times the workgroups,
    // two per CU.  Every output sees the same MFMA chain (the same K steps, halves and
    // instructions, at the same place in its 32 x 32 fragment), so the results are the 256 x 256
    // kernel's bit for bit.
    constexpr int BM = 128, BN = 128;
    a.tiles_m = (int)((n + BM - 1) / BM);
    a.tiles_n = (int)((h + BN - 1) / BN);
    a.tiles = (int64_t)E * a.tiles_m * a.tiles_n;
    dim3 grid((unsigned)xcd_launch_size(a.tiles));
    return accumulate ? launch<kModeWgrad, false, kFmtBf16, BM, BN, 64, 64, true, 0>(a, grid, stream)
                      : launch<kModeWgrad, false, kFmtBf16, BM, BN, 64, 64, false, 0>(a, grid, stream);
  }
  if (recipe == BSFP8_RECIPE_MX_1X32_E8M0 || recipe == BSFP8_RECIPE_MXFP4_1X32_E8M0) {
    constexpr int BM = 256, BN = 256;
    a.tiles_m = (int)((n + BM - 1) / BM);
    a.tiles_n = (int)((h + BN - 1) / BN);
    a.tiles = (int64_t)E * a.tiles_m * a.tiles_n;
    if (xcd_launch_size(a.tiles) > 0x7fffffff) return BSFP8_ERR_SHAPE;
    dim3 grid((unsigned)xcd_launch_size(a.tiles));
    if (recipe == BSFP8_RECIPE_MXFP4_1X32_E8M0)
      return accumulate ? launch<kModeWgrad, false, kFmtF4, BM, BN, 128, 64, true, 0>(a, grid, stream)
                        : launch<kModeWgrad, false, kFmtF4, BM, BN, 128, 64, false, 0>(a, grid, stream);
    if (f8)
      return accumulate ? launch<kModeWgrad, false, kFmtF8, BM, BN, 128, 64, true, 0>(a, grid, stream)
                        : launch<kModeWgrad, false, kFmtF8, BM, BN, 128, 64, false, 0>(a, grid, stream);
    return accumulate ? launch<kModeWgrad, false, kFmtBf16, BM, BN, 128, 64, true, 0>(a, grid, stream)
                      : launch<kModeWgrad, false, kFmtBf16, BM, BN, 128, 64, false, 0>(a, grid, stream);
  }
  constexpr int BM = 128, BN = 128;
  a.tiles_m = (int)((n + BM - 1) / BM);
  a.tiles_n = (int)((h + BN - 1) / BN);
  a.tiles = (int64_t)E * a.tiles_m * a.tiles_n;
  if (xcd_launch_size(a.tiles) > 0x7fffffff) return BSFP8_ERR_SHAPE;
  dim3 grid((unsigned)xcd_launch_size(a.tiles));
  return accumulate ? launch<kModeWgrad, true, kFmtBf16, BM, BN, 64, 64, true, 0>(a, grid, stream)
                    : launch<kModeWgrad, true, kFmtBf16, BM, BN, 64, 64, false, 0>(a, grid, stream);
}

// m-grouped GEMM: out[off_e + t][j] = sum_c A[off_e + t][c] B_e[j][c] over the rowwise A
// [R][K] and a per-group B described by its row length and strides (see GemmArgs).  K, b_ld and
// b_estride are in bytes (K elements / 2 for MXFP4); the scale strides count E8M0 bytes.
// fmt: kFmtBf16 (MXFP8, widened), kFmtF4 (MXFP4) or kFmtF8 (MXFP8 on the scaled fp8 MFMA).
static int launch_mgrouped(int fmt, const uint8_t* a_q, const uint8_t* a_s, int64_t R, int64_t K, const uint8_t* b_q,
                           const uint8_t* b_s, int64_t N, int64_t b_ld, int64_t b_estride, int64_t bs_estride,
                           int64_t bs_bstride, const int32_t* splits, int E, void* out, int out_dtype,
                           uint32_t* status, hipStream_t stream) {
  constexpr int BM = 256, BN = 256;
  GemmArgs a{};
  a.a_q = a_q;
  a.a_s = a_s;
  a.b_q = b_q;
  a.b_s = b_s;
  a.N = N;
  a.K = K;
  a.R = R;
  a.b_ld = b_ld;
  a.b_estride = b_estride;
  a.bs_estride = bs_estride;
  a.bs_bstride = bs_bstride;
  a.splits = splits;
  a.E = E;
  a.out = out;
  a.status = status;
  a.tiles_n = (int)((N + BN - 1) / BN);
  // upper bound of sum ceil(k_e / BM) over valid sizes, rounded up to whole runs of m-tiles
  const int64_t gm = fprop_run_mtiles(a.tiles_n);
  const int64_t mt = (R + (int64_t)(BM - 1) * E) / BM;
  if (mt <= 0) return BSFP8_OK;
  a.tiles = (mt + gm - 1) / gm * gm * a.tiles_n;
  if (xcd_launch_size(a.tiles) > 0x7fffffff) return BSFP8_ERR_SHAPE;
  dim3 grid((unsigned)xcd_launch_size(a.tiles));
  if (fmt == kFmtF4)
    return out_dtype == BSFP8_OUT_F32
               ? launch<kModeFprop, false, kFmtF4, BM, BN, 128, 64, false, BSFP8_OUT_F32>(a, grid, stream)
               : launch<kModeFprop, false, kFmtF4, BM, BN, 128, 64, false, BSFP8_OUT_BF16>(a, grid, stream);
  if (fmt == kFmtF8)
    return out_dtype == BSFP8_OUT_F32
               ? launch<kModeFprop, false, kFmtF8, BM, BN, 128, 64, false, BSFP8_OUT_F32>(a, grid, stream)
               : launch<kModeFprop, false, kFmtF8, BM, BN, 128, 64, false, BSFP8_OUT_BF16>(a, grid, stream);
  if (K % 128 != 0)
    return out_dtype == BSFP8_OUT_F32
               ? launch<kModeFprop, false, kFmtBf16, BM, BN, 128, 64, false, BSFP8_OUT_F32, true>(a, grid, stream)
               : launch<kModeFprop, false, kFmtBf16, BM, BN, 128, 64, false, BSFP8_OUT_BF16, true>(a, grid, stream);
  return out_dtype == BSFP8_OUT_F32
             ? launch<kModeFprop, false, kFmtBf16, BM, BN, 128, 64, false, BSFP8_OUT_F32>(a, grid, stream)
             : launch<kModeFprop, false, kFmtBf16, BM, BN, 128, 64, false, BSFP8_OUT_BF16>(a, grid, stream);
}

int launch_grouped_gemm_fprop(const uint8_t* x_q, const uint8_t* x_s, int64_t R, int64_t K, const uint8_t* w_q,
                              const uint8_t* w_s, int64_t N, const int32_t* splits, int E, int recipe, void* out,
                              int out_dtype, uint32_t* status, hipStream_t stream) {
  // W rowwise [E*N][K], scales [K/32][E*N]
  const bool f4 = recipe == BSFP8_RECIPE_MXFP4_1X32_E8M0;
  const int fmt = f4 ? kFmtF4 : (recipe & BSFP8_GEMM_FP8_MFMA) ? kFmtF8 : kFmtBf16;
  const int64_t kb = f4 ? K / 2 : K;  // bytes of a row
  return launch_mgrouped(fmt, x_q, x_s, R, kb, w_q, w_s, N, kb, N * kb, N, (int64_t)E * N, splits, E, out, out_dtype,
                         status, stream);
}

int launch_grouped_gemm_dgrad(const uint8_t* dy_q, const uint8_t* dy_s, int64_t R, int64_t n, const uint8_t* w_q,
                              const void* w_s, int64_t k, const int32_t* splits, int E, int recipe, void* out,
                              int out_dtype, uint32_t* status, hipStream_t stream) {
  // W colwise (group_layout.hpp with split sizes n, ..., n): group e's rows are its k output
  // channels of np = Kp(n) codes each (n along the contraction, pad lanes 0) and it starts at
  // packed row P_e = e * np, so the per-group strides are those of P = np
  const bool f4 = recipe == BSFP8_RECIPE_MXFP4_1X32_E8M0;
  const int fmt = f4 ? kFmtF4 : (recipe & BSFP8_GEMM_FP8_MFMA) ? kFmtF8 : kFmtBf16;
  const int epb = f4 ? 2 : 1;
  const int64_t np = col_padded_rows(n);
  return launch_mgrouped(fmt, dy_q, dy_s, R, n / epb, w_q, (const uint8_t*)w_s, k, col_row_bytes(np, epb),
                         col_group_bytes(k, np, epb), col_e8m0_group(k, np), col_e8m0_block_stride(k), splits, E, out,
                         out_dtype, status, stream);
}

}  // namespace bsfp8

"""The MFMA-only probe (libbsfp8_peak.so) does the work it is credited with: on all-ones operands
every MFMA adds K to each of a lane's 16 accumulators, so each lane's output is
chains x 16 x K x iters, which fixes K (16 for bf16 32x32x16, 64 for the scaled fp8 and fp4
32x32x64) and the number of MFMAs the FLOP count assumes; the clock stamps give a shader clock
within the chip's range.  And the fast reciprocal of the fused SwiGLU equals the IEEE division
for every fp32 in [1, 2^126], the range 1 + 2^x takes there (exhaustive, ~1.06e9 patterns)."""
import ctypes
import os

import pytest
import torch

from gpu_util import DEV, flush

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
WORDS = 8192

# one 32-bit pool word of ones: bf16 1.0 = 0x3F80, e4m3 1.0 = 0x38, e2m1 1.0 = code 2 per nibble
ONES = {1: 0x3F803F80, 2: 0x38383838, 3: 0x22222222}
K = {1: 16, 2: 64, 3: 64}


def _lib():
    L = ctypes.CDLL(os.path.join(ROOT, "block_scaled_fp8_grouped_amd", "libbsfp8_peak.so"))
    L.bsfp8_mfma_peak_probe.restype = ctypes.c_int
    L.bsfp8_mfma_peak_probe.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    L.bsfp8_wall_clock_khz.restype = ctypes.c_int
    L.bsfp8_wall_clock_khz.argtypes = [ctypes.c_int]
    L.bsfp8_mfma_peak_flops.restype = ctypes.c_double
    L.bsfp8_mfma_peak_flops.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64]
    return L


@pytest.mark.parametrize("kind", [1, 2, 3])
def test_probe_counts_its_mfmas(kind):
    flush(f"mfma probe kind={kind}")
    L = _lib()
    blocks, iters = 6, 37
    word = ONES[kind]
    pool = torch.full((WORDS,), word - (1 << 32) if word >= 1 << 31 else word, dtype=torch.int32, device=DEV)
    out = torch.full((blocks * 256,), float("nan"), dtype=torch.float32, device=DEV)
    stamps = torch.zeros(blocks, 4, dtype=torch.int64, device=DEV)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = L.bsfp8_mfma_peak_probe(kind, pool.data_ptr(), out.data_ptr(), blocks, iters, None, s)
    torch.cuda.synchronize()
    assert rc == 0
    assert torch.equal(out, torch.full_like(out, 4 * 16 * K[kind] * iters))
    out.fill_(float("nan"))
    rc = L.bsfp8_mfma_peak_probe(kind, pool.data_ptr(), out.data_ptr(), blocks, 20000, stamps.data_ptr(), s)
    torch.cuda.synchronize()
    assert rc == 0
    assert torch.equal(out, torch.full_like(out, 4 * 16 * K[kind] * 20000))
    st = stamps.cpu().double()
    assert (st[:, 2] > st[:, 0]).all() and (st[:, 3] > st[:, 1]).all()
    khz = L.bsfp8_wall_clock_khz(torch.cuda.current_device())
    assert khz > 0
    ghz = (st[:, 2] - st[:, 0]) / (st[:, 3] - st[:, 1]) * khz / 1e6
    flush(f"probe kind={kind}: wall clock {khz} kHz, shader clock {ghz.median().item():.3f} GHz")
    assert 0.3 < ghz.median().item() < 3.0
    # the credited FLOPs: 2 * 32 * 32 * K per MFMA, 4 chains per iteration, 4 waves per workgroup
    assert L.bsfp8_mfma_peak_flops(kind, blocks, iters) == 2 * 32 * 32 * K[kind] * 4 * iters * 4 * blocks


def test_recip_equals_ieee_division_on_its_domain():
    flush("recip check")
    L = _lib()
    L.bsfp8_recip_check.restype = ctypes.c_int
    L.bsfp8_recip_check.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p]
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for lo, hi, expect_exact in ((0x3F800000, 0x7E800001, True),   # [1, 2^126]
                                 (0x7E800001, 0x7E800101, False)):  # just above: subnormal 1/d
        mism = torch.zeros(1, dtype=torch.int64, device=DEV)
        first = torch.full((1,), -1, dtype=torch.int32, device=DEV)
        assert L.bsfp8_recip_check(lo, hi, mism.data_ptr(), first.data_ptr(), s) == 0
        torch.cuda.synchronize()
        n = int(mism.item())
        flush(f"recip [{lo:#x}, {hi:#x}): {n} mismatches")
        if expect_exact:
            assert n == 0, f"first mismatch {int(first.item()) & 0xFFFFFFFF:#x}"
        else:
            assert n > 0  # the check does see a difference where there is one


def test_bf16_output_conversion_is_round_to_nearest_even():
    """The GEMMs' bf16 outputs go through the hardware fp32 -> bf16 conversion: over all 2^32 fp32
    patterns it equals an integer round-to-nearest-even of the fp32 bits (NaN stays NaN), and the
    same check against truncation does report differences."""
    flush("bf16 conversion check")
    L = _lib()
    L.bsfp8_bf16_cvt_check.restype = ctypes.c_int
    L.bsfp8_bf16_cvt_check.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p]
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for mode, ranges in ((0, ((0, 0x80000000), (0x80000000, 0xFFFFFFFF), (0xFFFFFFFE, 0xFFFFFFFF))),
                         (1, ((0x3F800000, 0x3F810000),))):
        mism = torch.zeros(1, dtype=torch.int64, device=DEV)
        first = torch.full((1,), -1, dtype=torch.int32, device=DEV)
        for lo, hi in ranges:
            assert L.bsfp8_bf16_cvt_check(lo, hi, mode, mism.data_ptr(), first.data_ptr(), s) == 0
        torch.cuda.synchronize()
        n = int(mism.item())
        flush(f"bf16 conversion, mode {mode}: {n} mismatches")
        if mode == 0:
            assert n == 0, f"first mismatch {int(first.item()) & 0xFFFFFFFF:#x}"
        else:
            assert n > 0  # truncation differs from rounding on about half of the patterns


def test_lds_dma_probe_moves_the_named_bytes():
    """The global -> LDS DMA probe (bench.py's operand-delivery reference) moves exactly the bytes
    its header names: each lane's XOR of the 8 x 16 bytes of its last round, read back from LDS,
    equals the XOR of those source bytes computed on the host (private and shared sources)."""
    import numpy as np
    L = _lib()
    L.bsfp8_lds_dma_probe.restype = ctypes.c_int
    L.bsfp8_lds_dma_probe.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                      ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    blocks, waves, rounds, span = 6, 8, 5, 24 * 1024
    g = torch.Generator(device=DEV).manual_seed(11)
    src = torch.randint(0, 256, (blocks * span,), dtype=torch.uint8, device=DEV, generator=g)
    host = src.cpu().numpy().view(np.uint32)
    for shared in (0, 1):
        flush(f"lds dma probe shared={shared}")
        out = torch.zeros(blocks * 64 * waves, dtype=torch.int32, device=DEV)
        assert L.bsfp8_lds_dma_probe(src.data_ptr(), span, shared, blocks, waves, rounds, out.data_ptr(), s) == 0
        torch.cuda.synchronize()
        got = out.cpu().numpy().view(np.uint32)
        r = rounds - 1
        exp = np.zeros_like(got)
        for b in range(blocks):
            base = 0 if shared else b * span
            for t in range(64 * waves):
                w, l = divmod(t, 64)
                x = np.uint32(0)
                for u in range(8):
                    o = (r * waves * 8192 + w * 8192 + u * 1024 + 16 * l) % span
                    x ^= np.bitwise_xor.reduce(host[(base + o) // 4:(base + o) // 4 + 4])
                exp[b * 64 * waves + t] = x
        assert np.array_equal(got, exp)

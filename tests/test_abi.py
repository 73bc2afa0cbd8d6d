"""C-ABI checks that need no GPU: every function declared in include/bsfp8.h is exported by
libbsfp8.so (and those of include/bsfp8_peak.h by the probe library libbsfp8_peak.so), the size
queries follow their documented formulas, and every host-checkable error is returned before the
library touches a pointer or makes a HIP call (the fake pointers used below are never
dereferenced)."""
import ctypes
import os
import re

import pytest

import block_scaled_fp8_grouped_amd as bs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "bsfp8.h")

P = 1 << 20  # a fake, 16-byte-aligned device address; never dereferenced by these calls
MX, PC, MX4 = bs.RECIPE_MX, bs.RECIPE_PC, bs.RECIPE_MX4


def _declared(hdr=HDR):
    text = open(hdr).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsfp8_\w+)\s*\(", text)))


def _hdr_consts():
    text = open(HDR).read()
    return {k: int(v.strip("()")) for k, v in re.findall(r"#define\s+(BSFP8_\w+)\s+(\(?-?\d+\)?)u?\b", text)}


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) >= 9
    L = bs.lib()
    for n in names:
        assert hasattr(L, n), n


def _peak_lib():
    L = ctypes.CDLL(os.path.join(ROOT, "block_scaled_fp8_grouped_amd", "libbsfp8_peak.so"))
    L.bsfp8_mfma_peak_probe.restype = ctypes.c_int
    L.bsfp8_mfma_peak_probe.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    L.bsfp8_mfma_peak_flops.restype = ctypes.c_double
    L.bsfp8_mfma_peak_flops.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64]
    return L


def test_probe_library_exports_and_rejects_before_launch():
    L = _peak_lib()
    names = _declared(os.path.join(ROOT, "include", "bsfp8_peak.h"))
    assert names == ["bsfp8_bf16_cvt_check", "bsfp8_lds_dma_probe", "bsfp8_mfma_dot_probe", "bsfp8_mfma_peak_flops", "bsfp8_mfma_peak_probe",
                     "bsfp8_recip_check", "bsfp8_wall_clock_khz"]
    for n in names:
        assert hasattr(L, n), n
    def probe(kind, pool, out, blocks, iters):
        return L.bsfp8_mfma_peak_probe(kind, pool, out, blocks, iters, None, None)
    assert probe(1, None, P, 512, 10) == -1 and probe(1, P, None, 512, 10) == -1
    assert probe(0, P, P, 512, 10) == -2 and probe(4, P, P, 512, 10) == -2
    assert probe(1, P, P, 0, 10) == -3 and probe(1, P, P, 65537, 10) == -3
    assert probe(1, P, P, 512, 0) == -3 and probe(1, P, P, 512, (1 << 31) + 1) == -3
    # 2 M N K per MFMA x 4 chains x 4 waves per workgroup
    assert L.bsfp8_mfma_peak_flops(1, 512, 10) == 2 * 32 * 32 * 16 * 4 * 4 * 512 * 10
    assert L.bsfp8_mfma_peak_flops(3, 3, 7) == 2 * 32 * 32 * 64 * 4 * 4 * 3 * 7
    assert L.bsfp8_mfma_peak_flops(5, 3, 7) == 0.0
    L.bsfp8_recip_check.restype = ctypes.c_int
    L.bsfp8_recip_check.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    assert L.bsfp8_recip_check(1, 5, None, P, None) == -1 and L.bsfp8_recip_check(1, 5, P, None, None) == -1
    assert L.bsfp8_recip_check(5, 5, P, P, None) == -3 and L.bsfp8_recip_check(6, 5, P, P, None) == -3
    L.bsfp8_bf16_cvt_check.restype = ctypes.c_int
    L.bsfp8_bf16_cvt_check.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p]
    assert L.bsfp8_bf16_cvt_check(1, 5, 0, None, P, None) == -1 and L.bsfp8_bf16_cvt_check(1, 5, 0, P, None, None) == -1
    assert L.bsfp8_bf16_cvt_check(1, 5, 2, P, P, None) == -2 and L.bsfp8_bf16_cvt_check(5, 5, 0, P, P, None) == -3
    L.bsfp8_mfma_dot_probe.restype = ctypes.c_int
    L.bsfp8_mfma_dot_probe.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]

    def dot(kind=1, aq=P, as_=P, bq=P, bs_=P, k=128, out=P):
        return L.bsfp8_mfma_dot_probe(kind, aq, as_, bq, bs_, k, out, None)
    for i in range(5):
        args = [P] * 5
        args[i] = None
        assert dot(1, args[0], args[1], args[2], args[3], 128, args[4]) == -1
    assert dot(kind=0) == -2 and dot(kind=5) == -2
    assert dot(k=64) == -3 and dot(k=192) == -3 and dot(k=65536 + 128) == -3
    assert dot(aq=P + 16) == -5 and dot(bq=P + 8) == -5
    L.bsfp8_lds_dma_probe.restype = ctypes.c_int
    L.bsfp8_lds_dma_probe.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                      ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]

    def dma(src=P, span=65536, shared=0, blocks=256, waves=8, rounds=10, out=P):
        return L.bsfp8_lds_dma_probe(src, span, shared, blocks, waves, rounds, out, None)
    assert dma(src=None) == -1 and dma(out=None) == -1
    assert dma(span=4096) == -3 and dma(span=65536 + 512) == -3 and dma(span=(1 << 31) + 1024) == -3
    assert dma(blocks=0) == -3 and dma(blocks=4097) == -3 and dma(waves=0) == -3 and dma(waves=9) == -3
    assert dma(rounds=0) == -3 and dma(rounds=100001) == -3


def test_binding_constants_match_header():
    c = _hdr_consts()
    assert c["BSFP8_RECIPE_MX_1X32_E8M0"] == bs.RECIPE_MX and c["BSFP8_RECIPE_PER_CHANNEL_128_F32"] == bs.RECIPE_PC
    assert c["BSFP8_RECIPE_MXFP4_1X32_E8M0"] == bs.RECIPE_MX4
    text = open(HDR).read()
    assert "#define BSFP8_GEMM_FP8_MFMA 0x100" in text and bs.GEMM_FP8_MFMA == 0x100
    assert c["BSFP8_ROWWISE"] == bs.ROWWISE and c["BSFP8_COLWISE"] == bs.COLWISE
    assert c["BSFP8_OUT_F32"] == bs.OUT_F32 and c["BSFP8_OUT_BF16"] == bs.OUT_BF16
    assert c["BSFP8_MAX_GROUPS"] == bs.MAX_GROUPS


def test_size_queries():
    for R, E in [(1024, 4), (768, 4), (0, 1), (65664, 32), (1048576, 128), (5, 1024)]:
        rb = 128 * ((R + 127 * E) // 128)
        assert bs.colwise_rows_bound(R, E) == rb
        assert bs.colwise_data_bytes(R, 256, E) == rb * 256
        assert bs.colwise_data_bytes(R, 256, E, PC) == rb * 256
        assert bs.colwise_data_bytes(R, 256, E, MX4) == rb * 128
        assert bs.colwise_scale_bytes(R, 256, E, MX) == rb // 32 * 256
        assert bs.colwise_scale_bytes(R, 256, E, MX4) == rb // 32 * 256
        assert bs.colwise_scale_bytes(R, 256, E, PC) == rb // 128 * 256 * 4
    # the bound covers the worst case of any valid split
    for R, E in [(1000, 7), (129, 2), (1, 1)]:
        worst = sum(128 * ((k + 127) // 128) for k in [R - (E - 1)] + [1] * (E - 1))
        assert worst <= bs.colwise_rows_bound(R, E)
    assert bs.rowwise_data_bytes(10, 64) == 640 and bs.rowwise_scale_bytes(10, 64) == 20
    assert bs.rowwise_data_bytes(10, 64, MX4) == 320 and bs.rowwise_data_bytes(10, 64, PC) == 0
    assert bs.colwise_data_bytes(10, 33, 1) == 0 and bs.colwise_rows_bound(10, 0) == 0
    assert bs.colwise_scale_bytes(10, 64, 1, 7) == 0 and bs.colwise_data_bytes(10, 64, 1, 7) == 0


def _q(**kw):
    a = dict(inp=P, R=1024, C=256, splits=P, E=4, recipe=MX, which=bs.COLWISE, zas=1e-30, row_q=P, row_s=P,
             col_q=P, col_s=P, noop=None, status=P, stream=None)
    a.update(kw)
    return bs.lib().bsfp8_grouped_quantize(a["inp"], a["R"], a["C"], a["splits"], a["E"], a["recipe"], a["which"],
                                           a["zas"], a["row_q"], a["row_s"], a["col_q"], a["col_s"], a["noop"],
                                           a["status"], a["stream"])


def _w(**kw):
    a = dict(dyq=P, dys=P, n=256, xq=P, xs=P, h=256, splits=P, E=4, R=1024, recipe=MX, out=P, acc=0, status=P)
    a.update(kw)
    return bs.lib().bsfp8_grouped_gemm_wgrad(a["dyq"], a["dys"], a["n"], a["xq"], a["xs"], a["h"], a["splits"],
                                             a["E"], a["R"], a["recipe"], a["out"], a["acc"], a["status"], None)


def _f(**kw):
    a = dict(xq=P, xs=P, R=1024, k=256, wq=P, ws=P, n=256, splits=P, E=4, recipe=MX, out=P, dtype=bs.OUT_F32,
             status=P)
    a.update(kw)
    return bs.lib().bsfp8_grouped_gemm_fprop(a["xq"], a["xs"], a["R"], a["k"], a["wq"], a["ws"], a["n"],
                                             a["splits"], a["E"], a["recipe"], a["out"], a["dtype"], a["status"],
                                             None)


@pytest.mark.parametrize("kw,code", [
    (dict(recipe=0), -3), (dict(recipe=4), -3), (dict(recipe=MX | 0x100), -3),
    (dict(which=0), -7), (dict(which=4), -7),
    (dict(which=bs.ROWWISE, recipe=PC), -6), (dict(which=bs.ROWWISE | bs.COLWISE, recipe=PC), -6),
    (dict(C=33), -4), (dict(C=0), -4), (dict(R=-1), -4),
    (dict(recipe=PC, zas=float("nan")), -7), (dict(recipe=PC, zas=-1.0), -7), (dict(recipe=PC, zas=float("inf")), -7),
    (dict(splits=None), -1),
    (dict(E=0), -2), (dict(E=1025), -2),
    (dict(inp=None), -1), (dict(col_q=None), -1), (dict(col_s=None), -1),
    (dict(which=bs.ROWWISE | bs.COLWISE, row_q=None), -1),
    (dict(inp=P + 8), -5), (dict(col_q=P + 4), -5), (dict(splits=P + 2), -5), (dict(status=P + 1), -5),
    (dict(noop=P + 2), -5),
])
def test_quantize_rejects_before_launch(kw, code):
    assert _q(**kw) == code


def test_quantize_zero_rows_returns_without_touching_pointers():
    assert _q(R=0, inp=None, col_q=None, col_s=None) == 0
    assert _q(R=0, which=bs.ROWWISE, splits=None, inp=None, row_q=None, row_s=None) == 0
    assert _q(R=0, inp=None, col_q=None, col_s=None, noop=P + 2) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(recipe=5), -3), (dict(recipe=PC | 0x100), -3), (dict(recipe=MX4 | 0x100), -3), (dict(recipe=0x100), -3),
    (dict(E=0), -2), (dict(E=2000), -2),
    (dict(n=100), -4), (dict(h=0), -4), (dict(R=-5), -4),
    (dict(acc=2), -7), (dict(R=(1 << 24)), -4), (dict(h=(1 << 21) + 32), -4),
    (dict(splits=None), -1), (dict(out=None), -1), (dict(dyq=None), -1), (dict(xs=None), -1),
    (dict(out=P + 4), -5), (dict(dys=P + 1), -5), (dict(splits=P + 2), -5),
])
def test_wgrad_rejects_before_launch(kw, code):
    assert _w(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(E=0), -2), (dict(k=48), -4), (dict(n=-32), -4), (dict(dtype=2), -7), (dict(k=1 << 24), -4),
    (dict(n=(1 << 21) + 32), -4), (dict(recipe=PC), -3), (dict(recipe=0), -3), (dict(recipe=4), -3),
    (dict(recipe=MX4 | 0x100), -3), (dict(recipe=0x100), -3),
    (dict(xq=None), -1), (dict(ws=None), -1), (dict(splits=None), -1), (dict(out=None), -1),
    (dict(out=P + 2), -5), (dict(wq=P + 8), -5),
])
def test_fprop_rejects_before_launch(kw, code):
    assert _f(**kw) == code


def _d(**kw):
    a = dict(yq=P, ys=P, R=1024, n=256, wq=P, ws=P, k=256, splits=P, E=4, recipe=MX, out=P, dtype=bs.OUT_F32,
             status=P)
    a.update(kw)
    return bs.lib().bsfp8_grouped_gemm_dgrad(a["yq"], a["ys"], a["R"], a["n"], a["wq"], a["ws"], a["k"],
                                             a["splits"], a["E"], a["recipe"], a["out"], a["dtype"], a["status"],
                                             None)


@pytest.mark.parametrize("kw,code", [
    (dict(E=0), -2), (dict(E=2000), -2), (dict(n=48), -4), (dict(k=-32), -4), (dict(k=(1 << 21) + 32), -4),
    (dict(n=(1 << 24) - 224), -4), (dict(dtype=2), -7), (dict(R=-1), -4), (dict(recipe=PC), -3),
    (dict(recipe=PC | 0x100), -3), (dict(recipe=MX4 | 0x100), -3),
    (dict(yq=None), -1), (dict(ws=None), -1), (dict(splits=None), -1), (dict(out=None), -1),
    (dict(out=P + 2), -5), (dict(wq=P + 8), -5), (dict(ys=P + 1), -5),
])
def test_dgrad_rejects_before_launch(kw, code):
    assert _d(**kw) == code


def test_dgrad_zero_rows_returns_without_touching_pointers():
    assert _d(R=0, yq=None, ys=None, wq=None, ws=None, splits=None, out=None) == 0


def test_fprop_zero_rows_early_return():
    """TE PR #3224: a zero-row batch returns before any data pointer is used."""
    assert _f(R=0, xq=None, xs=None, wq=None, ws=None, splits=None, out=None) == 0


def _a(**kw):
    a = dict(act=bs.ACT_SRELU, h=P, probs=P, dy=None, R=1024, C=256, splits=P, E=4, recipe=MX, which=bs.COLWISE,
             row_q=P, row_s=P, col_q=P, col_s=P, status=P)
    a.update(kw)
    return bs.lib().bsfp8_grouped_act_quantize(a["act"], a["h"], a["probs"], a["dy"], a["R"], a["C"], a["splits"],
                                               a["E"], a["recipe"], a["which"], a["row_q"], a["row_s"], a["col_q"],
                                               a["col_s"], a["status"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(act=0), -7), (dict(act=5), -7), (dict(recipe=PC), -6), (dict(recipe=9), -3),
    (dict(which=0), -7), (dict(which=8), -7), (dict(C=48), -4), (dict(R=-1), -4),
    (dict(splits=None), -1), (dict(E=0), -2), (dict(E=1025), -2),
    (dict(h=None), -1), (dict(act=bs.ACT_SRELU_GRAD), -1), (dict(col_s=None), -1),
    (dict(which=bs.ROWWISE, row_q=None), -1),
    (dict(h=P + 8), -5), (dict(act=bs.ACT_SRELU_GRAD, dy=P + 2), -5), (dict(probs=P + 2), -5),
    (dict(col_q=P + 4), -5), (dict(status=P + 1), -5),
    (dict(act=bs.ACT_SWIGLU, C=48), -4), (dict(act=bs.ACT_SWIGLU, recipe=PC), -6),
    (dict(act=bs.ACT_SWIGLU_GRAD), -1), (dict(act=bs.ACT_SWIGLU_GRAD, dy=P + 2), -5),
])
def test_act_quantize_rejects_before_launch(kw, code):
    assert _a(**kw) == code


def test_act_quantize_zero_rows_and_optional_probs():
    assert _a(R=0, h=None, probs=None, col_q=None, col_s=None) == 0
    assert _a(R=0, act=bs.ACT_SRELU_GRAD, h=None, dy=None, col_q=None, col_s=None) == 0
    assert _a(R=0, act=bs.ACT_SWIGLU_GRAD, h=None, dy=None, col_q=None, col_s=None) == 0


def test_strerror_covers_codes():
    for c in range(-8, 1):
        assert bs.strerror(c) != "unknown error code"
    assert bs.strerror(-99) == "unknown error code"

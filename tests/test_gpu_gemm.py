"""GPU grouped wgrad / fprop vs the fp64 CPU oracle on the same quantized inputs.

* wgrad: per-expert relative Frobenius error <= 1e-5; empty experts exactly zero (store) or
  bitwise untouched (accumulate); an all-zero dy channel gives an exact zero output row.
* fprop: fp32 per-expert relative Frobenius error <= 1e-5; bf16 within one bf16 ulp of the
  oracle rounded to bf16 plus 1e-5 of the expert's rms output (fp32 accumulation error on
  cancelling sums); rows past sum(split_sizes) untouched.
* padding invariance (TE #3484 expected behaviour): capacity tails of 0.0, 3.0 or random bits
  give results bitwise equal to the unpadded run.
* device status word: a negative size or sum(k_e) > capacity sets its bit and nothing is written.
Tiles: n/h/N not multiples of 256 (partial tiles; output widths of 96 leave a wave's second
32-column fragment past the last column) and K not a multiple of 128 (fprop tail).
"""
import numpy as np
import pytest
import torch

import block_scaled_fp8_grouped_amd as bs
import oracle
import workloads as W
from gpu_util import (DEV, REL_TOL, assert_bf16_close, assert_quant_matches, flush, gpu_quantize, rel_err)

pytestmark = pytest.mark.gpu


def _operands(R, n, h, splits, seed, fill="garbage", scale=1.0):
    g = torch.Generator(device=DEV).manual_seed(seed)
    dy = W.randn_bf16((R, n), g, DEV, scale)
    x = W.randn_bf16((R, h), g, DEV, scale)
    T = sum(splits)
    if R > T:
        for t in (dy, x):
            if fill == "garbage":
                rng = np.random.default_rng(seed)
                bits = rng.integers(0, 1 << 16, size=(R - T, t.shape[1]), dtype=np.uint16)
                t[T:] = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
            else:
                t[T:] = fill
    return dy, x


def run_wgrad(dy, x, splits, recipe, accumulate=False, mg=None, zas=1e-30, status=None):
    R, n = dy.shape
    h = x.shape[1]
    E = len(splits)
    st = W.splits_tensor(splits, DEV)
    own = status is None
    if own:
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
    dq = gpu_quantize(dy, splits, recipe, bs.COLWISE, zas, status=status)
    xq = gpu_quantize(x, splits, recipe, bs.COLWISE, zas, status=status)
    out = mg.clone() if accumulate else torch.full((E, n, h), float("nan"), dtype=torch.float32, device=DEV)
    bs.grouped_gemm_wgrad(dq, n, xq, h, st, R, recipe, out, accumulate=accumulate, status=status)
    if own:
        torch.cuda.synchronize()
        assert int(status.item()) == 0
    return out, dq, xq


def check_wgrad(dy, x, splits, recipe, accumulate=False, mg=None, zas=1e-30, rows_sel=None, label=""):
    R, n = dy.shape
    h = x.shape[1]
    out, dq, xq = run_wgrad(dy, x, splits, recipe, accumulate, mg, zas)
    torch.cuda.synchronize()
    o_dy = oracle.grouped_quantize(W.bf16_bits(dy), splits, recipe, oracle.COLWISE, zas)
    o_x = oracle.grouped_quantize(W.bf16_bits(x), splits, recipe, oracle.COLWISE, zas)
    assert_quant_matches(dq, o_dy, splits, R, bs.COLWISE, label + " dy")
    assert_quant_matches(xq, o_x, splits, R, bs.COLWISE, label + " x")
    sel = np.arange(n, dtype=np.int32) if rows_sel is None else np.asarray(rows_sel, np.int32)
    ref = oracle.grouped_wgrad(o_dy["col_q"], o_dy["col_s"], n, o_x["col_q"], o_x["col_s"], h, splits, R, recipe,
                               rows_sel=sel)
    got = out.cpu().numpy()[:, sel, :].astype(np.float64)
    mg_h = None if mg is None else mg.cpu().numpy()[:, sel, :].astype(np.float64)
    for e, k in enumerate(splits):
        if k == 0:
            if accumulate:
                assert torch.equal(out[e].view(torch.int32), mg[e].view(torch.int32)), f"{label} expert {e}: main_grad touched"
            else:
                assert (out[e] == 0).all(), f"{label} empty expert {e} not zero"
            continue
        part = got[e] - mg_h[e] if accumulate else got[e]
        r = rel_err(part, ref[e])
        assert r <= REL_TOL, f"{label} expert {e} (k={k}): rel {r:.3e}"
    return out


# ------------------------------------------------------------------------------------------
# wgrad
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("recipe", [bs.RECIPE_MX, bs.RECIPE_PC])
@pytest.mark.parametrize("n,h", [(256, 256), (96, 320), (512, 64), (64, 96)])
@pytest.mark.parametrize("splits", [[0, 1, 31, 32, 33, 127, 128, 129, 256], [300, 0, 45, 1, 200], [1000]])
def test_wgrad_store_parity(recipe, n, h, splits):
    flush(f"wgrad store recipe={recipe} n={n} h={h} splits={splits}")
    R = sum(splits) + 50
    dy, x = _operands(R, n, h, splits, seed=n + h)
    check_wgrad(dy, x, splits, recipe, label=f"r{recipe} {n}x{h}")


@pytest.mark.parametrize("recipe", [bs.RECIPE_MX, bs.RECIPE_PC])
def test_wgrad_accumulate_parity_and_empty_untouched(recipe):
    splits = [0, 200, 0, 129, 64]
    R = sum(splits) + 128
    n, h = 128, 288
    flush(f"wgrad accumulate recipe={recipe}")
    dy, x = _operands(R, n, h, splits, seed=5)
    g = torch.Generator(device=DEV).manual_seed(6)
    mg = torch.randn(len(splits), n, h, dtype=torch.float32, device=DEV, generator=g)
    check_wgrad(dy, x, splits, recipe, accumulate=True, mg=mg, label=f"acc r{recipe}")


@pytest.mark.parametrize("recipe", [bs.RECIPE_MX, bs.RECIPE_PC])
def test_wgrad_skewed_split_many_tiles(recipe):
    """A skewed split (largest group above twice the mean non-empty size) over more tiles than
    one round of 256 workgroups: the kernel takes its groups largest first and deals the tiles
    to the XCDs in short runs; every expert is checked against the oracle."""
    rng = np.random.default_rng(11)
    splits = [int(c) for c in W.zipf_counts(rng, 40, 36, 7000)]
    live = [k for k in splits if k > 0]
    assert max(live) * len(live) > 2 * sum(live), splits  # the kernel's skew condition
    n, h = 512, 1024
    tiles = len(splits) * (n // 256) * (h // 256) if recipe == bs.RECIPE_MX else len(splits) * (n // 128) * (h // 128)
    assert tiles > 256
    flush(f"wgrad skewed recipe={recipe} splits={splits}")
    R = sum(splits) + 77
    dy, x = _operands(R, n, h, splits, seed=12)
    check_wgrad(dy, x, splits, recipe, label=f"skewed r{recipe}")


def test_wgrad_zero_channel_gives_zero_row():
    """DeepGEMM #365 structure: one all-zero dy channel in each 128-token expert."""
    case = W.deepgemm_case(DEV, 256, 256, R=1024)
    out = check_wgrad(case["dy"], case["x"], case["splits"], bs.RECIPE_PC, label="dg365")
    o = out.cpu()
    for e, k in enumerate(case["splits"]):
        if k == 128:
            assert (o[e, 0] == 0).all()
        else:
            assert (o[e, 0] != 0).all()


@pytest.mark.parametrize("fill", [0.0, 3.0, "garbage"])
@pytest.mark.parametrize("recipe", [bs.RECIPE_MX, bs.RECIPE_PC])
def test_wgrad_padding_bitwise_invariant(fill, recipe):
    splits = [77, 0, 300, 128]
    T = sum(splits)
    n, h = 160, 256
    dy0, x0 = _operands(T, n, h, splits, seed=11)
    ref, _, _ = run_wgrad(dy0, x0, splits, recipe)
    dy = torch.empty(T + 300, n, dtype=torch.bfloat16, device=DEV)
    x = torch.empty(T + 300, h, dtype=torch.bfloat16, device=DEV)
    dy[:T], x[:T] = dy0, x0
    if fill == "garbage":
        rng = np.random.default_rng(3)
        for t in (dy, x):
            bits = rng.integers(0, 1 << 16, size=(300, t.shape[1]), dtype=np.uint16)
            t[T:] = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    else:
        dy[T:], x[T:] = fill, fill
    got, _, _ = run_wgrad(dy, x, splits, recipe)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32))


@pytest.mark.parametrize("E", [1, 2, 4, 32, 128])
def test_wgrad_edge_matrix(E):
    rng = np.random.default_rng(E)
    edge = [0, 1, 31, 32, 33, 127, 128, 129, 256]
    splits = [int(edge[i % len(edge)]) if i % 3 else int(rng.integers(0, 300)) for i in range(E)]
    if E == 1:
        splits = [129]
    T = sum(splits)
    n, h = 64, 96
    for fill in (None, 0.0, "garbage"):
        R = T if fill is None else T + 96
        dy, x = _operands(R, n, h, splits, seed=E, fill=fill if fill is not None else 0.0)
        for recipe in (bs.RECIPE_MX, bs.RECIPE_PC):
            for acc in (False, True):
                flush(f"edge E={E} fill={fill} recipe={recipe} acc={acc}")
                mg = torch.randn(E, n, h, dtype=torch.float32, device=DEV) if acc else None
                check_wgrad(dy, x, splits, recipe, accumulate=acc, mg=mg, label=f"E={E} {fill} r{recipe} a{acc}")


def test_wgrad_zero_capacity_store_zero_fills():
    """All groups empty (capacity 0): store mode writes zeros, accumulate leaves out untouched."""
    E, n, h = 3, 64, 64
    st = W.splits_tensor([0, 0, 0], DEV)
    empty = {"col_q": torch.empty(0, dtype=torch.uint8, device=DEV), "col_s": torch.empty(0, dtype=torch.uint8, device=DEV)}
    out = torch.full((E, n, h), 7.0, device=DEV)
    bs.grouped_gemm_wgrad(empty, n, empty, h, st, 0, bs.RECIPE_MX, out)
    torch.cuda.synchronize()
    assert (out == 0).all()
    out.fill_(7.0)
    bs.grouped_gemm_wgrad(empty, n, empty, h, st, 0, bs.RECIPE_MX, out, accumulate=True)
    torch.cuda.synchronize()
    assert (out == 7.0).all()


# ------------------------------------------------------------------------------------------
# fprop
# ------------------------------------------------------------------------------------------

def run_fprop(x, w, splits, N, out_dtype, status=None):
    R, K = x.shape
    E = len(splits)
    st = W.splits_tensor(splits, DEV)
    xq = gpu_quantize(x, splits, bs.RECIPE_MX, bs.ROWWISE, status=status)
    wq = gpu_quantize(w, None, bs.RECIPE_MX, bs.ROWWISE)
    dt = torch.float32 if out_dtype == bs.OUT_F32 else torch.bfloat16
    out = torch.full((R, N), float("nan"), dtype=dt, device=DEV)
    bs.grouped_gemm_fprop(xq, K, wq, N, st, R, out, out_dtype, status=status)
    return out, xq, wq


def check_fprop(x, w, splits, N, out_dtype, cols_sel=None, label=""):
    R, K = x.shape
    T = sum(splits)
    out, xq, wq = run_fprop(x, w, splits, N, out_dtype)
    torch.cuda.synchronize()
    o_x = oracle.grouped_quantize(W.bf16_bits(x), splits, oracle.RECIPE_MX, oracle.ROWWISE)
    o_w = oracle.grouped_quantize(W.bf16_bits(w), None, oracle.RECIPE_MX, oracle.ROWWISE)
    assert_quant_matches(xq, o_x, splits, R, bs.ROWWISE, label + " x")
    assert_quant_matches(wq, o_w, None, w.shape[0], bs.ROWWISE, label + " w")
    sel = np.arange(N, dtype=np.int32) if cols_sel is None else np.asarray(cols_sel, np.int32)
    ref = oracle.grouped_fprop(o_x["row_q"], o_x["row_s"], o_w["row_q"], o_w["row_s"], N, splits, cols_sel=sel)
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.isnan(got[T:]).all(), f"{label}: rows past the live rows were written"
    got = got[:, sel]
    off = 0
    for e, k in enumerate(splits):
        if k:
            g_e, r_e = got[off:off + k], ref[off:off + k]
            if out_dtype == bs.OUT_F32:
                r = rel_err(g_e, r_e)
                assert r <= REL_TOL, f"{label} expert {e}: rel {r:.3e}"
            else:
                assert_bf16_close(g_e, r_e, f"{label} expert {e}")
        off += k
    return out


@pytest.mark.parametrize("out_dtype", [bs.OUT_F32, bs.OUT_BF16])
@pytest.mark.parametrize("K,N", [(256, 256), (96, 320), (160, 64), (512, 512), (256, 96)])
@pytest.mark.parametrize("splits", [[0, 1, 31, 32, 33, 127, 128, 129, 256], [300, 0, 45, 1, 200], [600]])
def test_fprop_parity(out_dtype, K, N, splits):
    flush(f"fprop dtype={out_dtype} K={K} N={N} splits={splits}")
    T = sum(splits)
    R = T + 64
    g = torch.Generator(device=DEV).manual_seed(K + N)
    x = W.randn_bf16((R, K), g, DEV)
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 16, size=(R - T, K), dtype=np.uint16)
    x[T:] = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    w = W.randn_bf16((len(splits) * N, K), g, DEV)
    check_fprop(x, w, splits, N, out_dtype, label=f"K={K} N={N}")


def test_fprop_padding_bitwise_invariant():
    splits = [70, 0, 333]
    T, K, N = sum(splits), 256, 128
    g = torch.Generator(device=DEV).manual_seed(2)
    x0 = W.randn_bf16((T, K), g, DEV)
    w = W.randn_bf16((3 * N, K), g, DEV)
    ref, _, _ = run_fprop(x0, w, splits, N, bs.OUT_F32)
    for fill in (0.0, 3.0, "garbage"):
        x = torch.empty(T + 200, K, dtype=torch.bfloat16, device=DEV)
        x[:T] = x0
        if fill == "garbage":
            bits = np.random.default_rng(4).integers(0, 1 << 16, size=(200, K), dtype=np.uint16)
            x[T:] = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
        else:
            x[T:] = fill
        got, _, _ = run_fprop(x, w, splits, N, bs.OUT_F32)
        torch.cuda.synchronize()
        assert torch.equal(got[:T].view(torch.int32), ref[:T].view(torch.int32)), fill
        assert torch.isnan(got[T:]).all()


# ------------------------------------------------------------------------------------------
# device status word
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("splits,R,bit", [([100, -5, 50], 400, bs.STATUS_NEGATIVE_SPLIT),
                                          ([200, 100, 50], 300, bs.STATUS_EXCEEDS_CAPACITY)])
def test_status_bits_and_no_writes(splits, R, bit):
    n = h = 64
    E = len(splits)
    st = W.splits_tensor(splits, DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(0)
    x = W.randn_bf16((R, h), g, DEV)
    q = {}
    for recipe, which in ((bs.RECIPE_MX, bs.COLWISE | bs.ROWWISE), (bs.RECIPE_PC, bs.COLWISE)):
        out = bs.alloc_quantized(R, h, E, recipe, which, DEV)
        for t in out.values():
            t.view(torch.uint8).fill_(0xFF)
        bs.grouped_quantize(x, st, recipe, which, out, status=status)
        torch.cuda.synchronize()
        assert int(status.item()) == bit
        for name, t in out.items():
            assert (t.view(torch.uint8) == 0xFF).all(), f"quantize wrote {name} despite invalid sizes"
        q[recipe] = out
        status.zero_()
    for recipe in (bs.RECIPE_MX, bs.RECIPE_PC):
        for acc in (False, True):
            out = torch.full((E, n, h), 5.0, device=DEV)
            bs.grouped_gemm_wgrad(q[recipe], n, q[recipe], h, st, R, recipe, out, accumulate=acc, status=status)
            torch.cuda.synchronize()
            assert int(status.item()) == bit and (out == 5.0).all()
            status.zero_()
    w = bs.alloc_quantized(E * n, h, 1, bs.RECIPE_MX, bs.ROWWISE, DEV)
    for t in w.values():
        t.zero_()
    fo = torch.full((R, n), 5.0, device=DEV)
    bs.grouped_gemm_fprop(q[bs.RECIPE_MX], h, w, n, st, R, fo, bs.OUT_F32, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == bit and (fo == 5.0).all()


def test_max_groups_wgrad_and_fprop():
    """num_groups at the 1024 maximum: the scan spans two entries per thread of a 512-thread
    workgroup; empty groups, one-row groups and 128-row groups mixed, garbage padding."""
    E = bs.MAX_GROUPS
    rng = np.random.default_rng(1024)
    splits = [int(v) for v in rng.choice([0, 1, 2, 31, 33, 64, 128, 129], size=E)]
    T = sum(splits)
    n = h = 64
    R = T + 40
    flush(f"max groups E={E} T={T}")
    dy, x = _operands(R, n, h, splits, seed=7)
    for recipe in (bs.RECIPE_MX, bs.RECIPE_PC):
        check_wgrad(dy, x, splits, recipe, label=f"E={E} r{recipe}")
    mg = torch.randn(E, n, h, dtype=torch.float32, device=DEV)
    check_wgrad(dy, x, splits, bs.RECIPE_MX, accumulate=True, mg=mg, label=f"E={E} acc")
    g = torch.Generator(device=DEV).manual_seed(8)
    w = W.randn_bf16((E * 64, h), g, DEV)
    check_fprop(x, w, splits, 64, bs.OUT_F32, label=f"E={E} fprop")

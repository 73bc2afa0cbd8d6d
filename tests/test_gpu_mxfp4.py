"""MXFP4 (e2m1, one E8M0 scale per 32 values) on the GPU vs the fp64 CPU oracle.

The same gated grouped paths accept a 4-bit block-scaled quantizer (TransformerEngine issue #3484,
additional context, scope); here it is the OCP MXFP4 format on the scaled fp4 MFMA.

* quantize: packed codes and scales bit-exact against the oracle, rowwise and colwise, ragged
  groups, outputs pre-poisoned so that writes past the documented extents show up.
* wgrad / fprop / dgrad: per-expert relative Frobenius error <= 1e-5 (fp32 out); bf16 within one
  bf16 ulp plus 1e-5 of the rms; empty experts zero or untouched; rows past sum(split_sizes)
  untouched; padding bitwise invariant; repeated calls bitwise identical.
Shapes cover K extents that end in half a K step (the run-time tail: a group with an odd number of
128-row blocks, K not a multiple of 256) and partial output tiles.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp8_grouped_amd as bs
import oracle
import workloads as W
from gpu_util import (DEV, REL_TOL, assert_bf16_close, assert_quant_matches, flush, gpu_quantize, rel_err)

pytestmark = pytest.mark.gpu
MX4 = bs.RECIPE_MX4
RAGGED = [[0, 1, 31, 32, 33, 127, 128, 129, 256], [300, 0, 45, 1, 200], [1000], [0, 0, 5]]


def _garbage_pad(t, T, seed):
    R = t.shape[0]
    if R > T:
        rng = np.random.default_rng(seed)
        bits = rng.integers(0, 1 << 16, size=(R - T, t.shape[1]), dtype=np.uint16)
        t[T:] = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    return t


# ------------------------------------------------------------------------------------------
# quantize
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("splits", RAGGED)
@pytest.mark.parametrize("C", [32, 160, 512])
def test_mx4_quantize_row_and_col(splits, C):
    flush(f"mx4 quantize C={C} splits={splits}")
    T = sum(splits)
    R = T + 37
    g = torch.Generator(device=DEV).manual_seed(C + T)
    x = _garbage_pad(W.randn_bf16((R, C), g, DEV, scale=2.0), T, C)
    which = bs.ROWWISE | bs.COLWISE
    got = gpu_quantize(x, splits, MX4, which)
    torch.cuda.synchronize()
    ref = oracle.grouped_quantize(W.bf16_bits(x), splits, oracle.RECIPE_MX4, which)
    assert_quant_matches(got, ref, splits, R, which, f"mx4 C={C}")


def test_mx4_quantize_rowwise_weight_and_special_values():
    flush("mx4 quantize special values")
    v = torch.tensor([0.0, -0.0, 1e-30, -1e-30, 6.0, -6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 448.0,
                      3e38, -3e38, 1.0, 2.0, 3.0, 4.0, 1e-40, -1e-40, 7.0, -5.0] + [0.5] * 8)
    x = torch.stack([v, v * 0.75, v * 1e-20, -v]).to(torch.bfloat16).to(DEV)  # all finite
    x = torch.cat([x, W.randn_bf16((60, 32), torch.Generator(device=DEV).manual_seed(3), DEV)])
    got = gpu_quantize(x, None, MX4, bs.ROWWISE)
    torch.cuda.synchronize()
    ref = oracle.grouped_quantize(W.bf16_bits(x), None, oracle.RECIPE_MX4, oracle.ROWWISE)
    assert_quant_matches(got, ref, None, x.shape[0], bs.ROWWISE, "mx4 special")


# ------------------------------------------------------------------------------------------
# wgrad
# ------------------------------------------------------------------------------------------

def _wgrad_case(R, n, h, splits, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    T = sum(splits)
    dy = _garbage_pad(W.randn_bf16((R, n), g, DEV), T, seed)
    x = _garbage_pad(W.randn_bf16((R, h), g, DEV), T, seed + 1)
    return dy, x


def _run_wgrad(dy, x, splits, accumulate=False, mg=None):
    R, n = dy.shape
    h = x.shape[1]
    st = W.splits_tensor(splits, DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    dq = gpu_quantize(dy, splits, MX4, bs.COLWISE, status=status)
    xq = gpu_quantize(x, splits, MX4, bs.COLWISE, status=status)
    out = mg.clone() if accumulate else torch.full((len(splits), n, h), float("nan"), device=DEV)
    bs.grouped_gemm_wgrad(dq, n, xq, h, st, R, MX4, out, accumulate=accumulate, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    return out, dq, xq


def _check_wgrad(dy, x, splits, accumulate=False, mg=None, label=""):
    R, n = dy.shape
    h = x.shape[1]
    out, dq, xq = _run_wgrad(dy, x, splits, accumulate, mg)
    o_dy = oracle.grouped_quantize(W.bf16_bits(dy), splits, oracle.RECIPE_MX4, oracle.COLWISE)
    o_x = oracle.grouped_quantize(W.bf16_bits(x), splits, oracle.RECIPE_MX4, oracle.COLWISE)
    assert_quant_matches(dq, o_dy, splits, R, bs.COLWISE, label + " dy")
    assert_quant_matches(xq, o_x, splits, R, bs.COLWISE, label + " x")
    ref = oracle.grouped_wgrad(o_dy["col_q"], o_dy["col_s"], n, o_x["col_q"], o_x["col_s"], h, splits, R,
                               oracle.RECIPE_MX4)
    got = out.cpu().numpy().astype(np.float64)
    for e, k in enumerate(splits):
        if k == 0:
            if accumulate:
                assert torch.equal(out[e].view(torch.int32), mg[e].view(torch.int32)), f"{label} e={e} touched"
            else:
                assert (out[e] == 0).all(), f"{label} empty expert {e} not zero"
            continue
        part = got[e] - mg[e].cpu().numpy().astype(np.float64) if accumulate else got[e]
        r = rel_err(part, ref[e])
        assert r <= REL_TOL, f"{label} expert {e} (k={k}): rel {r:.3e}"
    return out


@pytest.mark.parametrize("n,h", [(256, 256), (96, 320), (512, 64)])
@pytest.mark.parametrize("splits", RAGGED[:3])
def test_mx4_wgrad_store_parity(n, h, splits):
    flush(f"mx4 wgrad n={n} h={h} splits={splits}")
    R = sum(splits) + 50
    dy, x = _wgrad_case(R, n, h, splits, seed=n + h)
    _check_wgrad(dy, x, splits, label=f"mx4 {n}x{h}")


def test_mx4_wgrad_accumulate_and_empty_untouched():
    flush("mx4 wgrad accumulate")
    splits = [129, 0, 384, 1, 255]
    R, n, h = sum(splits) + 10, 288, 160
    dy, x = _wgrad_case(R, n, h, splits, seed=5)
    mg = torch.randn(len(splits), n, h, device=DEV, generator=torch.Generator(device=DEV).manual_seed(6))
    _check_wgrad(dy, x, splits, accumulate=True, mg=mg, label="mx4 acc")


@pytest.mark.parametrize("fill", [0.0, 3.0, "garbage"])
def test_mx4_wgrad_padding_bitwise_invariant(fill):
    flush(f"mx4 wgrad padding {fill}")
    splits = [200, 0, 77]
    T, n, h = sum(splits), 128, 192
    g = torch.Generator(device=DEV).manual_seed(8)
    dy0, x0 = W.randn_bf16((T, n), g, DEV), W.randn_bf16((T, h), g, DEV)
    base, _, _ = _run_wgrad(dy0, x0, splits)
    R = T + 150
    dy = torch.empty((R, n), dtype=torch.bfloat16, device=DEV)
    x = torch.empty((R, h), dtype=torch.bfloat16, device=DEV)
    dy[:T], x[:T] = dy0, x0
    if fill == "garbage":
        _garbage_pad(dy, T, 9)
        _garbage_pad(x, T, 10)
    else:
        dy[T:], x[T:] = fill, fill
    padded, _, _ = _run_wgrad(dy, x, splits)
    assert torch.equal(base.view(torch.int32), padded.view(torch.int32))


# ------------------------------------------------------------------------------------------
# fprop and dgrad
# ------------------------------------------------------------------------------------------

def _check_rows(got, ref, splits, out_dtype, label):
    T = sum(splits)
    assert np.isnan(got[T:]).all(), f"{label}: rows past the live rows were written"
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


@pytest.mark.parametrize("out_dtype", [bs.OUT_F32, bs.OUT_BF16])
@pytest.mark.parametrize("K,N", [(256, 256), (96, 320), (160, 64), (768, 512)])
@pytest.mark.parametrize("splits", RAGGED[:3])
def test_mx4_fprop_parity(out_dtype, K, N, splits):
    flush(f"mx4 fprop dtype={out_dtype} K={K} N={N} splits={splits}")
    T = sum(splits)
    R = T + 64
    g = torch.Generator(device=DEV).manual_seed(K + N)
    x = _garbage_pad(W.randn_bf16((R, K), g, DEV), T, K)
    w = W.randn_bf16((len(splits) * N, K), g, DEV)
    st = W.splits_tensor(splits, DEV)
    xq = gpu_quantize(x, splits, MX4, bs.ROWWISE)
    wq = gpu_quantize(w, None, MX4, bs.ROWWISE)
    dt = torch.float32 if out_dtype == bs.OUT_F32 else torch.bfloat16
    out = torch.full((R, N), float("nan"), dtype=dt, device=DEV)
    bs.grouped_gemm_fprop(xq, K, wq, N, st, R, out, out_dtype, recipe=MX4)
    torch.cuda.synchronize()
    o_x = oracle.grouped_quantize(W.bf16_bits(x), splits, oracle.RECIPE_MX4, oracle.ROWWISE)
    o_w = oracle.grouped_quantize(W.bf16_bits(w), None, oracle.RECIPE_MX4, oracle.ROWWISE)
    assert_quant_matches(xq, o_x, splits, R, bs.ROWWISE, "x")
    assert_quant_matches(wq, o_w, None, w.shape[0], bs.ROWWISE, "w")
    ref = oracle.grouped_fprop(o_x["row_q"], o_x["row_s"], o_w["row_q"], o_w["row_s"], N, splits,
                               recipe=oracle.RECIPE_MX4)
    _check_rows(out.float().cpu().numpy().astype(np.float64), ref, splits, out_dtype, f"mx4 fprop K={K} N={N}")


@pytest.mark.parametrize("out_dtype", [bs.OUT_F32, bs.OUT_BF16])
@pytest.mark.parametrize("n,k", [(256, 256), (96, 320), (160, 64), (512, 512)])
@pytest.mark.parametrize("splits", RAGGED[:3])
def test_mx4_dgrad_parity(out_dtype, n, k, splits):
    flush(f"mx4 dgrad dtype={out_dtype} n={n} k={k} splits={splits}")
    T = sum(splits)
    R, E = T + 64, len(splits)
    g = torch.Generator(device=DEV).manual_seed(n + k + 1)
    dy = _garbage_pad(W.randn_bf16((R, n), g, DEV), T, n)
    w = W.randn_bf16((E * n, k), g, DEV)
    st = W.splits_tensor(splits, DEV)
    dyq = gpu_quantize(dy, splits, MX4, bs.ROWWISE)
    wq = gpu_quantize(w, [n] * E, MX4, bs.COLWISE)
    dt = torch.float32 if out_dtype == bs.OUT_F32 else torch.bfloat16
    out = torch.full((R, k), float("nan"), dtype=dt, device=DEV)
    bs.grouped_gemm_dgrad(dyq, n, wq, k, st, R, out, out_dtype, recipe=MX4)
    torch.cuda.synchronize()
    o_dy = oracle.grouped_quantize(W.bf16_bits(dy), splits, oracle.RECIPE_MX4, oracle.ROWWISE)
    o_w = oracle.grouped_quantize(W.bf16_bits(w), [n] * E, oracle.RECIPE_MX4, oracle.COLWISE)
    assert_quant_matches(dyq, o_dy, splits, R, bs.ROWWISE, "dy")
    assert_quant_matches(wq, o_w, [n] * E, E * n, bs.COLWISE, "w")
    ref = oracle.grouped_dgrad(o_dy["row_q"], o_dy["row_s"], o_w["col_q"], o_w["col_s"], k, splits,
                               recipe=oracle.RECIPE_MX4)
    _check_rows(out.float().cpu().numpy().astype(np.float64), ref, splits, out_dtype, f"mx4 dgrad n={n} k={k}")


def test_mx4_repeated_calls_bitwise_identical():
    flush("mx4 determinism")
    splits = [300, 0, 45, 1, 200]
    R, n, h = sum(splits) + 20, 256, 320
    dy, x = _wgrad_case(R, n, h, splits, seed=12)
    first, dq, xq = _run_wgrad(dy, x, splits)
    st = W.splits_tensor(splits, DEV)
    for _ in range(20):
        out = torch.empty_like(first)
        bs.grouped_gemm_wgrad(dq, n, xq, h, st, R, MX4, out)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), first.view(torch.int32))

"""GPU m-grouped dgrad (dx_e = dy_e @ W_e, the weight quantized colwise along n) vs the fp64 CPU
oracle on the same quantized inputs.

* fp32 out: per-expert relative Frobenius error <= 1e-5; bf16 out: within one bf16 ulp of the
  oracle rounded to bf16 plus 1e-5 of the expert's rms output; rows past sum(split_sizes)
  untouched.
* the quantized operands (dy rowwise, W colwise with splits [n] * E) bit-exact against the oracle.
* padding invariance: capacity tails of 0.0, 3.0 or random bits give results bitwise equal to the
  unpadded run.
* device status word: invalid sizes set their bit and nothing is written.
Shapes: n not a multiple of 128 (padded weight rows and the K-tail kernel), k not a multiple of
256 (partial output tiles), empty experts, and the 32- and 128-expert MoE shapes on sampled columns.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp8_grouped_amd as bs
import oracle
import workloads as W
from gpu_util import (DEV, REL_TOL, assert_bf16_close, assert_quant_matches, flush, gpu_quantize, rel_err)

pytestmark = pytest.mark.gpu


def run_dgrad(dy, w, splits, out_dtype, status=None):
    """dy [R, n] bf16, w [E, n, k] bf16 -> (out [R, k], dy rowwise dict, W colwise dict)."""
    R, n = dy.shape
    E, _, k = w.shape
    st = W.splits_tensor(splits, DEV)
    dyq = gpu_quantize(dy, splits, bs.RECIPE_MX, bs.ROWWISE, status=status)
    wq = gpu_quantize(w.reshape(E * n, k), [n] * E, bs.RECIPE_MX, bs.COLWISE)
    dt = torch.float32 if out_dtype == bs.OUT_F32 else torch.bfloat16
    out = torch.full((R, k), float("nan"), dtype=dt, device=DEV)
    bs.grouped_gemm_dgrad(dyq, n, wq, k, st, R, out, out_dtype, status=status)
    return out, dyq, wq


def check_dgrad(dy, w, splits, out_dtype, cols_sel=None, experts=None, label=""):
    R, n = dy.shape
    E, _, k = w.shape
    T = sum(splits)
    out, dyq, wq = run_dgrad(dy, w, splits, out_dtype)
    torch.cuda.synchronize()
    offs = np.concatenate([[0], np.cumsum(splits)]).astype(np.int64)
    experts = range(E) if experts is None else experts
    sel = np.arange(k, dtype=np.int32) if cols_sel is None else np.asarray(cols_sel, np.int32)
    got_all = out.float()
    assert torch.isnan(got_all[T:]).all(), f"{label}: rows past the live rows were written"
    np_ = 128 * ((n + 127) // 128)
    for e in experts:
        ke, off = splits[e], int(offs[e])
        if ke == 0:
            continue
        # this expert alone, quantized by the oracle: its rows of dy and its weight block
        o_dy = oracle.grouped_quantize(W.bf16_bits(dy[off:off + ke]), [ke], oracle.RECIPE_MX, oracle.ROWWISE)
        o_w = oracle.grouped_quantize(W.bf16_bits(w[e]), [n], oracle.RECIPE_MX, oracle.COLWISE)
        assert np.array_equal(dyq["row_q"][off:off + ke].cpu().numpy(), o_dy["row_q"]), f"{label} dy bytes e={e}"
        assert np.array_equal(dyq["row_s"][:, off:off + ke].cpu().numpy(), o_dy["row_s"]), f"{label} dy scales e={e}"
        assert np.array_equal(wq["col_q"][k * np_ * e: k * np_ * (e + 1)].cpu().numpy(), o_w["col_q"]), \
            f"{label} W bytes e={e}"
        assert np.array_equal(wq["col_s"][k * np_ * e // 32: k * np_ * (e + 1) // 32].cpu().numpy(), o_w["col_s"]), \
            f"{label} W scales e={e}"
        ref = oracle.grouped_dgrad(o_dy["row_q"], o_dy["row_s"], o_w["col_q"], o_w["col_s"], k, [ke], cols_sel=sel)
        g_e = got_all[off:off + ke].cpu().numpy().astype(np.float64)[:, sel]
        if out_dtype == bs.OUT_F32:
            r = rel_err(g_e, ref)
            assert r <= REL_TOL, f"{label} expert {e}: rel {r:.3e}"
        else:
            assert_bf16_close(g_e, ref, f"{label} expert {e}")
    return out


@pytest.mark.parametrize("out_dtype", [bs.OUT_F32, bs.OUT_BF16])
@pytest.mark.parametrize("n,k", [(256, 256), (96, 320), (160, 64), (512, 512), (128, 96)])
@pytest.mark.parametrize("splits", [[0, 1, 31, 32, 33, 127, 128, 129, 256], [300, 0, 45, 1, 200], [600]])
def test_dgrad_parity(out_dtype, n, k, splits):
    flush(f"dgrad dtype={out_dtype} n={n} k={k} splits={splits}")
    T = sum(splits)
    R = T + 64
    g = torch.Generator(device=DEV).manual_seed(n + 3 * k)
    dy = W.randn_bf16((R, n), g, DEV)
    bits = np.random.default_rng(2).integers(0, 1 << 16, size=(R - T, n), dtype=np.uint16)
    dy[T:] = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    w = W.randn_bf16((len(splits), n, k), g, DEV)
    check_dgrad(dy, w, splits, out_dtype, label=f"n={n} k={k}")


def test_dgrad_padding_bitwise_invariant():
    splits = [70, 0, 333]
    T, n, k = sum(splits), 256, 128
    g = torch.Generator(device=DEV).manual_seed(5)
    dy0 = W.randn_bf16((T, n), g, DEV)
    w = W.randn_bf16((3, n, k), g, DEV)
    ref, _, _ = run_dgrad(dy0, w, splits, bs.OUT_F32)
    for fill in (0.0, 3.0, "garbage"):
        dy = torch.empty(T + 200, n, dtype=torch.bfloat16, device=DEV)
        dy[:T] = dy0
        if fill == "garbage":
            bits = np.random.default_rng(6).integers(0, 1 << 16, size=(200, n), dtype=np.uint16)
            dy[T:] = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
        else:
            dy[T:] = fill
        got, _, _ = run_dgrad(dy, w, splits, bs.OUT_F32)
        torch.cuda.synchronize()
        assert torch.equal(got[:T].view(torch.int32), ref[:T].view(torch.int32)), fill
        assert torch.isnan(got[T:]).all()


@pytest.mark.parametrize("splits,R,bit", [([100, -5, 50], 400, bs.STATUS_NEGATIVE_SPLIT),
                                          ([200, 100, 50], 300, bs.STATUS_EXCEEDS_CAPACITY)])
def test_dgrad_status_bits_and_no_writes(splits, R, bit):
    n, k, E = 64, 96, len(splits)
    st = W.splits_tensor(splits, DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    dyq = bs.alloc_quantized(R, n, E, bs.RECIPE_MX, bs.ROWWISE, DEV)
    wq = bs.alloc_quantized(E * n, k, E, bs.RECIPE_MX, bs.COLWISE, DEV)
    for t in list(dyq.values()) + list(wq.values()):
        t.zero_()
    out = torch.full((R, k), 5.0, device=DEV)
    bs.grouped_gemm_dgrad(dyq, n, wq, k, st, R, out, bs.OUT_F32, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == bit and (out == 5.0).all()


def test_dgrad_zero_capacity_returns_ok():
    st = W.splits_tensor([0, 0], DEV)
    dyq = bs.alloc_quantized(0, 64, 2, bs.RECIPE_MX, bs.ROWWISE, DEV)
    wq = bs.alloc_quantized(2 * 64, 64, 2, bs.RECIPE_MX, bs.COLWISE, DEV)
    out = torch.empty(0, 64, device=DEV)
    bs.grouped_gemm_dgrad(dyq, 64, wq, 64, st, 0, out, bs.OUT_F32)


def test_dgrad_moe32_shape_sampled():
    """32 experts, 65,536 routed rows with Zipf counts (4 empty), n = 1536 -> k = 4096, fp32 out:
    the oracle on 6 experts x 96 sampled columns."""
    case = W.moe32_zipf(DEV)
    splits, R = case["splits"], case["R"]
    n, k = case["n"], case["h"]
    E = len(splits)
    g = torch.Generator(device=DEV).manual_seed(41)
    w = W.randn_bf16((E, n, k), g, DEV)
    rng = np.random.default_rng(41)
    live = [e for e in range(E) if splits[e]]
    experts = sorted(set(rng.choice(live, 5, replace=False).tolist()) | {int(np.argmax(splits))})
    cols = np.sort(rng.choice(k, 96, replace=False)).astype(np.int32)
    flush(f"dgrad moe32 experts {experts}")
    check_dgrad(case["dy"], w, splits, bs.OUT_F32, cols_sel=cols, experts=experts, label="moe32")


def test_dgrad_moe128_shape_sampled():
    """128 experts (6 empty) with n = 2048 -> k = 7168 and bf16 out, 131,072 routed rows (a
    shorter run of the 128-expert layer's token count): the oracle on 4 experts x 64 columns."""
    rng = np.random.default_rng(43)
    E, n, k, T = 128, 2048, 7168, 131072
    empty = rng.choice(E, 6, replace=False)
    p = np.ones(E)
    p[empty] = 0
    splits = [int(c) for c in rng.multinomial(T, p / p.sum())]
    g = torch.Generator(device=DEV).manual_seed(43)
    dy = W.randn_bf16((T, n), g, DEV, 0.5)
    w = W.randn_bf16((E, n, k), g, DEV, 0.5)
    live = [e for e in range(E) if splits[e]]
    experts = sorted(rng.choice(live, 4, replace=False).tolist())
    cols = np.sort(rng.choice(k, 64, replace=False)).astype(np.int32)
    flush(f"dgrad moe128 experts {experts}")
    check_dgrad(dy, w, splits, bs.OUT_BF16, cols_sel=cols, experts=experts, label="moe128")

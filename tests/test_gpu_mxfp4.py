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


def _check_wgrad(dy, x, splits, accumulate=False, mg=None, label="", rows_sel=None):
    R, n = dy.shape
    h = x.shape[1]
    out, dq, xq = _run_wgrad(dy, x, splits, accumulate, mg)
    o_dy = oracle.grouped_quantize(W.bf16_bits(dy), splits, oracle.RECIPE_MX4, oracle.COLWISE)
    o_x = oracle.grouped_quantize(W.bf16_bits(x), splits, oracle.RECIPE_MX4, oracle.COLWISE)
    assert_quant_matches(dq, o_dy, splits, R, bs.COLWISE, label + " dy")
    assert_quant_matches(xq, o_x, splits, R, bs.COLWISE, label + " x")
    sel = np.arange(n, dtype=np.int32) if rows_sel is None else np.asarray(rows_sel, np.int32)
    ref = oracle.grouped_wgrad(o_dy["col_q"], o_dy["col_s"], n, o_x["col_q"], o_x["col_s"], h, splits, R,
                               oracle.RECIPE_MX4, rows_sel=sel)
    got = out.cpu().numpy()[:, sel, :].astype(np.float64)
    for e, k in enumerate(splits):
        if k == 0:
            if accumulate:
                assert torch.equal(out[e].view(torch.int32), mg[e].view(torch.int32)), f"{label} e={e} touched"
            else:
                assert (out[e] == 0).all(), f"{label} empty expert {e} not zero"
            continue
        part = got[e] - mg[e].cpu().numpy()[sel].astype(np.float64) if accumulate else got[e]
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


def test_mx4_wgrad_skewed_split_many_tiles():
    """Zipf split sizes over 40 experts (largest group above twice the mean non-empty size) and
    more 256x256 tiles than one round of 256 workgroups: the largest-first group order and the
    short per-XCD runs on the fp4 path.  Tile-edge rows and 40 random rows of every expert are
    held to the oracle."""
    rng = np.random.default_rng(11)
    splits = [int(c) for c in W.zipf_counts(rng, 40, 36, 7000)]
    live = [k for k in splits if k > 0]
    assert max(live) * len(live) > 2 * sum(live), splits  # the kernel's skew condition
    n, h = 512, 1024
    assert len(splits) * (n // 256) * (h // 256) > 256
    flush(f"mx4 wgrad skewed splits={splits}")
    R = sum(splits) + 77
    dy, x = _wgrad_case(R, n, h, splits, seed=13)
    edges = [0, 127, 128, 255, 256, 383, 384, 511]
    sel = np.union1d(edges, np.random.default_rng(14).choice(n, size=40, replace=False))
    _check_wgrad(dy, x, splits, label="mx4 skewed", rows_sel=sel)


def test_mx4_wgrad_and_fprop_max_groups():
    """num_groups at the 1024 maximum on the fp4 path: empty, one-row and 128-row groups mixed,
    garbage padding; wgrad store and accumulate, and the m-grouped forward."""
    E = bs.MAX_GROUPS
    rng = np.random.default_rng(1024)
    splits = [int(v) for v in rng.choice([0, 1, 2, 31, 33, 64, 128, 129], size=E)]
    n = h = 64
    R = sum(splits) + 40
    flush(f"mx4 max groups E={E} T={sum(splits)}")
    dy, x = _wgrad_case(R, n, h, splits, seed=7)
    _check_wgrad(dy, x, splits, label=f"mx4 E={E}")
    mg = torch.randn(E, n, h, device=DEV, generator=torch.Generator(device=DEV).manual_seed(9))
    _check_wgrad(dy, x, splits, accumulate=True, mg=mg, label=f"mx4 E={E} acc")
    N = 64
    w = W.randn_bf16((E * N, h), torch.Generator(device=DEV).manual_seed(8), DEV)
    _check_fprop(x, w, splits, N, bs.OUT_F32, f"mx4 E={E} fprop")


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
    _check_fprop(x, w, splits, N, out_dtype, f"mx4 fprop K={K} N={N}")


def _check_fprop(x, w, splits, N, out_dtype, label):
    R, K = x.shape
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
    _check_rows(out.float().cpu().numpy().astype(np.float64), ref, splits, out_dtype, label)


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


# ------------------------------------------------------------------------------------------
# the MoE shapes at full size
# ------------------------------------------------------------------------------------------

def test_mx4_moe32_full_size_sampled():
    """32 experts, 65,536 Zipf-routed rows (empty experts, counts not multiples of 32), garbage
    padding, hidden 4096, ffn 1536: quantize bit-exact on the full tensors, wgrad on 64 sampled dy
    channels of every expert, fprop fp32 on 32 sampled output columns."""
    case = W.moe32_zipf(DEV)
    splits, R = case["splits"], case["R"]
    flush(f"mx4 moe32 R={R}")
    rng = np.random.default_rng(41)
    rows = np.sort(rng.choice(case["n"], 64, replace=False)).astype(np.int32)
    _check_wgrad(case["dy"], case["x"], splits, label="mx4 moe32 wgrad", rows_sel=rows)
    K, N = case["K"], case["N"]
    cols = np.sort(rng.choice(N, 32, replace=False)).astype(np.int32)
    w = case["W"].view(-1, K)
    st = W.splits_tensor(splits, DEV)
    xq = gpu_quantize(case["x"], splits, MX4, bs.ROWWISE)
    wq = gpu_quantize(w, None, MX4, bs.ROWWISE)
    out = torch.full((R, N), float("nan"), device=DEV)
    bs.grouped_gemm_fprop(xq, K, wq, N, st, R, out, bs.OUT_F32, recipe=MX4)
    torch.cuda.synchronize()
    o_x = oracle.grouped_quantize(W.bf16_bits(case["x"]), splits, oracle.RECIPE_MX4, oracle.ROWWISE)
    o_w = oracle.grouped_quantize(W.bf16_bits(w), None, oracle.RECIPE_MX4, oracle.ROWWISE)
    assert_quant_matches(xq, o_x, splits, R, bs.ROWWISE, "mx4 moe32 x")
    assert_quant_matches(wq, o_w, None, w.shape[0], bs.ROWWISE, "mx4 moe32 w")
    ref = oracle.grouped_fprop(o_x["row_q"], o_x["row_s"], o_w["row_q"], o_w["row_s"], N, splits, cols_sel=cols,
                               recipe=oracle.RECIPE_MX4)
    got = out.cpu().numpy().astype(np.float64)
    assert np.isnan(got[sum(splits):]).all()
    _check_rows(got[:, cols], ref, splits, bs.OUT_F32, "mx4 moe32 fprop")


def test_mx4_moe128_sampled_experts():
    """The benchmark's MXFP4 launches on the 128-expert shape (wgrad accumulating into main_grad,
    fprop bf16), checked on three experts (largest, smallest non-empty, one between) against the
    oracle on those experts' rows; empty experts' main_grad bitwise untouched."""
    case = W.moe128_top8(DEV)
    splits, R = case["splits"], case["R"]
    n, h, K, N = case["n"], case["h"], case["K"], case["N"]
    E = len(splits)
    st = W.splits_tensor(splits, DEV)
    flush("mx4 moe128")
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    xq = gpu_quantize(case["x"], splits, MX4, bs.COLWISE | bs.ROWWISE, status=status)
    dq = gpu_quantize(case["dy"], splits, MX4, bs.COLWISE, status=status)
    w2 = case["W"].view(E * N, K)
    wq = gpu_quantize(w2, None, MX4, bs.ROWWISE)
    mg0 = case["main_grad"]
    empty = [e for e, k in enumerate(splits) if k == 0]
    mg_empty = mg0[empty].clone()
    live = [e for e, k in enumerate(splits) if k > 0]
    sample = sorted({max(live, key=lambda e: splits[e]), min(live, key=lambda e: splits[e]), live[len(live) // 2]})
    mg_before = {e: mg0[e].cpu().numpy().astype(np.float64) for e in sample}
    rng = np.random.default_rng(51)
    rows = np.sort(rng.choice(n, 32, replace=False)).astype(np.int32)
    cols = np.sort(rng.choice(N, 16, replace=False)).astype(np.int32)
    bs.grouped_gemm_wgrad(dq, n, xq, h, st, R, MX4, mg0, accumulate=True, status=status)
    fout = torch.empty(R, N, dtype=torch.bfloat16, device=DEV)
    bs.grouped_gemm_fprop(xq, K, wq, N, st, R, fout, bs.OUT_BF16, status=status, recipe=MX4)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(mg0[empty].view(torch.int32), mg_empty.view(torch.int32))
    offs = np.concatenate([[0], np.cumsum(splits)])
    kps = [128 * ((k + 127) // 128) for k in splits]
    pofs = np.concatenate([[0], np.cumsum(kps)])
    for e in sample:
        k, off, P, kp = splits[e], int(offs[e]), int(pofs[e]), kps[e]
        flush(f"mx4 moe128 expert {e} k={k}")
        ox = oracle.grouped_quantize(W.bf16_bits(case["x"][off:off + k]), [k], oracle.RECIPE_MX4,
                                     oracle.COLWISE | oracle.ROWWISE)
        ody = oracle.grouped_quantize(W.bf16_bits(case["dy"][off:off + k]), [k], oracle.RECIPE_MX4, oracle.COLWISE)
        ow = oracle.grouped_quantize(W.bf16_bits(w2[e * N:(e + 1) * N]), None, oracle.RECIPE_MX4, oracle.ROWWISE)
        assert np.array_equal(xq["col_q"][h * P // 2:h * (P + kp) // 2].cpu().numpy(), ox["col_q"])
        assert np.array_equal(dq["col_q"][n * P // 2:n * (P + kp) // 2].cpu().numpy(), ody["col_q"])
        assert np.array_equal(dq["col_s"][n * P // 32:n * (P + kp) // 32].cpu().numpy(), ody["col_s"])
        assert np.array_equal(xq["row_q"][off:off + k].cpu().numpy(), ox["row_q"])
        assert np.array_equal(wq["row_q"][e * N:(e + 1) * N].cpu().numpy(), ow["row_q"])
        ref = oracle.grouped_wgrad(ody["col_q"], ody["col_s"], n, ox["col_q"], ox["col_s"], h, [k], k,
                                   oracle.RECIPE_MX4, rows_sel=rows)
        got = mg0[e].cpu().numpy()[rows].astype(np.float64) - mg_before[e][rows]
        r = rel_err(got, ref[0])
        assert r <= REL_TOL, f"mx4 moe128 wgrad expert {e}: rel {r:.3e}"
        fref = oracle.grouped_fprop(ox["row_q"], ox["row_s"], ow["row_q"], ow["row_s"], N, [k], cols_sel=cols,
                                    recipe=oracle.RECIPE_MX4)
        fgot = fout[off:off + k].float().cpu().numpy().astype(np.float64)[:, cols]
        assert_bf16_close(fgot, fref, f"mx4 moe128 fprop expert {e}")

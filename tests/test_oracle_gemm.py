"""Pins of the oracle's grouped wgrad / fprop against things fixed outside it.

* Each group reduces to a textbook dense GEMM: torch float64 matmul of the dequantized live rows
  (dequantized and unpacked here with torch, not with the oracle) agrees to 1e-12.
* Tiny cases against exact rational sums (fractions): the fp64 result is within the fp64
  summation bound of the exact value.
* Unquantized brute force: the quantized result is within the closed-form quantization bound
  of the sum over the bf16 values themselves; that brute force in turn equals torch's matmul.
* Invariants the pages fix: padding rows never matter (TE #3484 expected behaviour, printed
  rel_err 0 / non_finite 0); an all-zero dy channel gives an all-zero output row; an empty group
  gives zeros or leaves main_grad untouched; num_groups == 1 equals the dense GEMM.
* The DeepGEMM #365 reproducer's printed reference max norm (1.311e-03) pins the generator.
"""
import fractions
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_printed_values.json")))


def _deq_colwise_torch(col_q, col_s, C, splits, recipe):
    """Per group [k_e, C] float64 dequantized operand, unpacked with torch reshapes."""
    out, P = [], 0
    blk = 32 if recipe == oracle.RECIPE_MX else 128
    for k in splits:
        kp = 128 * ((k + 127) // 128)
        q = torch.from_numpy(col_q[C * P:C * (P + kp)].copy()).view(torch.float8_e4m3fn).double().view(C, kp)
        if recipe == oracle.RECIPE_MX:
            s = torch.from_numpy(col_s[C * P // 32:C * (P + kp) // 32].astype(np.float64)).view(kp // 32, C)
            s = torch.pow(2.0, s - 127)
        else:
            s = torch.from_numpy(col_s[C * P // 128:C * (P + kp) // 128].astype(np.float64)).view(kp // 128, C)
        s = s.t().repeat_interleave(blk, dim=1)
        out.append((q * s)[:, :k].t().contiguous())
        P += kp
    return out


def _quant_case(case, recipe, sf_val=1e-30):
    dq = oracle.grouped_quantize(W.bf16_bits(case["dy"]), case["splits"], recipe, oracle.COLWISE, sf_val)
    xq = oracle.grouped_quantize(W.bf16_bits(case["x"]), case["splits"], recipe, oracle.COLWISE, sf_val)
    return dq, xq


def _wgrad(case, dq, xq, recipe, **kw):
    return oracle.grouped_wgrad(dq["col_q"], dq["col_s"], case["n"], xq["col_q"], xq["col_s"], case["h"],
                                case["splits"], case["R"], recipe, **kw)


@pytest.mark.parametrize("recipe,splits", [(oracle.RECIPE_PC, (256, 128, 128, 256)),
                                           (oracle.RECIPE_MX, (300, 0, 45, 1, 200)),
                                           (oracle.RECIPE_MX, (512,))])
def test_wgrad_equals_dense_matmul_per_group(recipe, splits):
    case = W.deepgemm_case("cpu", 64, 96, splits=splits, R=sum(splits) + 50)
    if recipe == oracle.RECIPE_MX:  # unit-scale data so MX exponents vary across blocks
        case["dy"] = (case["dy"].float() * 1e7).to(torch.bfloat16)
    dq, xq = _quant_case(case, recipe)
    got = _wgrad(case, dq, xq, recipe)
    A = _deq_colwise_torch(dq["col_q"], dq["col_s"], case["n"], case["splits"], recipe)
    B = _deq_colwise_torch(xq["col_q"], xq["col_s"], case["h"], case["splits"], recipe)
    for e, k in enumerate(case["splits"]):
        ref = (A[e].t() @ B[e]).numpy()
        if k == 0:
            assert not got[e].any()
            continue
        rel = np.linalg.norm(got[e] - ref) / max(np.linalg.norm(ref), 1e-300)
        assert rel <= 1e-12, (e, rel)


def test_wgrad_row_selection_matches_full():
    case = W.deepgemm_case("cpu", 64, 32, splits=(130, 7, 0, 64), R=300)
    dq, xq = _quant_case(case, oracle.RECIPE_MX)
    full = _wgrad(case, dq, xq, oracle.RECIPE_MX)
    sel = np.array([63, 0, 17, 17, 5], np.int32)
    part = _wgrad(case, dq, xq, oracle.RECIPE_MX, rows_sel=sel)
    assert np.array_equal(part, full[:, sel, :])


def test_wgrad_tiny_exact_rational():
    case = W.deepgemm_case("cpu", 32, 32, splits=(33, 7, 0, 40), R=100)
    case["dy"] = (case["dy"].float() * 1e7).to(torch.bfloat16)
    for recipe in (oracle.RECIPE_MX, oracle.RECIPE_PC):
        dq, xq = _quant_case(case, recipe)
        got = _wgrad(case, dq, xq, recipe)
        A = _deq_colwise_torch(dq["col_q"], dq["col_s"], 32, case["splits"], recipe)
        B = _deq_colwise_torch(xq["col_q"], xq["col_s"], 32, case["splits"], recipe)
        for e, k in enumerate(case["splits"]):
            if k == 0:
                continue
            a = A[e].numpy()
            b = B[e].numpy()
            for i, j in [(0, 0), (3, 31), (31, 7), (16, 16)]:
                exact = sum(fractions.Fraction(float(a[t, i])) * fractions.Fraction(float(b[t, j])) for t in range(k))
                mag = sum(abs(float(a[t, i]) * float(b[t, j])) for t in range(k))
                assert abs(fractions.Fraction(got[e, i, j]) - exact) <= k * 2.0 ** -52 * mag + 1e-300


def test_unquantized_brute_force_matches_torch_and_bound():
    case = W.deepgemm_case("cpu", 32, 64, splits=(70, 0, 33), R=120)
    case["dy"] = (case["dy"].float() * 1e7).to(torch.bfloat16)
    splits, T = case["splits"], case["T"]
    unq = oracle.wgrad_unquantized(W.bf16_bits(case["dy"]), W.bf16_bits(case["x"]), splits, case["R"])
    dyf, xf = case["dy"].double(), case["x"].double()
    off = 0
    for e, k in enumerate(splits):
        ref = (dyf[off:off + k].t() @ xf[off:off + k]).numpy()
        assert np.allclose(unq[e], ref, rtol=1e-13, atol=1e-300)
        off += k
    for recipe in (oracle.RECIPE_MX, oracle.RECIPE_PC):
        dq, xq = _quant_case(case, recipe)
        got = _wgrad(case, dq, xq, recipe)
        A = _deq_colwise_torch(dq["col_q"], dq["col_s"], 32, splits, recipe)
        B = _deq_colwise_torch(xq["col_q"], xq["col_s"], 64, splits, recipe)
        off = 0
        for e, k in enumerate(splits):
            a = dyf[off:off + k].numpy()
            b = xf[off:off + k].numpy()
            # per-element quantization error bound: half an ulp relative (2^-4, plus fp32
            # rounding of the per-channel multiply) or half the subnormal step times the scale
            sa = np.abs(A[e].numpy() - a).max(initial=0)  # not used in the bound, sanity only
            da = (2.0 ** -4 + 2.0 ** -20) * np.abs(a) + 2.0 ** -10 * _scale_per_elem(dq, 32, splits, e, recipe)
            db = (2.0 ** -4 + 2.0 ** -20) * np.abs(b) + 2.0 ** -10 * _scale_per_elem(xq, 64, splits, e, recipe)
            bound = da.T @ (np.abs(b) + db) + np.abs(a).T @ db
            assert np.all(np.abs(got[e] - unq[e]) <= bound * (1 + 1e-12) + 1e-300), recipe
            assert sa < np.inf
            off += k


def _scale_per_elem(qd, C, splits, e, recipe):
    """[k_e, C] block scale (float64) of every live element of group e."""
    P = sum(128 * ((k + 127) // 128) for k in splits[:e])
    k = splits[e]
    kp = 128 * ((k + 127) // 128)
    if recipe == oracle.RECIPE_MX:
        s = qd["col_s"][C * P // 32:C * (P + kp) // 32].reshape(kp // 32, C).astype(np.float64)
        s = np.ldexp(1.0, s.astype(np.int64) - 127)
        return np.repeat(s, 32, axis=0)[:k]
    s = qd["col_s"][C * P // 128:C * (P + kp) // 128].reshape(kp // 128, C).astype(np.float64)
    return np.repeat(s, 128, axis=0)[:k]


def test_zero_channel_gives_zero_row_and_empty_group_zero():
    case = W.deepgemm_case("cpu", 256, 256, R=1024)  # the DeepGEMM #365 structure with padding 3.0
    dq, xq = _quant_case(case, oracle.RECIPE_PC)
    got = _wgrad(case, dq, xq, oracle.RECIPE_PC)
    for e, k in enumerate(case["splits"]):
        if k == 128:
            assert not got[e, 0].any()  # the zeroed dy channel -> exact zero output row
        else:
            assert np.all(got[e, 0] != 0)
    # empty group, store and accumulate
    case = W.deepgemm_case("cpu", 32, 64, splits=(64, 0, 32), R=100)
    dq, xq = _quant_case(case, oracle.RECIPE_MX)
    got = _wgrad(case, dq, xq, oracle.RECIPE_MX)
    assert not got[1].any()
    mg = np.random.default_rng(0).standard_normal((3, 32, 64)).astype(np.float32)
    acc = _wgrad(case, dq, xq, oracle.RECIPE_MX, accumulate=True, mg_in=mg)
    assert np.array_equal(acc[1], mg[1].astype(np.float64))
    assert np.array_equal(acc[0], mg[0].astype(np.float64) + got[0])


def test_padding_invariance_matches_printed_expectation():
    """TE #3484: padded (0.0 and 3.0) vs unpadded runs agree exactly (printed rel_err 0)."""
    exp = GOLDEN["te3484_expected"]
    results = {}
    for R, fill in ((512, 0.0), (768, 0.0), (768, 3.0)):
        case = W.te_single_group_case("cpu", R=R, pad_fill=fill)
        dq, xq = _quant_case(case, oracle.RECIPE_MX)
        mg = case["main_grad"].numpy()
        results[(R, fill)] = _wgrad(case, dq, xq, oracle.RECIPE_MX, accumulate=True, mg_in=mg)
    ref = results[(512, 0.0)]
    assert ref.size == exp["numel"]
    for key in ((768, 0.0), (768, 3.0)):
        got = results[key]
        rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        assert rel == exp["rel_err"]
        assert int((~np.isfinite(got)).sum()) == exp["non_finite"]
        assert np.array_equal(got, ref)


def test_generator_matches_printed_reference_norm():
    """DeepGEMM #365 printed the max per-expert norm of its unquantized reference as 1.311e-03;
    the closed form sqrt(n*H*k)*sigma_dy*sigma_x gives 1.3107e-3 for k = 256."""
    g = GOLDEN["dg365_reference_max_norm"]
    case = W.deepgemm_case("cpu", 2048, 2048)
    dyf, xf = case["dy"].float(), case["x"].float()
    norms, off = [], 0
    for k in case["splits"]:
        norms.append(torch.linalg.vector_norm(dyf[off:off + k].t() @ xf[off:off + k]).item())
        off += k
    assert abs(max(norms) - g["value"]) / g["value"] < 0.01
    assert abs(np.sqrt(2048 * 2048 * 256) * 1e-7 * 0.4 - g["value"]) / g["value"] < 1e-3


def _rowwise_deq_torch(q, s):
    R, K = q.shape
    v = torch.from_numpy(q.copy()).view(torch.float8_e4m3fn).double()
    sc = torch.pow(2.0, torch.from_numpy(s.astype(np.float64)) - 127).t().repeat_interleave(32, dim=1)
    return v * sc


def test_fprop_equals_dense_matmul_per_group():
    rng = np.random.default_rng(9)
    splits = [40, 0, 129, 3]
    T, K, N, E = sum(splits), 96, 64, 4
    R = T + 20
    x = torch.from_numpy(rng.standard_normal((R, K)).astype(np.float32)).to(torch.bfloat16)
    x[T:] = float("nan")
    w = torch.from_numpy(rng.standard_normal((E * N, K)).astype(np.float32)).to(torch.bfloat16)
    xq = oracle.grouped_quantize(W.bf16_bits(x), splits, oracle.RECIPE_MX, oracle.ROWWISE)
    wq = oracle.grouped_quantize(W.bf16_bits(w), None, oracle.RECIPE_MX, oracle.ROWWISE)
    got = oracle.grouped_fprop(xq["row_q"], xq["row_s"], wq["row_q"], wq["row_s"], N, splits)
    X = _rowwise_deq_torch(xq["row_q"], xq["row_s"])
    Wd = _rowwise_deq_torch(wq["row_q"], wq["row_s"]).view(E, N, K)
    off = 0
    for e, k in enumerate(splits):
        ref = (X[off:off + k] @ Wd[e].t()).numpy()
        assert np.allclose(got[off:off + k], ref, rtol=1e-12, atol=1e-300)
        off += k
    assert np.isnan(got[T:]).all()  # rows outside every group are not written
    sel = np.array([5, 63, 0], np.int32)
    part = oracle.grouped_fprop(xq["row_q"], xq["row_s"], wq["row_q"], wq["row_s"], N, splits, cols_sel=sel)
    assert np.array_equal(part[:T], got[:T, sel])


def _dgrad_case(seed, splits, n, k, E, pad=10):
    rng = np.random.default_rng(seed)
    T = sum(splits)
    dy = torch.from_numpy(rng.standard_normal((T + pad, n)).astype(np.float32)).to(torch.bfloat16)
    dy[T:] = float("nan")  # padding that must never be read
    w = torch.from_numpy(rng.standard_normal((E, n, k)).astype(np.float32)).to(torch.bfloat16)
    dyq = oracle.grouped_quantize(W.bf16_bits(dy), splits, oracle.RECIPE_MX, oracle.ROWWISE)
    # the weight quantized colwise: E groups of n rows, 32-blocks along n inside each expert
    wc = oracle.grouped_quantize(W.bf16_bits(w.view(E * n, k)), [n] * E, oracle.RECIPE_MX, oracle.COLWISE)
    # the same weight transposed per expert, [E*k][n], quantized rowwise (blocks along n)
    wt = w.transpose(1, 2).contiguous().view(E * k, n)
    wr = oracle.grouped_quantize(W.bf16_bits(wt), None, oracle.RECIPE_MX, oracle.ROWWISE)
    return T, dyq, wc, wr


@pytest.mark.parametrize("splits,n,k", [([40, 0, 77], 96, 64), ([128, 5], 256, 32), ([0, 33, 1, 0], 32, 96)])
def test_dgrad_equals_fprop_on_the_transposed_weight(splits, n, k):
    """The colwise weight of dgrad holds exactly the blocks of the rowwise transpose (32 along n),
    so dgrad must reproduce the forward GEMM over W^T value for value: same products, same fp64
    order (c ascending).  Pins the colwise index arithmetic of the dgrad oracle against the
    rowwise path, which is itself pinned to a dense matmul."""
    E = len(splits)
    T, dyq, wc, wr = _dgrad_case(11, splits, n, k, E)
    np_ = 128 * ((n + 127) // 128)
    # the bytes agree element by element under the two layouts
    for e in range(E):
        for j in range(k):
            row = wr["row_q"][e * k + j]
            assert np.array_equal(wc["col_q"][k * np_ * e + j * np_: k * np_ * e + j * np_ + n], row)
            assert not wc["col_q"][k * np_ * e + j * np_ + n: k * np_ * e + (j + 1) * np_].any()  # pad lanes
            for b in range(n // 32):
                assert wc["col_s"][k * np_ * e // 32 + b * k + j] == wr["row_s"][b, e * k + j]
    d = oracle.grouped_dgrad(dyq["row_q"], dyq["row_s"], wc["col_q"], wc["col_s"], k, splits)
    f = oracle.grouped_fprop(dyq["row_q"], dyq["row_s"], wr["row_q"], wr["row_s"], k, splits)
    assert np.array_equal(d, f, equal_nan=True)
    assert np.isnan(d[T:]).all()  # rows outside every group are not written


def test_dgrad_equals_dense_matmul_per_group():
    splits, n, k = [40, 0, 129, 3], 96, 64
    E = len(splits)
    T, dyq, wc, wr = _dgrad_case(12, splits, n, k, E, pad=20)
    got = oracle.grouped_dgrad(dyq["row_q"], dyq["row_s"], wc["col_q"], wc["col_s"], k, splits)
    Y = _rowwise_deq_torch(dyq["row_q"], dyq["row_s"])
    Wt = _rowwise_deq_torch(wr["row_q"], wr["row_s"]).view(E, k, n)  # W_e^T
    off = 0
    for e, ke in enumerate(splits):
        ref = (Y[off:off + ke] @ Wt[e].t()).numpy()  # dy_e @ W_e
        assert np.allclose(got[off:off + ke], ref, rtol=1e-12, atol=1e-300)
        off += ke
    sel = np.array([63, 0, 17], np.int32)
    part = oracle.grouped_dgrad(dyq["row_q"], dyq["row_s"], wc["col_q"], wc["col_s"], k, splits, cols_sel=sel)
    assert np.array_equal(part[:T], got[:T, sel])

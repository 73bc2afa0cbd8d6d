"""Pins of the oracle's scaled SwiGLU (and its gradient) fused with the grouped quantize.

The GLU activations need exp, whose last bits differ between libraries, so the method states its
own fp32 exp2 (range reduction to |r| <= 1/2 and the degree-7 Taylor polynomial of 2^r); the pins
are against the mathematics, in double precision:

* the stated 2^x: exact at integers; relative error <= 3e-7 over [-126, 126]; clamped outside;
  on the reduced range bit-equal to the polynomial with coefficients (ln 2)^n / n! computed from
  their definition;
* silu(a) = a / (1 + e^-a), its derivative sigma(a) (1 + a (1 - sigma(a))), and the product rule
  of the gradient (da, db) against double-precision formulas and a central finite difference;
* the quantized outputs equal the torch MXFP8 route applied to the oracle's own activation values
  laid out as the documented [R, F] (forward) and [R, 2F] = (da | db) (backward) matrices, on
  ragged groups; padding never read.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from test_oracle_quantize import _torch_colwise_mx, _torch_rowwise_mx

FWD, BWD = oracle.ACT_SWIGLU_FWD, oracle.ACT_SWIGLU_BWD


def test_exp2_spec_against_the_exact_power():
    ks = np.arange(-126, 127, dtype=np.float32)
    assert np.array_equal(oracle.exp2_spec(ks), np.ldexp(np.float32(1), ks.astype(np.int64)).astype(np.float32))
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.uniform(-126, 126, 4000), rng.uniform(-2, 2, 4000), [0.5, -0.5, 0.4999999, 125.7]])
    x = x.astype(np.float32)
    got = oracle.exp2_spec(x).astype(np.float64)
    ref = np.array([math.pow(2.0, float(v)) for v in x])
    assert np.max(np.abs(got / ref - 1)) <= 3e-7
    # clamped outside [-126, 126]
    assert oracle.exp2_spec(np.float32([300.0]))[0] == np.float32(2.0 ** 126)
    assert oracle.exp2_spec(np.float32([-300.0]))[0] == np.float32(2.0 ** -126)


def test_exp2_spec_is_the_stated_polynomial():
    """On the reduced range the value is the stated polynomial, bit for bit: coefficients
    (ln 2)^n / n! computed here from their definition and rounded to fp32, Horner order, fp32
    operations."""
    c = [np.float32(math.log(2.0) ** n / math.factorial(n)) for n in range(8)]
    rng = np.random.default_rng(3)
    r = np.concatenate([rng.uniform(-0.5, 0.4999, 5000), [0.0, -0.5, 0.25, -0.25]]).astype(np.float32)
    poly = np.full(r.shape, c[7], np.float32)
    for n in range(6, -1, -1):
        poly = (poly * r + c[n]).astype(np.float32)
    assert np.array_equal(oracle.exp2_spec(r), poly)


def test_silu_and_its_gradient_against_double_precision():
    g = torch.Generator().manual_seed(1)
    a = W.randn_bf16((20000,), g, "cpu", scale=4.0)
    a[:6] = torch.tensor([0.0, -0.0, 30.0, -30.0, 1e-3, -88.0])
    one = torch.ones_like(a)
    af = a.double().numpy()
    silu = af / (1.0 + np.exp(-af))
    sig = 1.0 / (1.0 + np.exp(-af))
    dsilu = sig * (1.0 + af * (1.0 - sig))
    y = oracle.glu_values(FWD, W.bf16_bits(a), W.bf16_bits(one), np.ones(a.numel(), np.float32)).astype(np.float64)
    da, db = oracle.glu_values(BWD, W.bf16_bits(a), W.bf16_bits(one), np.ones(a.numel(), np.float32), W.bf16_bits(one))
    tol = 2e-6 * np.abs(silu) + 1e-30
    assert np.all(np.abs(y - silu) <= tol)
    assert np.array_equal(db, y.astype(np.float32))  # db = dy p silu(a) with dy = p = 1
    # the error scale is that of the terms (the derivative crosses zero near a = -1.28)
    assert np.all(np.abs(da - dsilu) <= 3e-6 * sig * (1.0 + np.abs(af) * (1.0 - sig)) + 1e-12)
    # the derivative against a central difference of the double-precision silu
    hstep = 1e-4
    fd = ((af + hstep) / (1 + np.exp(-(af + hstep))) - (af - hstep) / (1 + np.exp(-(af - hstep)))) / (2 * hstep)
    keep = np.abs(af) < 20
    assert np.all(np.abs(da[keep] - fd[keep]) <= 1e-5 * (1 + np.abs(fd[keep])))


def test_scaling_by_b_and_p_and_dy():
    g = torch.Generator().manual_seed(2)
    n = 4096
    a, b, dy = (W.randn_bf16((n,), g, "cpu") for _ in range(3))
    p = (torch.rand(n, generator=g) - 0.3).numpy().astype(np.float32)
    one = torch.ones(n, dtype=torch.bfloat16)
    s = oracle.glu_values(FWD, W.bf16_bits(a), W.bf16_bits(one), np.ones(n, np.float32))
    y = oracle.glu_values(FWD, W.bf16_bits(a), W.bf16_bits(b), p)
    assert np.array_equal(y, (s * b.float().numpy()) * p)  # y = (silu(a) b) p, fp32 in that order
    da, db = oracle.glu_values(BWD, W.bf16_bits(a), W.bf16_bits(b), p, W.bf16_bits(dy))
    q = dy.float().numpy() * p
    assert np.array_equal(db, q * s)
    d1, _ = oracle.glu_values(BWD, W.bf16_bits(a), W.bf16_bits(one), np.ones(n, np.float32), W.bf16_bits(one))
    assert np.array_equal(da, (q * b.float().numpy()) * d1)


@pytest.mark.parametrize("act", [FWD, BWD])
@pytest.mark.parametrize("splits", [[300, 0, 45, 1, 200], [31, 32, 33, 127, 128, 129], [77]])
def test_glu_quantize_layout(act, splits):
    T = sum(splits)
    R, F = T + 11, 64
    g = torch.Generator().manual_seed(len(splits) + act)
    h = W.randn_bf16((R, 2 * F), g, "cpu", scale=2.0)
    dy = W.randn_bf16((R, F), g, "cpu")
    p = torch.rand(R, generator=g)
    h[T:] = float("nan")
    dy[T:] = float("inf")
    p[T:] = float("nan")
    got = oracle.grouped_act_quantize(act, W.bf16_bits(h), p.numpy(), W.bf16_bits(dy) if act == BWD else None,
                                      splits, oracle.RECIPE_MX, oracle.ROWWISE | oracle.COLWISE)
    a, b = W.bf16_bits(h[:T, :F]), W.bf16_bits(h[:T, F:])
    pp = np.repeat(p[:T].numpy()[:, None], F, axis=1)
    if act == FWD:
        vals = oracle.glu_values(FWD, a, b, pp)
    else:
        da, db = oracle.glu_values(BWD, a, b, pp, W.bf16_bits(dy[:T]))
        vals = np.concatenate([da, db], axis=1)
    y = torch.zeros(R, vals.shape[1])
    y[:T] = torch.from_numpy(vals)
    cq, cs = _torch_colwise_mx(y, splits)
    assert np.array_equal(got["col_q"], cq) and np.array_equal(got["col_s"], cs)
    rq, rs = _torch_rowwise_mx(y, T)
    assert np.array_equal(got["row_q"][:T], rq) and np.array_equal(got["row_s"][:, :T], rs)

"""Pins of the oracle's fused activation + quantize (the ScaledSReLU step between fc1 and fc2 in
the TransformerEngine #3484 reproducer, and its gradient) against independent routes.

* the fp32 activation restated with torch CPU ops in the documented order, then quantized by the
  torch MXFP8 route and the numpy MXFP4 route of the quantize pins: bit-exact, both layouts,
  ragged groups, forward and backward, with and without probs;
* closed forms: p = 1 on non-negative h gives h^2 (exact in fp32 for bf16 h); h <= 0 gives +0
  codes for p >= 0; the gradient is 2 p h dy on h > 0 and zero elsewhere;
* padding rows (garbage, NaN) never change an output.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from test_oracle_fp4 import _np_colwise, _np_rowwise
from test_oracle_quantize import _torch_colwise_mx, _torch_rowwise_mx

FWD, BWD = oracle.ACT_SRELU_FWD, oracle.ACT_SRELU_BWD


def _torch_act(act, h, p, dy):
    hf = h.float()
    r = torch.where(hf > 0, hf, torch.zeros_like(hf))
    pc = torch.ones(h.shape[0], 1) if p is None else p.float()[:, None]
    if act == FWD:
        return (r * r) * pc
    return ((2.0 * r) * pc) * dy.float()


def _case(R, C, splits, seed, negative_probs=False):
    g = torch.Generator().manual_seed(seed)
    h = W.randn_bf16((R, C), g, "cpu", scale=2.0)
    dy = W.randn_bf16((R, C), g, "cpu", scale=0.5)
    p = torch.rand(R, generator=g, dtype=torch.float32)
    if negative_probs:
        p = p - 0.5
    T = sum(splits)
    rng = np.random.default_rng(seed)
    for t in (h, dy):  # garbage padding, NaN/Inf included
        bits = rng.integers(0, 1 << 16, size=(R - T, C), dtype=np.uint16)
        t[T:] = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    p[T:] = float("nan")
    return h, dy, p


@pytest.mark.parametrize("act", [FWD, BWD])
def test_activation_values_bitwise_against_torch(act):
    """Element by element against torch's IEEE fp32 products in the documented order: catches a
    reordered product (r (r p) differs from (r r) p in about a third of the elements)."""
    g = torch.Generator().manual_seed(11)
    n = 1 << 16
    h = W.randn_bf16((n,), g, "cpu", scale=3.0)
    h[:4] = torch.tensor([0.0, -0.0, -1.0, 1.0])
    dy = W.randn_bf16((n,), g, "cpu")
    p = torch.rand(n, generator=g) * 2 - 0.5
    got = oracle.act_values(act, W.bf16_bits(h), p.numpy(), W.bf16_bits(dy) if act == BWD else None)
    r = torch.where(h.float() > 0, h.float(), torch.zeros(n))
    ref = (r * r) * p if act == FWD else ((2.0 * r) * p) * dy.float()
    assert np.array_equal(got.view(np.uint32), ref.numpy().view(np.uint32))
    # the reordered product does differ on this data, so the comparison above can tell
    alt = r * (r * p) if act == FWD else (2.0 * r) * (p * dy.float())
    assert (alt != ref).float().mean() > 0.05


@pytest.mark.parametrize("act", [FWD, BWD])
@pytest.mark.parametrize("splits", [[300, 0, 45, 1, 200], [31, 32, 33, 127, 128, 129], [77]])
@pytest.mark.parametrize("with_probs", [True, False])
def test_act_quantize_matches_torch_route_mxfp8(act, splits, with_probs):
    T = sum(splits)
    R, C = T + 19, 96
    h, dy, p = _case(R, C, splits, seed=len(splits) + act)
    probs = p if with_probs else None
    got = oracle.grouped_act_quantize(act, W.bf16_bits(h), None if probs is None else probs.numpy(),
                                      W.bf16_bits(dy) if act == BWD else None, splits, oracle.RECIPE_MX,
                                      oracle.ROWWISE | oracle.COLWISE)
    y = torch.zeros(R, C)
    y[:T] = _torch_act(act, h[:T], None if probs is None else probs[:T], dy[:T])
    cq, cs = _torch_colwise_mx(y, splits)
    assert np.array_equal(got["col_q"], cq) and np.array_equal(got["col_s"], cs)
    rq, rs = _torch_rowwise_mx(y, T)
    assert np.array_equal(got["row_q"][:T], rq) and np.array_equal(got["row_s"][:, :T], rs)


@pytest.mark.parametrize("act", [FWD, BWD])
def test_act_quantize_matches_numpy_route_mxfp4(act):
    splits = [130, 0, 257, 31]
    T = sum(splits)
    R, C = T + 7, 64
    h, dy, p = _case(R, C, splits, seed=9, negative_probs=True)
    got = oracle.grouped_act_quantize(act, W.bf16_bits(h), p.numpy(), W.bf16_bits(dy) if act == BWD else None,
                                      splits, oracle.RECIPE_MX4, oracle.ROWWISE | oracle.COLWISE)
    y = np.zeros((R, C))
    y[:T] = _torch_act(act, h[:T], p[:T], dy[:T]).double().numpy()
    cq, cs = _np_colwise(y, splits)
    assert np.array_equal(got["col_q"], cq) and np.array_equal(got["col_s"], cs)
    rq, rs = _np_rowwise(y, T)
    assert np.array_equal(got["row_q"][:T], rq) and np.array_equal(got["row_s"][:, :T], rs)


def test_closed_forms():
    splits = [64]
    C = 32
    # non-negative h, p = 1: the squares themselves (exact in fp32 for bf16 inputs)
    g = torch.Generator().manual_seed(3)
    h = W.randn_bf16((64, C), g, "cpu").abs()
    sq = oracle.grouped_act_quantize(FWD, W.bf16_bits(h), None, None, splits, oracle.RECIPE_MX, oracle.ROWWISE)
    exact = (h.double() ** 2).float()
    assert torch.equal(exact.double(), h.double() ** 2)
    rq, rs = _torch_rowwise_mx(exact, 64)
    assert np.array_equal(sq["row_q"], rq) and np.array_equal(sq["row_s"], rs)
    # h <= 0 (including -0): every code is +0 for p >= 0, and the block exponent is -127
    hn = -W.randn_bf16((64, C), g, "cpu").abs()
    hn[0] = -0.0
    z = oracle.grouped_act_quantize(FWD, W.bf16_bits(hn), np.full(64, 0.7, np.float32), None, splits,
                                    oracle.RECIPE_MX, oracle.ROWWISE | oracle.COLWISE)
    assert not z["row_q"].any() and not z["col_q"].any()
    assert (z["row_s"] == 0).all() and (z["col_s"] == 0).all()
    # gradient: 2 p h dy on h > 0 (exact: 2 h and the product with p = 1 and dy = 1 are exact)
    ones = torch.ones(64, C, dtype=torch.bfloat16)
    gr = oracle.grouped_act_quantize(BWD, W.bf16_bits(h), None, W.bf16_bits(ones), splits, oracle.RECIPE_MX,
                                     oracle.ROWWISE)
    rq, rs = _torch_rowwise_mx((2.0 * h.float()), 64)
    assert np.array_equal(gr["row_q"], rq) and np.array_equal(gr["row_s"], rs)


@pytest.mark.parametrize("act", [FWD, BWD])
def test_padding_never_read(act):
    splits = [100, 0, 60]
    T = sum(splits)
    h, dy, p = _case(T + 40, 64, splits, seed=5)
    a = oracle.grouped_act_quantize(act, W.bf16_bits(h), p.numpy(), W.bf16_bits(dy) if act == BWD else None,
                                    splits, oracle.RECIPE_MX, oracle.ROWWISE | oracle.COLWISE)
    b = oracle.grouped_act_quantize(act, W.bf16_bits(h[:T]), p[:T].numpy(),
                                    W.bf16_bits(dy[:T]) if act == BWD else None, splits, oracle.RECIPE_MX,
                                    oracle.ROWWISE | oracle.COLWISE)
    assert np.array_equal(a["col_q"], b["col_q"]) and np.array_equal(a["col_s"], b["col_s"])
    assert np.array_equal(a["row_q"][:T], b["row_q"]) and np.array_equal(a["row_s"][:, :T], b["row_s"])

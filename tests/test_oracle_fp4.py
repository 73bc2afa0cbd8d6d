"""Pins of the oracle's MXFP4 path (e2m1 codec, the 6 * 2^e scale rule, the packed layouts and
the three GEMMs over packed operands) against routes that share nothing with it.

* e2m1 decode: the 16 values the OCP FP4 E2M1 format defines (sign, 2 exponent bits with bias 1,
  1 mantissa bit, no NaN or infinity).
* e2m1 encode: exact rational nearest-value search over every bf16 value below 8 in magnitude,
  the seven rounding ties, saturation and signed zero.
* scale rule: the defining inequality in exact arithmetic on every positive bf16 amax, and a
  frexp closed form (amax = m 2^E, 6 = 0.75 2^3: e = E - 3, plus one when m > 0.75).
* layouts: a numpy route (the frexp exponent, the e2m1 code as a count of rounding thresholds,
  nibble packing written out) on ragged groups, rowwise and colwise.
* GEMMs: float64 matmuls of the numpy-dequantized packed operands, and the unquantized brute
  force within the e2m1 quantization bound.
"""
import fractions

import numpy as np
import pytest
import torch

import oracle
import workloads as W

MX4 = oracle.RECIPE_MX4
OCP_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]  # codes 0..7; codes 8..15 are the negatives


def _all_bf16_as_f32():
    return (np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32)


def test_decode_all_codes_match_the_format_table():
    got = oracle.e2m1_decode(np.arange(16, dtype=np.uint8))
    for c in range(16):
        mag = OCP_E2M1[c & 7]
        want = -mag if c & 8 else mag
        assert got[c] == want and np.signbit(got[c]) == bool(c & 8), c


def _brute_force_code(v):
    """Nearest of the 8 magnitudes in exact arithmetic; ties to the even code; >= 6 gives 6."""
    a = abs(fractions.Fraction(float(v)))
    sign = 8 if np.signbit(v) else 0
    if a >= 6:
        return sign | 7
    best = None
    for c, m in enumerate(OCP_E2M1):
        d = abs(a - fractions.Fraction(m))
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0 and best[1] % 2 == 1):
            best = (d, c)
    return sign | best[1]


def test_encode_matches_exact_nearest_search_on_bf16():
    v = _all_bf16_as_f32()
    v = v[np.isfinite(v) & (np.abs(v) < 8.0)]
    got = oracle.e2m1_encode(v)
    step = 7  # every 7th value in exact arithmetic (about 4,800 values), all of them below
    for x, g in zip(v[::step].tolist(), got[::step].tolist()):
        assert g == _brute_force_code(np.float32(x)), x
    # all values: the threshold form of round-to-nearest-even (a second derivation)
    a = np.abs(v.astype(np.float64))
    code = ((a > 0.25).astype(int) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5) + (a >= 3.5) + (a > 5.0))
    code = code + 8 * np.signbit(v)
    assert np.array_equal(got, code.astype(np.uint8))


def test_encode_ties_saturation_and_sign():
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for t, c in ties.items():
        assert oracle.e2m1_encode(np.float32([t]))[0] == c, t
        assert oracle.e2m1_encode(np.float32([-t]))[0] == c | 8, -t
        up, dn = np.nextafter(np.float32(t), np.float32(9)), np.nextafter(np.float32(t), np.float32(0))
        assert oracle.e2m1_encode(np.float32([up]))[0] == _brute_force_code(up)
        assert oracle.e2m1_encode(np.float32([dn]))[0] == _brute_force_code(dn)
    assert list(oracle.e2m1_encode(np.float32([6.0, 7.0, 1e30, -6.5]))) == [7, 7, 7, 15]
    assert list(oracle.e2m1_encode(np.float32([0.0, -0.0, -1e-30]))) == [0, 8, 8]


def test_fp4_scale_rule_on_every_positive_bf16():
    v = _all_bf16_as_f32()
    v = v[np.isfinite(v) & (v > 0)]
    e = oracle.e8m0_exponent_fp4(v)
    assert e.min() >= -127 and e.max() <= 127
    for a, ex in zip(v[::37].tolist(), e[::37].tolist()):
        fa = fractions.Fraction(a)
        assert fa <= 6 * fractions.Fraction(2) ** ex
        if ex > -127:
            assert fa > 6 * fractions.Fraction(2) ** (ex - 1)
    scaled = v.astype(np.float64) * np.ldexp(1.0, -e.astype(np.int64))
    assert np.all(scaled <= 6.0)
    assert np.all(scaled[e > -127] > 3.0)
    m, E = np.frexp(v.astype(np.float64))
    assert np.array_equal(e, np.clip(E - 3 + (m > 0.75), -127, 127))
    assert oracle.e8m0_exponent_fp4(np.float32([0.0]))[0] == -127


# ------------------------------------------------------------------------------------------
# layouts: a numpy route
# ------------------------------------------------------------------------------------------

def _np_exponent(amax):
    m, E = np.frexp(amax.astype(np.float64))
    e = np.clip(E - 3 + (m > 0.75), -127, 127)
    return np.where(amax == 0, -127, e).astype(np.int64)


def _np_codes(y):
    a = np.abs(y)
    c = ((a > 0.25).astype(np.int64) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5) + (a >= 3.5) + (a > 5.0))
    return (c + 8 * np.signbit(y)).astype(np.uint8)


def _np_pack(codes):
    """codes [..., 2m] -> bytes [..., m]: element 2i in the low nibble, 2i + 1 in the high one."""
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def _np_blocks(v):
    """v float64 [nb, 32, C] (zeros where not live) -> (codes [nb, 32, C], exponents [nb, C])."""
    e = _np_exponent(np.abs(v).max(axis=1))
    return _np_codes(v * np.ldexp(1.0, -e)[:, None, :]), e


def _np_colwise(x, splits):
    C = x.shape[1]
    qs, ss, off = [], [], 0
    for k in splits:
        kp = 128 * ((k + 127) // 128)
        blk = np.zeros((kp, C))
        blk[:k] = x[off:off + k]
        q, e = _np_blocks(blk.reshape(kp // 32, 32, C))
        qs.append(_np_pack(q.reshape(kp, C).T).reshape(-1))  # each channel's tokens, packed
        ss.append((e + 127).astype(np.uint8).reshape(-1))
        off += k
    return np.concatenate(qs), np.concatenate(ss)


def _np_rowwise(x, T):
    C = x.shape[1]
    v = x[:T].reshape(T, C // 32, 32).transpose(0, 2, 1)  # [T, 32, C/32]
    q, e = _np_blocks(v)
    q = q.transpose(0, 2, 1).reshape(T, C)
    return _np_pack(q), (e + 127).astype(np.uint8).T


@pytest.mark.parametrize("splits", [[300, 0, 45, 1, 200], [31, 32, 33, 127, 128, 129], [0, 0, 5], [77]])
def test_mx4_layouts_match_numpy_route(splits):
    T = sum(splits)
    R, C = T + 24, 96
    g = torch.Generator().manual_seed(41)
    x = W.randn_bf16((R, C), g, "cpu", scale=3.0)
    x[T:] = 3.0  # padding, never read
    xb = W.bf16_bits(x)
    xf = x.double().numpy()
    got = oracle.grouped_quantize(xb, splits, MX4, oracle.COLWISE | oracle.ROWWISE)
    cq, cs = _np_colwise(xf, splits)
    assert np.array_equal(got["col_q"], cq)
    assert np.array_equal(got["col_s"], cs)
    rq, rs = _np_rowwise(xf, T)
    assert np.array_equal(got["row_q"][:T], rq)
    assert np.array_equal(got["row_s"][:, :T], rs)
    assert not got["row_q"][T:].any()
    assert got["col_q"].size == C * oracle.padded_rows(splits) // 2


def test_mx4_rowwise_without_splits_and_special_values():
    v = np.float32([0, -0.0, 1e-30, -1e-30, 6, -6, 0.25, 448, 3e38, -3e38, 1, 2, 3, 4, 5, 7] * 2).reshape(1, 32)
    xb = (v.view(np.uint32) >> 16).astype(np.uint16)  # every value above is a bf16 value
    x = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    got = oracle.grouped_quantize(xb, None, MX4, oracle.ROWWISE)
    rq, rs = _np_rowwise(x, 1)
    assert np.array_equal(got["row_q"], rq) and np.array_equal(got["row_s"], rs)


# ------------------------------------------------------------------------------------------
# GEMMs over packed operands
# ------------------------------------------------------------------------------------------

def _unpack(b):
    """bytes [..., m] -> codes [..., 2m]."""
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.uint8)
    out[..., 0::2] = b & 15
    out[..., 1::2] = b >> 4
    return out


def _dec(codes):
    mag = np.array(OCP_E2M1)[codes & 7]
    return np.where(codes & 8, -mag, mag)


def _deq_colwise(col_q, col_s, C, splits):
    vals = _dec(_unpack(col_q))
    out, p = [], 0
    for k in splits:
        kp = 128 * ((k + 127) // 128)
        q = vals[C * p: C * (p + kp)].reshape(C, kp).T  # [kp, C]
        s = np.ldexp(1.0, col_s[C * p // 32: C * (p + kp) // 32].astype(np.int64) - 127).reshape(kp // 32, C)
        out.append(q[:k] * np.repeat(s, 32, axis=0)[:k])
        p += kp
    return out


def _deq_rowwise(row_q, row_s):
    v = _dec(_unpack(row_q))
    return v * np.repeat(np.ldexp(1.0, row_s.astype(np.int64) - 127).T, 32, axis=1)


def test_mx4_wgrad_equals_dense_matmul_per_group():
    splits = [70, 0, 130, 33]
    T = sum(splits)
    R, n, h = T + 20, 64, 96
    g = torch.Generator().manual_seed(43)
    dy = W.randn_bf16((R, n), g, "cpu")
    x = W.randn_bf16((R, h), g, "cpu")
    dq = oracle.grouped_quantize(W.bf16_bits(dy), splits, MX4, oracle.COLWISE)
    xq = oracle.grouped_quantize(W.bf16_bits(x), splits, MX4, oracle.COLWISE)
    got = oracle.grouped_wgrad(dq["col_q"], dq["col_s"], n, xq["col_q"], xq["col_s"], h, splits, R, MX4)
    A, B = _deq_colwise(dq["col_q"], dq["col_s"], n, splits), _deq_colwise(xq["col_q"], xq["col_s"], h, splits)
    for e in range(len(splits)):
        ref = A[e].T @ B[e]
        assert np.allclose(got[e], ref, rtol=1e-12, atol=1e-300), e
    assert not got[1].any()
    # the unquantized sums, within the e2m1 bound: half a step of the value's binade (at most a
    # quarter of |v|, or a quarter of the block scale below it)
    unq = oracle.wgrad_unquantized(W.bf16_bits(dy), W.bf16_bits(x), splits, R)
    off = 0
    for e, k in enumerate(splits):
        a, b = dy[off:off + k].double().numpy(), x[off:off + k].double().numpy()
        sa = _block_scales(dq["col_s"], n, splits, e)
        sb = _block_scales(xq["col_s"], h, splits, e)
        da = 0.25 * np.abs(a) + 0.25 * sa
        db = 0.25 * np.abs(b) + 0.25 * sb
        bound = da.T @ (np.abs(b) + db) + np.abs(a).T @ db
        assert np.all(np.abs(got[e] - unq[e]) <= bound * (1 + 1e-12) + 1e-300)
        off += k


def _block_scales(col_s, C, splits, e):
    p = sum(128 * ((k + 127) // 128) for k in splits[:e])
    k = splits[e]
    kp = 128 * ((k + 127) // 128)
    s = np.ldexp(1.0, col_s[C * p // 32: C * (p + kp) // 32].astype(np.int64) - 127).reshape(kp // 32, C)
    return np.repeat(s, 32, axis=0)[:k]


def test_mx4_fprop_and_dgrad_equal_dense_matmul_per_group():
    splits = [40, 0, 77, 129]
    T = sum(splits)
    R, K, N, E = T + 9, 96, 64, len(splits)
    g = torch.Generator().manual_seed(44)
    x = W.randn_bf16((R, K), g, "cpu")
    w = W.randn_bf16((E * N, K), g, "cpu")
    xq = oracle.grouped_quantize(W.bf16_bits(x), splits, MX4, oracle.ROWWISE)
    wq = oracle.grouped_quantize(W.bf16_bits(w), None, MX4, oracle.ROWWISE)
    got = oracle.grouped_fprop(xq["row_q"], xq["row_s"], wq["row_q"], wq["row_s"], N, splits, recipe=MX4)
    X, Wd = _deq_rowwise(xq["row_q"], xq["row_s"]), _deq_rowwise(wq["row_q"], wq["row_s"])
    off = 0
    for e, k in enumerate(splits):
        ref = X[off:off + k] @ Wd[e * N:(e + 1) * N].T
        assert np.allclose(got[off:off + k], ref, rtol=1e-12, atol=1e-300)
        off += k
    assert np.isnan(got[T:]).all()
    # dgrad: dy [R, n] rowwise, the weight [E*n, k] colwise along n with splits [n] * E
    n, k = 64, 96
    dy = W.randn_bf16((R, n), g, "cpu")
    wt = W.randn_bf16((E * n, k), g, "cpu")
    dq = oracle.grouped_quantize(W.bf16_bits(dy), splits, MX4, oracle.ROWWISE)
    wc = oracle.grouped_quantize(W.bf16_bits(wt), [n] * E, MX4, oracle.COLWISE)
    got = oracle.grouped_dgrad(dq["row_q"], dq["row_s"], wc["col_q"], wc["col_s"], k, splits, recipe=MX4)
    Y = _deq_rowwise(dq["row_q"], dq["row_s"])
    Wc = _deq_colwise(wc["col_q"], wc["col_s"], k, [n] * E)  # per expert [n, k]
    off = 0
    for e, ke in enumerate(splits):
        ref = Y[off:off + ke] @ Wc[e]
        assert np.allclose(got[off:off + ke], ref, rtol=1e-12, atol=1e-300)
        off += ke
    assert np.isnan(got[T:]).all()

"""Pins of the oracle's e4m3 codec and MXFP8 scale rule against things fixed outside it.

* decode: every one of the 256 codes against torch's float8_e4m3fn (a library routine).
* encode: against torch's float8_e4m3fn conversion and against a brute-force nearest-value
  search written here with numpy, on every rounding boundary of the format (all fp32 patterns
  that share their top 10 mantissa bits with a boundary region, with several low-bit tails),
  on every bf16 value, and on a random sample of fp32 patterns.
* E8M0 rule: on every positive finite bf16 amax, the defining property checked in exact
  integer arithmetic, and the closed-form band 224 < amax * 2^-e <= 448 when e is not clamped.
"""
import fractions

import numpy as np
import pytest
import torch

import oracle


def _torch_e4m3(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _all_bf16_as_f32():
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    return bits.view(np.float32)


def _finite_table():
    """Non-negative finite e4m3 magnitudes by code, from torch's decoder."""
    codes = np.arange(127, dtype=np.uint8)
    return torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _brute_force_encode(v):
    """Nearest finite e4m3 code by exhaustive distance to all 127 magnitudes; ties to even code."""
    tab = _finite_table()
    a = np.abs(v.astype(np.float64))
    d = np.abs(a[:, None] - tab[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    even = cand & ((np.arange(127) % 2) == 0)[None, :]
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    pick = np.where(a >= 448.0, 126, pick)
    return (pick | (np.signbit(v).astype(np.int64) << 7)).astype(np.uint8)


def test_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(got[~nan], ref[~nan])
    # sign of zero is kept
    assert np.signbit(got[0x80]) and not np.signbit(got[0x00])


def _boundary_patterns():
    """All fp32 patterns with |v| < 2^9 whose low 13 mantissa bits are one of several tails.

    Every midpoint between neighbouring e4m3 values has at most 5 significant bits, so its
    pattern and both its fp32 neighbours appear here, for every exponent and sign."""
    tails = np.array([0, 1, 0x0FFF, 0x1000, 0x1001, 0x1FFF], dtype=np.uint32)
    heads = np.arange(1 << 19, dtype=np.uint32) << 13  # sign, exponent, top 10 mantissa bits
    pats = (heads[:, None] | tails[None, :]).ravel()
    v = pats.view(np.float32)
    keep = np.isfinite(v) & (np.abs(v) < 464.0)
    return v[keep]


def test_encode_matches_torch_on_boundaries_bf16_and_random():
    rng = np.random.default_rng(0)
    rand = rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32).view(np.float32)
    for v in (_boundary_patterns(), _all_bf16_as_f32(), rand):
        v = v[np.isfinite(v) & (np.abs(v) < 464.0)]
        got = oracle.e4m3_encode(v)
        ref = _torch_e4m3(v)
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, f"{bad.size} mismatches, first v={v[bad[0]]!r} got {got[bad[0]]:#x} torch {ref[bad[0]]:#x}"


def test_encode_matches_brute_force_search():
    v = _boundary_patterns()
    rng = np.random.default_rng(1)
    idx = rng.choice(v.size, 200_000, replace=False)
    v = np.concatenate([v[idx], np.float32([0.0, -0.0, 448.0, -448.0, 450.0, 463.9, 1e-30, -1e-30])])
    got = oracle.e4m3_encode(v)
    ref = np.concatenate([_brute_force_encode(v[i:i + 20000]) for i in range(0, v.size, 20000)])
    assert np.array_equal(got, ref)


def test_encode_saturates_and_keeps_sign():
    v = np.float32([448.0, 464.0, 1e6, 3.0e38, -464.0, -1e9, -0.0, -1e-12, 1e-12])
    got = oracle.e4m3_encode(v)
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x80, 0x80, 0x00]


def test_e8m0_rule_on_every_positive_bf16():
    v = _all_bf16_as_f32()
    v = v[np.isfinite(v) & (v > 0)]
    e = oracle.e8m0_exponent(v)
    assert e.min() >= -127 and e.max() <= 127
    # defining property in exact arithmetic: amax <= 448 * 2^e, and e is the smallest such
    # (or clamped at -127)
    for a, ex in zip(v[::37].tolist(), e[::37].tolist()):
        fa = fractions.Fraction(a)
        assert fa <= 448 * fractions.Fraction(2) ** ex
        if ex > -127:
            assert fa > 448 * fractions.Fraction(2) ** (ex - 1)
    # closed-form band for every value (float64 is exact for these products)
    scaled = v.astype(np.float64) * np.ldexp(1.0, -e.astype(np.int64))
    unclamped = e > -127
    assert np.all(scaled <= 448.0)
    assert np.all(scaled[unclamped] > 224.0)
    assert oracle.e8m0_exponent(np.float32([0.0]))[0] == -127


def test_e8m0_rule_matches_frexp_route():
    """Second route: amax = m * 2^E with m in [0.5, 1); 448 = 0.875 * 2^9, so the smallest e with
    amax <= 448 * 2^e is E - 9, plus one when m > 0.875; clamped to [-127, 127]."""
    v = _all_bf16_as_f32()
    v = v[np.isfinite(v) & (v > 0)]
    m, E = np.frexp(v.astype(np.float64))
    ref = np.clip(E - 9 + (m > 0.875), -127, 127)
    assert np.array_equal(oracle.e8m0_exponent(v), ref)

"""Pins of the oracle's grouped quantize (both recipes, both layouts) against independent routes.

* Per-channel 128-row recipe: the recipe's definition (DeepGEMM #365, "Non-deterministic
  numerical problem of k_grouped_fp8_gemm_nt_contiguous", reproducer: fp32 amax, divide by
  448, zero -> sf_val, clamp at 1e-30, multiply by the fp32 reciprocal, e4m3 conversion; each
  expert's tokens packed K-major, experts back to back) written out as an explicit loop over
  experts and 128-token blocks in numpy, on that page's shapes, where every expert count is a
  multiple of 128.
* MXFP8 1x32: a torch route that takes the exponent from frexp and converts with torch, and
  unpacks the group layout with torch reshapes, on ragged groups (counts not multiples of 32,
  empty groups) — this pins offsets, per-group block restarts and pad lanes.
* Invariants: padding contents (0.0, 3.0, random bits with NaN/Inf) never change any output.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W


def _e8m0_torch(amax):
    m, E = torch.frexp(amax.double())
    e = E - 9 + (m > 0.875).to(E.dtype)
    e = torch.where(amax == 0, torch.full_like(e, -127), e)
    return e.clamp(-127, 127)


def _mx_blocks_torch(v):
    """v: float32 [nb, 32, C] blocks (zeros where not live) -> (codes uint8 [nb,32,C], exps [nb,C])."""
    amax = v.abs().amax(dim=1)
    e = _e8m0_torch(amax)
    scaled = v.double() * torch.pow(2.0, -e.double())[:, None, :]
    q = scaled.float().to(torch.float8_e4m3fn).view(torch.uint8)
    return q, e


def _torch_colwise_mx(x, splits):
    """Expected colwise bytes / scales from torch, packing per group K-major."""
    C = x.shape[1]
    q_parts, s_parts, off = [], [], 0
    for k in splits:
        kp = 128 * ((k + 127) // 128)
        blk = torch.zeros(kp, C, dtype=torch.float32)
        blk[:k] = x[off:off + k].float()
        q, e = _mx_blocks_torch(blk.view(kp // 32, 32, C))
        q_parts.append(q.view(kp, C).t().contiguous().view(-1))
        s_parts.append((e + 127).to(torch.uint8).view(-1))
        off += k
    return torch.cat(q_parts).numpy(), torch.cat(s_parts).numpy()


def _torch_rowwise_mx(x, T):
    R, C = x.shape
    v = x[:T].float().view(T, C // 32, 32).transpose(1, 2)  # [T, 32, C/32]: blocks along dim 1
    q, e = _mx_blocks_torch(v)
    q = q.transpose(1, 2).reshape(T, C)
    return q.numpy(), (e + 127).to(torch.uint8).t().contiguous().numpy()  # scales [C/32, T]


def _per_channel_expected(x_live, splits, sf_val):
    """The per-channel 128-row recipe written out group by group and block by block, in numpy
    fp32: for each expert, each 128-token block and every channel, the block's amax, the scale
    fp32(amax / 448) (sf_val where that is zero, never below 1e-30), and the codes of
    v * fp32(1 / scale) by torch's e4m3 conversion; each expert's codes laid out channel by
    channel (its tokens contiguous), experts back to back, scales [block][channel] per expert."""
    x = x_live.float().numpy()
    C = x.shape[1]
    codes, scales, off = [], [], 0
    for k in splits:
        assert k % 128 == 0
        q_e = np.zeros((C, k), np.uint8)
        s_e = np.zeros((k // 128, C), np.float32)
        for b in range(k // 128):
            rows = x[off + 128 * b: off + 128 * (b + 1)]           # [128][C]
            amax = np.abs(rows).max(axis=0).astype(np.float32)
            sf = (amax / np.float32(448.0)).astype(np.float32)
            sf = np.where(sf == 0, np.float32(sf_val), sf).astype(np.float32)
            sf = np.maximum(sf, np.float32(1e-30))
            r = (np.float32(1.0) / sf).astype(np.float32)
            v = (rows * r[None, :]).astype(np.float32)
            q = torch.from_numpy(np.ascontiguousarray(v)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            q_e[:, 128 * b: 128 * (b + 1)] = q.T
            s_e[b] = sf
        codes.append(q_e.reshape(-1))
        scales.append(s_e.reshape(-1))
        off += k
    return np.concatenate(codes), np.concatenate(scales)


@pytest.mark.parametrize("n,sf_val", [(256, 1e-30), (2048, 1e-30), (256, 1.0), (256, 1e-4)])
def test_per_channel_matches_page_recipe(n, sf_val):
    case = W.deepgemm_case("cpu", n, n, R=1024 if n == 256 else None)
    T = case["T"]
    for name in ("dy", "x"):
        buf = case[name]
        got = oracle.grouped_quantize(W.bf16_bits(buf), case["splits"], oracle.RECIPE_PC, oracle.COLWISE,
                                      zero_amax_scale=sf_val)
        q, sf = _per_channel_expected(buf[:T], case["splits"], sf_val)
        assert np.array_equal(got["col_q"], q), name
        assert np.array_equal(got["col_s"].view(np.uint32), sf.view(np.uint32)), name
    # the zeroed dy channel of the 128-token experts gets sf_val (clamped at 1e-30)
    got = oracle.grouped_quantize(W.bf16_bits(case["dy"]), case["splits"], oracle.RECIPE_PC, oracle.COLWISE,
                                  zero_amax_scale=sf_val)
    s = got["col_s"].reshape(-1, n)
    assert s[2, 0] == np.float32(max(sf_val, 1e-30)) and s[3, 0] == np.float32(max(sf_val, 1e-30))


@pytest.mark.parametrize("splits", [[300, 0, 45, 1, 200], [31, 32, 33, 127, 128, 129], [0, 0, 5], [77]])
def test_mx_colwise_matches_torch_route_ragged(splits):
    rng = np.random.default_rng(sum(splits))
    T = sum(splits)
    C = 96
    x = torch.from_numpy(rng.standard_normal((T + 40, C)).astype(np.float32)).to(torch.bfloat16)
    x[:T:7] *= 1e-3  # mixed magnitudes so blocks get different exponents
    x[T:] = float("nan")  # padding that must never be read
    got = oracle.grouped_quantize(W.bf16_bits(x), splits, oracle.RECIPE_MX, oracle.COLWISE | oracle.ROWWISE)
    q_ref, s_ref = _torch_colwise_mx(x, splits)
    assert np.array_equal(got["col_q"], q_ref)
    assert np.array_equal(got["col_s"], s_ref)
    rq, rs = _torch_rowwise_mx(x, T)
    assert np.array_equal(got["row_q"][:T], rq)
    assert np.array_equal(got["row_s"][:, :T], rs)
    assert not got["row_q"][T:].any() and not got["row_s"][:, T:].any()  # padding rows untouched


def test_rowwise_without_splits_covers_all_rows():
    rng = np.random.default_rng(7)
    x = torch.from_numpy(rng.standard_normal((64, 128)).astype(np.float32)).to(torch.bfloat16)
    got = oracle.grouped_quantize(W.bf16_bits(x), None, oracle.RECIPE_MX, oracle.ROWWISE)
    rq, rs = _torch_rowwise_mx(x, 64)
    assert np.array_equal(got["row_q"], rq) and np.array_equal(got["row_s"], rs)


def test_pad_lanes_zero_and_dequant_error_bound():
    rng = np.random.default_rng(3)
    splits = [45, 0, 130]
    T, C = sum(splits), 64
    x = torch.from_numpy(rng.standard_normal((T, C)).astype(np.float32)).to(torch.bfloat16)
    got = oracle.grouped_quantize(W.bf16_bits(x), splits, oracle.RECIPE_MX, oracle.COLWISE)
    P = 0
    xf = x.double().numpy()
    for e, k in enumerate(splits):
        kp = 128 * ((k + 127) // 128)
        q = got["col_q"][C * P:C * (P + kp)].reshape(C, kp)
        s = got["col_s"][C * P // 32:C * (P + kp) // 32].reshape(kp // 32, C)
        assert not q[:, k:].any()  # pad lanes hold 0x00
        deq = oracle.e4m3_decode(q) * np.ldexp(1.0, s.astype(np.int64) - 127).T.repeat(32, axis=1)
        ref = xf[sum(splits[:e]):sum(splits[:e]) + k].T
        scale = np.ldexp(1.0, s.astype(np.int64) - 127).T.repeat(32, axis=1)[:, :k]
        bound = 2.0 ** -4 * np.abs(ref) + 2.0 ** -10 * scale
        assert np.all(np.abs(deq[:, :k] - ref) <= bound)
        P += kp


@pytest.mark.parametrize("recipe", [oracle.RECIPE_MX, oracle.RECIPE_PC])
def test_padding_contents_never_matter(recipe):
    outs = []
    for fill in (0.0, 3.0, "garbage"):
        rng = np.random.default_rng(11)
        case = W.deepgemm_case("cpu", 64, 96, splits=(256, 128, 0, 128, 40), R=700,
                               pad_fill=0.0 if fill == "garbage" else fill)
        if fill == "garbage":
            bits = rng.integers(0, 1 << 16, size=(700 - case["T"], 64), dtype=np.uint16)
            case["dy"][case["T"]:] = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
        which = oracle.COLWISE | (oracle.ROWWISE if recipe == oracle.RECIPE_MX else 0)
        o = oracle.grouped_quantize(W.bf16_bits(case["dy"]), case["splits"], recipe, which)
        outs.append(o)
    for o in outs[1:]:
        for key in outs[0]:
            assert np.array_equal(np.asarray(o[key]).view(np.uint8), np.asarray(outs[0][key]).view(np.uint8)), key


def test_group_independence():
    """Quantizing a multi-group buffer equals quantizing each group alone, placed at its slot."""
    rng = np.random.default_rng(5)
    splits = [129, 0, 31, 256]
    C = 64
    x = torch.from_numpy(rng.standard_normal((sum(splits), C)).astype(np.float32)).to(torch.bfloat16)
    for recipe in (oracle.RECIPE_MX, oracle.RECIPE_PC):
        whole = oracle.grouped_quantize(W.bf16_bits(x), splits, recipe, oracle.COLWISE)
        qs, ss, off = [], [], 0
        for k in splits:
            part = oracle.grouped_quantize(W.bf16_bits(x[off:off + k]) if k else np.zeros((0, C), np.uint16),
                                           [k], recipe, oracle.COLWISE)
            qs.append(part["col_q"])
            ss.append(part["col_s"])
            off += k
        assert np.array_equal(whole["col_q"], np.concatenate(qs))
        assert np.array_equal(whole["col_s"], np.concatenate(ss))


@pytest.mark.parametrize("sf_val", [0.0, 1e-40, 1e-30])
def test_per_channel_clamp_on_tiny_amax(sf_val):
    """Blocks whose amax / 448 underflows 1e-30, and a zero-amax replacement below 1e-30, are
    both clamped to 1e-30 (the reproducer's clamp_min); checked against the written-out recipe."""
    rng = np.random.default_rng(2)
    x = torch.from_numpy(rng.standard_normal((256, 64)).astype(np.float32) * 1e-29).to(torch.bfloat16)
    x[:, 3] = 0.0          # zero channel -> sf_val, then the clamp
    x[128:, 5] *= 1e-8     # amax/448 far below 1e-30
    got = oracle.grouped_quantize(W.bf16_bits(x), [256], oracle.RECIPE_PC, oracle.COLWISE, zero_amax_scale=sf_val)
    q, sf = _per_channel_expected(x, [256], sf_val)
    assert np.array_equal(got["col_q"], q)
    assert np.array_equal(got["col_s"].view(np.uint32), sf.view(np.uint32))
    assert got["col_s"].reshape(2, 64)[1, 5] == np.float32(1e-30)

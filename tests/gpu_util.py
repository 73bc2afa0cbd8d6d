"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI and the CPU oracle
on the same seeded inputs, and compare.

Outputs of the HIP path are pre-poisoned (0xFF bytes, NaN floats) so that any byte the library
must not write, and any byte it failed to write, shows up."""
import numpy as np
import torch

import block_scaled_fp8_grouped_amd as bs
import oracle
import workloads as W

DEV = "cuda"
REL_TOL = 1e-5  # per-expert relative Frobenius error against the fp64 oracle


def flush(msg):
    print(msg, flush=True)


def poisoned_quant_outputs(R, C, E, recipe, which):
    out = bs.alloc_quantized(R, C, E, recipe, which, DEV)
    for t in out.values():
        t.view(torch.uint8).fill_(0xFF)
    return out


def gpu_quantize(x, splits, recipe, which, zas=1e-30, status=None):
    """Quantize on the GPU into poisoned buffers; returns the device dict."""
    R, C = x.shape
    E = len(splits) if splits is not None else 1
    st = None if splits is None else W.splits_tensor(splits, DEV)
    out = poisoned_quant_outputs(R, C, E, recipe, which)
    own = status is None
    if own:
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
    bs.grouped_quantize(x, st, recipe, which, out, zas, status=status)
    if own:
        torch.cuda.synchronize()
        assert int(status.item()) == 0
    return out


def _first_diff(a, b):
    idx = np.nonzero(a != b)[0]
    return f"{idx.size} differ; first at {idx[0]}: got {a[idx[0]]:#x} expected {b[idx[0]]:#x}" if idx.size else ""


def assert_quant_matches(got, ref, splits, R, which, label=""):
    """Bit-exact comparison of the GPU outputs (device dict) with the oracle's (host dict), and
    check that nothing past the documented extents was written."""
    T = R if splits is None else sum(splits)
    if which & bs.COLWISE:
        gq = got["col_q"].cpu().numpy()
        nq = ref["col_q"].size
        assert np.array_equal(gq[:nq], ref["col_q"]), f"{label} col_q: " + _first_diff(gq[:nq], ref["col_q"])
        assert (gq[nq:] == 0xFF).all(), f"{label} col_q written past sum(Kp_e)"
        gs = got["col_s"].cpu().numpy().view(np.uint8)
        rs = ref["col_s"].view(np.uint8)
        assert np.array_equal(gs[:rs.size], rs), f"{label} col_s: " + _first_diff(gs[:rs.size], rs)
        assert (gs[rs.size:] == 0xFF).all(), f"{label} col_s written past sum(Kp_e)"
    if which & bs.ROWWISE:
        gq = got["row_q"].cpu().numpy()
        assert np.array_equal(gq[:T], ref["row_q"][:T]), f"{label} row_q: " + _first_diff(gq[:T].ravel(), ref["row_q"][:T].ravel())
        assert (gq[T:] == 0xFF).all(), f"{label} row_q written past the live rows"
        gs = got["row_s"].cpu().numpy()
        assert np.array_equal(gs[:, :T], ref["row_s"][:, :T]), f"{label} row_s: " + _first_diff(gs[:, :T].ravel(), ref["row_s"][:, :T].ravel())
        assert (gs[:, T:] == 0xFF).all(), f"{label} row_s written past the live rows"


def check_quantize(x, splits, recipe, which, zas=1e-30, label=""):
    got = gpu_quantize(x, splits, recipe, which, zas)
    torch.cuda.synchronize()
    ref = oracle.grouped_quantize(W.bf16_bits(x), splits, recipe, which, zas)
    assert_quant_matches(got, ref, splits, x.shape[0], which, label)
    return got, ref


def rel_err(got, ref):
    """Relative Frobenius error; an all-zero reference requires an all-zero result."""
    nr = np.linalg.norm(ref)
    if nr == 0:
        return 0.0 if not np.any(got) else np.inf
    return float(np.linalg.norm(got - ref) / nr)


def bf16_round(a64):
    """fp64 -> fp32 -> bf16 (round to nearest even), returned as float64 values."""
    t = torch.from_numpy(np.asarray(a64, np.float64)).float().to(torch.bfloat16)
    return t.double().numpy()


def bf16_ulp(v):
    """Spacing of bf16 numbers at |v| (8 significant bits)."""
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.ldexp(1.0, (e - 7).astype(np.int64))


def assert_bf16_close(got, ref, label=""):
    """bf16 output check: |got - ref| <= 1 bf16 ulp of round_bf16(ref) + 1e-5 * rms(ref).

    The ulp covers the final rounding to bf16 (including a near-tie that the fp32 sum puts on
    the other side); the rms term is the same 1e-5 budget the fp32 outputs get, and matters
    only for outputs near zero, where cancellation makes a bf16 ulp smaller than the fp32
    accumulation error of the sum."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rb = bf16_round(ref)
    tol = bf16_ulp(rb) + REL_TOL * np.sqrt(np.mean(ref * ref))
    err = np.abs(got - ref)
    bad = err > tol
    if bad.any():
        i = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(f"{label}: {int(bad.sum())} bf16 values out of tolerance; worst at {i}: got {got[i]!r} "
                             f"ref {ref[i]!r} (bf16 {rb[i]!r}), tol {tol[i]:.3e}")

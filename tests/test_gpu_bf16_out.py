"""bf16 outputs of the m-grouped GEMMs, per element and exactly: the bf16 and fp32 variants of a
call run the same MFMA sequence on the same quantized operands, so every live bf16 output must be
the round-to-nearest-even of the fp32 output of the same call, bit for bit (the fp32 outputs are
held to the oracle by the parity tests).  This pins each bf16 value on its own, outputs near zero
included, with no tolerance.  Rows past sum(split_sizes) stay untouched in both variants.

Covered: fprop and dgrad; MXFP8 widened, MXFP8 on the scaled fp8 MFMA, MXFP4; a K that is not a
multiple of 128 (the K-tail kernel and the scaled paths' tail step), output widths with a
partial tile, empty and 1-row groups; and the 128-expert MoE fprop at full size.
"""
import pytest
import torch

import block_scaled_fp8_grouped_amd as bs
import workloads as W
from gpu_util import DEV, flush, gpu_quantize

pytestmark = pytest.mark.gpu

F8 = bs.RECIPE_MX | bs.GEMM_FP8_MFMA


def _quant_recipe(recipe):
    return bs.RECIPE_MX4 if recipe == bs.RECIPE_MX4 else bs.RECIPE_MX


def _both(call, R, width):
    """Run ``call(out, out_dtype)`` with fp32 and with bf16 outputs (NaN-filled beforehand)."""
    o32 = torch.full((R, width), float("nan"), dtype=torch.float32, device=DEV)
    o16 = torch.full((R, width), float("nan"), dtype=torch.bfloat16, device=DEV)
    call(o32, bs.OUT_F32)
    call(o16, bs.OUT_BF16)
    torch.cuda.synchronize()
    return o32, o16


def _assert_rne(o32, o16, T, label):
    live32, live16 = o32[:T], o16[:T]
    assert not torch.isnan(live32).any(), f"{label}: a live fp32 output is NaN"
    want = live32.to(torch.bfloat16)  # round to nearest even
    same = live16.view(torch.int16) == want.view(torch.int16)
    if not bool(same.all()):
        r, c = [int(v) for v in torch.nonzero(~same)[0]]
        raise AssertionError(f"{label}: {int((~same).sum())} bf16 outputs differ from RNE(fp32); first at "
                             f"[{r}, {c}]: bf16 {float(live16[r, c])!r}, fp32 {float(live32[r, c])!r}")
    assert torch.isnan(o32[T:]).all() and torch.isnan(o16[T:].float()).all(), f"{label}: rows past the live ones written"


CASES = [
    # splits, K (contraction), N (output width)
    ([0, 1, 31, 32, 33, 127, 128, 129, 256], 256, 256),
    ([300, 0, 45, 1, 200], 160, 320),   # K tail (160 = 128 + 32), partial output tile
    ([600], 512, 96),
    ([257, 0, 0, 513], 384, 512),
]


@pytest.mark.parametrize("recipe", [bs.RECIPE_MX, F8, bs.RECIPE_MX4], ids=["mxfp8", "fp8mfma", "mxfp4"])
@pytest.mark.parametrize("splits,K,N", CASES)
def test_fprop_bf16_is_rne_of_fp32(recipe, splits, K, N):
    flush(f"fprop bf16 vs fp32 recipe={recipe} splits={splits} K={K} N={N}")
    T = sum(splits)
    R = T + 40
    E = len(splits)
    g = torch.Generator(device=DEV).manual_seed(11)
    x = W.randn_bf16((R, K), g, DEV)
    w = W.randn_bf16((E * N, K), g, DEV)
    qr = _quant_recipe(recipe)
    xq = gpu_quantize(x, splits, qr, bs.ROWWISE)
    wq = gpu_quantize(w, None, qr, bs.ROWWISE)
    st = W.splits_tensor(splits, DEV)
    o32, o16 = _both(lambda o, dt: bs.grouped_gemm_fprop(xq, K, wq, N, st, R, o, dt, recipe=recipe), R, N)
    _assert_rne(o32, o16, T, f"fprop recipe {recipe}")


@pytest.mark.parametrize("recipe", [bs.RECIPE_MX, F8, bs.RECIPE_MX4], ids=["mxfp8", "fp8mfma", "mxfp4"])
@pytest.mark.parametrize("splits,n,k", [([0, 1, 31, 200, 0, 129], 256, 256), ([333, 64], 160, 320), ([700], 96, 96)])
def test_dgrad_bf16_is_rne_of_fp32(recipe, splits, n, k):
    flush(f"dgrad bf16 vs fp32 recipe={recipe} splits={splits} n={n} k={k}")
    T = sum(splits)
    R = T + 24
    E = len(splits)
    g = torch.Generator(device=DEV).manual_seed(12)
    dy = W.randn_bf16((R, n), g, DEV)
    w = W.randn_bf16((E * n, k), g, DEV)
    qr = _quant_recipe(recipe)
    dyq = gpu_quantize(dy, splits, qr, bs.ROWWISE)
    wq = gpu_quantize(w, [n] * E, qr, bs.COLWISE)
    st = W.splits_tensor(splits, DEV)
    o32, o16 = _both(lambda o, dt: bs.grouped_gemm_dgrad(dyq, n, wq, k, st, R, o, dt, recipe=recipe), R, k)
    _assert_rne(o32, o16, T, f"dgrad recipe {recipe}")


def test_moe128_fprop_bf16_is_rne_of_fp32():
    """The 128-expert MoE forward at full size (1,048,576 rows x 2048 outputs, K = 7168)."""
    flush("moe128 fprop bf16 vs fp32")
    case = W.moe128_top8(DEV, with_main_grad=False)
    splits, R, T = case["splits"], case["R"], case["T"]
    K, N = case["K"], case["N"]
    E = len(splits)
    st = W.splits_tensor(splits, DEV)
    xq = bs.alloc_quantized(R, K, E, bs.RECIPE_MX, bs.ROWWISE, DEV)
    wq = bs.alloc_quantized(E * N, K, 1, bs.RECIPE_MX, bs.ROWWISE, DEV)
    bs.grouped_quantize(case["x"], st, bs.RECIPE_MX, bs.ROWWISE, xq)
    bs.grouped_quantize(case["W"].view(E * N, K), None, bs.RECIPE_MX, bs.ROWWISE, wq)
    del case
    o32, o16 = _both(lambda o, dt: bs.grouped_gemm_fprop(xq, K, wq, N, st, R, o, dt), R, N)
    _assert_rne(o32, o16, T, "moe128 fprop")

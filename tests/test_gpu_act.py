"""The activation fused with the grouped quantize (the ScaledSReLU step between fc1 and fc2 in the
TransformerEngine #3484 reproducer, the ScaledSwiGLU of the same family, and their gradients) on
the GPU vs the CPU oracle: quantized bytes and scales bit-exact (both sides compute the
activation in fp32 with the same rounding order and the same stated exp2, then take every
quantization decision on the same fp32 value).

Ragged groups, both layouts, MXFP8 and MXFP4, with and without probs (negative ones too),
garbage padding (NaN/Inf in h, dy and probs past the live rows), signed zeros, the device status
word, GLU widths that are and are not multiples of the 128-column tile (the gradient's da | db
boundary inside a tile), and the 32-expert MoE shape at full size.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp8_grouped_amd as bs
import oracle
import workloads as W
from gpu_util import DEV, assert_quant_matches, flush, poisoned_quant_outputs

pytestmark = pytest.mark.gpu
RAGGED = [[0, 1, 31, 32, 33, 127, 128, 129, 256], [300, 0, 45, 1, 200], [1000], [0, 0, 5]]


def _inputs(R, C, splits, seed, negative_probs=False):
    g = torch.Generator(device=DEV).manual_seed(seed)
    h = W.randn_bf16((R, C), g, DEV, scale=2.0)
    dy = W.randn_bf16((R, C), g, DEV, scale=0.5)
    p = torch.rand(R, generator=g, device=DEV)
    if negative_probs:
        p = p - 0.5
    T = sum(splits)
    rng = np.random.default_rng(seed)
    for t in (h, dy):
        bits = rng.integers(0, 1 << 16, size=(R - T, C), dtype=np.uint16)
        t[T:] = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    p[T:] = float("nan")
    return h, dy, p


GRADS = (bs.ACT_SRELU_GRAD, bs.ACT_SWIGLU_GRAD)


def _out_cols(act, h):
    """Columns of the quantized output: h's, F = half of them (SwiGLU) or 2F = all (its gradient)."""
    return h.shape[1] // 2 if act == bs.ACT_SWIGLU else h.shape[1]


def _check(act, h, dy, p, splits, recipe, which, label):
    R = h.shape[0]
    st = W.splits_tensor(splits, DEV)
    out = poisoned_quant_outputs(R, _out_cols(act, h), len(splits), recipe, which)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    bs.grouped_act_quantize(act, h, st, recipe, which, out, probs=p, dy=dy if act in GRADS else None,
                            status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    ref = oracle.grouped_act_quantize(act, W.bf16_bits(h), None if p is None else p.cpu().numpy(),
                                      W.bf16_bits(dy) if act in GRADS else None, splits, recipe, which)
    assert_quant_matches(out, ref, splits, R, which, label)


def _glu_inputs(R, F, splits, seed, negative_probs=False):
    """h = (a | b) [R, 2F] and dy [R, F] with the garbage padding of _inputs."""
    h, _, p = _inputs(R, 2 * F, splits, seed, negative_probs)
    _, dy, _ = _inputs(R, F, splits, seed + 1)
    return h, dy, p


@pytest.mark.parametrize("act", [bs.ACT_SRELU, bs.ACT_SRELU_GRAD])
@pytest.mark.parametrize("recipe", [bs.RECIPE_MX, bs.RECIPE_MX4])
@pytest.mark.parametrize("splits", RAGGED)
@pytest.mark.parametrize("C", [32, 160, 512])
def test_act_quantize_parity(act, recipe, splits, C):
    flush(f"act={act} recipe={recipe} C={C} splits={splits}")
    T = sum(splits)
    h, dy, p = _inputs(T + 37, C, splits, seed=C + T + act, negative_probs=(C == 160))
    _check(act, h, dy, p, splits, recipe, bs.ROWWISE | bs.COLWISE, f"act{act} r{recipe} C={C}")


@pytest.mark.parametrize("which", [bs.ROWWISE, bs.COLWISE])
@pytest.mark.parametrize("act", [bs.ACT_SRELU, bs.ACT_SRELU_GRAD])
def test_act_quantize_single_layout_and_no_probs(which, act):
    flush(f"act={act} which={which} no probs")
    splits = [130, 0, 257, 31]
    h, dy, _ = _inputs(sum(splits) + 20, 288, splits, seed=7)
    _check(act, h, dy, None, splits, bs.RECIPE_MX, which, f"act{act} which{which}")


def test_act_quantize_signed_zeros_and_negative_inputs():
    flush("act signed zeros")
    splits = [64]
    C = 64
    g = torch.Generator(device=DEV).manual_seed(2)
    h = W.randn_bf16((64, C), g, DEV)
    h[:, :8] = -0.0
    h[:, 8:16] = 0.0
    h[:4] = -h[:4].abs()
    dy = W.randn_bf16((64, C), g, DEV)
    p = torch.linspace(-1, 1, 64, device=DEV)
    for act in (bs.ACT_SRELU, bs.ACT_SRELU_GRAD):
        _check(act, h, dy, p, splits, bs.RECIPE_MX, bs.ROWWISE | bs.COLWISE, f"zeros act{act}")


def test_act_quantize_status_bits_and_no_writes():
    flush("act status")
    R, C = 300, 64
    h, dy, p = _inputs(R, C, [R], seed=3)
    for splits, bit in (([100, -5, 50], bs.STATUS_NEGATIVE_SPLIT), ([200, 200], bs.STATUS_EXCEEDS_CAPACITY)):
        st = W.splits_tensor(splits, DEV)
        out = poisoned_quant_outputs(R, C, len(splits), bs.RECIPE_MX, bs.ROWWISE | bs.COLWISE)
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
        bs.grouped_act_quantize(bs.ACT_SRELU, h, st, bs.RECIPE_MX, bs.ROWWISE | bs.COLWISE, out, probs=p,
                                status=status)
        torch.cuda.synchronize()
        assert int(status.item()) & bit
        for t in out.values():
            assert (t.view(torch.uint8) == 0xFF).all()


def test_act_quantize_moe32_shape():
    """fc1's output of the 32-expert layer (65,536 routed rows, ffn 1536, Zipf routing with empty
    experts, garbage padding): forward activation + both MXFP8 layouts, all bytes."""
    flush("act moe32")
    case = W.moe32_zipf(DEV, with_weight=False)
    splits, R = case["splits"], case["R"]
    T = case["T"]
    g = torch.Generator(device=DEV).manual_seed(40)
    h = case["dy"]  # any [R, 1536] bf16 buffer of this shape and padding serves as fc1's output
    p = torch.rand(R, generator=g, device=DEV)
    _check(bs.ACT_SRELU, h, None, p, splits, bs.RECIPE_MX, bs.ROWWISE | bs.COLWISE, "moe32")
    assert T < R


@pytest.mark.parametrize("act", [bs.ACT_SWIGLU, bs.ACT_SWIGLU_GRAD])
@pytest.mark.parametrize("recipe", [bs.RECIPE_MX, bs.RECIPE_MX4])
@pytest.mark.parametrize("splits", RAGGED)
@pytest.mark.parametrize("F", [32, 96, 256])
def test_swiglu_quantize_parity(act, recipe, splits, F):
    """F = 96: the gradient's 192 output columns put the da | db boundary inside the first tile."""
    flush(f"swiglu act={act} recipe={recipe} F={F} splits={splits}")
    T = sum(splits)
    h, dy, p = _glu_inputs(T + 29, F, splits, seed=F + T + act, negative_probs=(F == 96))
    _check(act, h, dy, p, splits, recipe, bs.ROWWISE | bs.COLWISE, f"act{act} r{recipe} F={F}")


@pytest.mark.parametrize("which", [bs.ROWWISE, bs.COLWISE])
@pytest.mark.parametrize("act", [bs.ACT_SWIGLU, bs.ACT_SWIGLU_GRAD])
def test_swiglu_single_layout_no_probs_and_large_inputs(which, act):
    """Inputs up to |a| = 96 (2^(-a log2 e) at the clamp of the stated exp2 on both sides), signed
    zeros, no probs."""
    flush(f"swiglu act={act} which={which} wide range")
    splits = [130, 0, 257, 31]
    h, dy, _ = _glu_inputs(sum(splits) + 20, 160, splits, seed=8)
    h[:, :32] = h[:, :32] * 48.0
    h[:8, 32:40] = -0.0
    h[8:16, 32:40] = 0.0
    _check(act, h, dy, None, splits, bs.RECIPE_MX, which, f"swiglu act{act} which{which}")


def test_swiglu_moe32_shape():
    """fc1's GLU output of the 32-expert layer (65,536 routed rows, ffn 1536 so h is [R, 3072]),
    Zipf routing with empty experts, garbage padding: the gradient, both MXFP8 layouts, all
    bytes."""
    flush("swiglu moe32")
    case = W.moe32_zipf(DEV, with_weight=False)
    splits, R = case["splits"], case["R"]
    g = torch.Generator(device=DEV).manual_seed(41)
    dy = case["dy"]
    h = torch.cat([dy, W.randn_bf16(dy.shape, g, DEV, scale=2.0)], dim=1)
    p = torch.rand(R, generator=g, device=DEV)
    _check(bs.ACT_SWIGLU_GRAD, h, dy, p, splits, bs.RECIPE_MX, bs.ROWWISE | bs.COLWISE, "swiglu moe32")


@pytest.mark.parametrize("act", [bs.ACT_SRELU, bs.ACT_SWIGLU_GRAD])
def test_act_quantize_max_groups(act):
    """1024 groups of 0 to 129 rows (the scan's maximum), both layouts, garbage padding."""
    rng = np.random.default_rng(33)
    splits = [int(v) for v in rng.choice([0, 1, 2, 31, 33, 64, 128, 129], size=bs.MAX_GROUPS)]
    flush(f"act={act} max groups T={sum(splits)}")
    T = sum(splits)
    if act == bs.ACT_SWIGLU_GRAD:
        h, dy, p = _glu_inputs(T + 17, 32, splits, seed=34)
    else:
        h, dy, p = _inputs(T + 17, 64, splits, seed=34)
    _check(act, h, dy, p, splits, bs.RECIPE_MX, bs.ROWWISE | bs.COLWISE, f"act{act} E=1024")

"""GPU grouped quantize vs the CPU oracle: bytes and scales bit-exact, in both layouts and both
recipes, on ragged groups (counts 0, 1, 31, 32, 33, 127, 128, 129, ...), partial channel tiles,
garbage padding, special values, and nothing written past the documented extents."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_grouped_amd as bs
import workloads as W
from gpu_util import DEV, check_quantize, flush

pytestmark = pytest.mark.gpu

RAGGED = [[0, 1, 31, 32, 33, 127, 128, 129, 256], [300, 0, 45, 1, 200], [77], [512], [0, 0, 5]]


def _mixed(R, C, seed):
    """randn with per-row and per-column magnitude spread (many different block exponents),
    exact zeros, negative zeros and a few bf16 subnormals; padding rows get random bits."""
    g = torch.Generator(device=DEV).manual_seed(seed)
    x = W.randn_bf16((R, C), g, DEV).float()
    rs = torch.pow(2.0, torch.randint(-20, 20, (R, 1), generator=g, device=DEV).float())
    cs = torch.pow(2.0, torch.randint(-6, 6, (1, C), generator=g, device=DEV).float())
    x = x * rs * cs
    x[::17, ::5] = 0.0
    x[3::19, 1::7] = -0.0
    x[5::23, 2::11] = 1e-39  # fp32/bf16 subnormal
    return x.to(torch.bfloat16)


def _with_garbage_tail(x, T, seed):
    R, C = x.shape
    if R > T:
        rng = np.random.default_rng(seed)
        bits = rng.integers(0, 1 << 16, size=(R - T, C), dtype=np.uint16)
        x[T:] = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    return x


@pytest.mark.parametrize("splits", RAGGED)
@pytest.mark.parametrize("C", [32, 160, 512])
def test_mx_row_and_col_ragged(splits, C):
    T = sum(splits)
    R = T + 64
    flush(f"mx quantize splits={splits} C={C}")
    x = _with_garbage_tail(_mixed(R, C, seed=C + T), T, seed=1)
    check_quantize(x, splits, bs.RECIPE_MX, bs.COLWISE | bs.ROWWISE, label=f"{splits} C={C}")
    check_quantize(x, splits, bs.RECIPE_MX, bs.COLWISE, label=f"col {splits} C={C}")
    check_quantize(x, splits, bs.RECIPE_MX, bs.ROWWISE, label=f"row {splits} C={C}")


@pytest.mark.parametrize("splits", RAGGED[:3] + [[256, 128, 128, 256]])
@pytest.mark.parametrize("zas", [1.0, 1e-4, 1e-8, 1e-30, 0.0])
def test_per_channel_ragged_and_sf_val_sweep(splits, zas):
    T = sum(splits)
    R = T + 40
    flush(f"pc quantize splits={splits} zas={zas}")
    x = _with_garbage_tail(_mixed(R, 96, seed=T), T, seed=2)
    x[:T, 7] = 0.0  # an all-zero channel in every group
    check_quantize(x, splits, bs.RECIPE_PC, bs.COLWISE, zas=zas, label=f"{splits} zas={zas}")


@pytest.mark.parametrize("n", [256, 2048])
def test_per_channel_deepgemm_shapes(n):
    """The DeepGEMM #365 operands (dy randn*1e-7, x randn*0.4, zeroed channel, padding 3.0)."""
    case = W.deepgemm_case(DEV, n, n, R=1024 if n == 256 else None)
    for name in ("dy", "x"):
        check_quantize(case[name], case["splits"], bs.RECIPE_PC, bs.COLWISE, label=name)


def test_rowwise_without_splits_weight_buffer():
    w = _mixed(4 * 96, 256, seed=9)
    check_quantize(w, None, bs.RECIPE_MX, bs.ROWWISE, label="weight")


def test_special_values():
    vals = torch.tensor([0.0, -0.0, 1.0, -1.0, 448.0, -448.0, 3.3895e38, -3.3895e38, 1e-39, -1e-39, 9.2e-41,
                         2.0 ** -133, 0.1, 300.0, 1e-30, 65504.0], dtype=torch.float32)
    R, C = 128, 64
    x = torch.zeros(R, C, dtype=torch.float32)
    g = torch.Generator().manual_seed(3)
    for r in range(R):
        x[r] = vals[torch.randint(0, vals.numel(), (C,), generator=g)] * (1.0 if r % 3 else 2.0 ** -(r % 60))
    x[:32, :32] = 1e-39  # a block of subnormals only (E8M0 exponent clamps at -127)
    x[32:64, 32:] = 0.0  # all-zero blocks
    x = x.to(torch.bfloat16).to(DEV)
    check_quantize(x, [128], bs.RECIPE_MX, bs.COLWISE | bs.ROWWISE, label="special")
    check_quantize(x, [100, 28], bs.RECIPE_PC, bs.COLWISE, label="special pc")


def test_many_groups_and_tiny_groups():
    rng = np.random.default_rng(12)
    for E in (32, 128, 1024):
        splits = [int(v) for v in rng.integers(0, 70, size=E)]
        splits[rng.integers(0, E)] = 0
        T = sum(splits)
        flush(f"E={E} T={T}")
        x = _with_garbage_tail(_mixed(T + 10, 64, seed=E), T, seed=E)
        check_quantize(x, splits, bs.RECIPE_MX, bs.COLWISE | bs.ROWWISE, label=f"E={E}")
        check_quantize(x, splits, bs.RECIPE_PC, bs.COLWISE, label=f"E={E} pc")

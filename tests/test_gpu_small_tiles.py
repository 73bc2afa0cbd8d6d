"""The MXFP8 weight gradient on launches of few tiles.

A launch with fewer than 128 tiles of 256 x 256 (fewer than half the CUs) takes 128 x 128
tiles of 4 waves on the widened path. TE #3484's reproducer is such a launch: one group, a
1024 x 1024 output and 16 big tiles. Every output sees the same MFMA chain in either kernel,
so the bar here is bitwise:
* parity with the fp64 oracle: ragged and empty groups, output widths that are not multiples
  of 128, store and accumulate (empty groups left bitwise untouched);
* the same groups computed in a launch made large enough for 256 x 256 tiles (groups appended
  after them) give the same bits;
* TE #3484's single-group shape: padding of 0.0 or 3.0 gives results bitwise equal to the
  unpadded run (TE #3484, expected behaviour).
"""
import numpy as np
import pytest
import torch

import block_scaled_fp8_grouped_amd as bs
import workloads as W
from gpu_util import DEV, flush
from test_gpu_gemm import _operands, check_wgrad, run_wgrad

pytestmark = pytest.mark.gpu

BIG_TILES = 128  # launches with at least this many 256 x 256 tiles keep them


def _big_tiles(E, n, h):
    return E * -(-n // 256) * -(-h // 256)


@pytest.mark.parametrize("accumulate", [False, True])
@pytest.mark.parametrize("n,h,splits", [
    (96, 320, [0, 33, 128, 300, 0, 1]),
    (1024, 1024, [512]),
    (384, 160, [129, 31, 0, 64]),
])
def test_small_launch_parity(n, h, splits, accumulate):
    assert _big_tiles(len(splits), n, h) < BIG_TILES
    flush(f"small-launch wgrad n={n} h={h} splits={splits} accumulate={accumulate}")
    R = sum(splits) + 40
    dy, x = _operands(R, n, h, splits, seed=7 + n)
    mg = None
    if accumulate:
        g = torch.Generator(device=DEV).manual_seed(3)
        mg = torch.randn((len(splits), n, h), generator=g, device=DEV, dtype=torch.float32)
    check_wgrad(dy, x, splits, bs.RECIPE_MX, accumulate=accumulate, mg=mg, label=f"small {n}x{h}")


@pytest.mark.parametrize("accumulate", [False, True])
def test_small_and_big_tiles_bitwise_equal(accumulate):
    n, h = 320, 448
    splits = [200, 0, 64, 129, 1]
    extra = [40] * 28
    assert _big_tiles(len(splits), n, h) < BIG_TILES <= _big_tiles(len(splits) + len(extra), n, h)
    flush(f"small vs big tiles, accumulate={accumulate}")
    big_splits = splits + extra
    T = sum(splits)
    R = sum(big_splits) + 32
    dy, x = _operands(R, n, h, big_splits, seed=11)
    mg = None
    if accumulate:
        g = torch.Generator(device=DEV).manual_seed(5)
        mg = torch.randn((len(big_splits), n, h), generator=g, device=DEV, dtype=torch.float32)
    # the small launch sees only the first groups' rows; the rows after them are its padding
    small, _, _ = run_wgrad(dy, x, splits, bs.RECIPE_MX, accumulate, None if mg is None else mg[:len(splits)])
    big, _, _ = run_wgrad(dy, x, big_splits, bs.RECIPE_MX, accumulate, mg)
    torch.cuda.synchronize()
    E = len(splits)
    assert T < R
    a = small.view(torch.int32)
    b = big[:E].view(torch.int32)
    diff = (a != b).nonzero()
    assert diff.numel() == 0, f"{diff.shape[0]} outputs differ, first at {diff[0].tolist()}"


def test_single_group_padding_bitwise_invariant():
    n = h = 1024
    live = 512
    flush("TE #3484 single-group shape on the small launch: padded runs vs unpadded")
    g = torch.Generator(device=DEV).manual_seed(1)
    live_x = W.randn_bf16((live, h), g, DEV)
    live_dy = W.randn_bf16((live, n), g, DEV)
    mg0 = torch.zeros((1, n, h), dtype=torch.float32, device=DEV)
    outs = []
    for R, fill in ((live, None), (768, 0.0), (768, 3.0)):
        dy = torch.full((R, n), fill if fill is not None else 0.0, dtype=torch.bfloat16, device=DEV)
        x = torch.full((R, h), fill if fill is not None else 0.0, dtype=torch.bfloat16, device=DEV)
        dy[:live] = live_dy
        x[:live] = live_x
        out, _, _ = run_wgrad(dy, x, [live], bs.RECIPE_MX, accumulate=True, mg=mg0)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.isfinite(outs[0]).all()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int32), outs[0].view(torch.int32))

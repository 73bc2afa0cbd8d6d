"""The library holds no state between calls and is reentrant (include/bsfp8.h conventions): the
same quantize -> wgrad -> fprop -> dgrad sequences issued on two streams at once, over different
inputs and split sizes, give results bitwise equal to the same calls run one after the other on
one stream, and the status words stay zero."""
import pytest
import torch

import block_scaled_fp8_grouped_amd as bs
import workloads as W
from gpu_util import DEV, flush

pytestmark = pytest.mark.gpu


def _problem(seed, splits, n, h, N):
    T = sum(splits)
    R = T + 96
    g = torch.Generator(device=DEV).manual_seed(seed)
    E = len(splits)
    return dict(splits=W.splits_tensor(splits, DEV), E=E, R=R, n=n, h=h, N=N,
                dy=W.randn_bf16((R, n), g, DEV), x=W.randn_bf16((R, h), g, DEV),
                w=W.randn_bf16((E * N, h), g, DEV), ns=W.splits_tensor([N] * E, DEV))


def _run(p, recipe, stream):
    """quantize dy (row + col), x (row + col), W (row, and col along N) -> wgrad, fprop, dgrad."""
    with torch.cuda.stream(stream):
        st, E, R, n, h, N = p["splits"], p["E"], p["R"], p["n"], p["h"], p["N"]
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
        both = bs.COLWISE | bs.ROWWISE
        dq = bs.grouped_quantize(p["dy"], st, recipe, both, bs.alloc_quantized(R, n, E, recipe, both, DEV), status=status)
        xq = bs.grouped_quantize(p["x"], st, recipe, both, bs.alloc_quantized(R, h, E, recipe, both, DEV), status=status)
        wr = bs.grouped_quantize(p["w"], None, recipe, bs.ROWWISE, bs.alloc_quantized(E * N, h, 1, recipe, bs.ROWWISE, DEV))
        # dgrad's weight: [E][N][h] viewed as [E*N][h] with split sizes N: blocks along N per expert
        wc = bs.grouped_quantize(p["w"], p["ns"], recipe, bs.COLWISE,
                                 bs.alloc_quantized(E * N, h, E, recipe, bs.COLWISE, DEV), status=status)
        dw = torch.empty(E, n, h, dtype=torch.float32, device=DEV)
        bs.grouped_gemm_wgrad(dq, n, xq, h, st, R, recipe, dw, status=status)
        y = torch.full((R, N), float("nan"), dtype=torch.float32, device=DEV)
        bs.grouped_gemm_fprop(xq, h, wr, N, st, R, y, bs.OUT_F32, status=status, recipe=recipe)
        # dgrad: the forward output's gradient [R, N] (here dy's first N channels) times W_e
        dx = torch.full((R, h), float("nan"), dtype=torch.bfloat16, device=DEV)
        yq = bs.grouped_quantize(p["dy"][:, :N].contiguous(), st, recipe, bs.ROWWISE,
                                 bs.alloc_quantized(R, N, E, recipe, bs.ROWWISE, DEV), status=status)
        bs.grouped_gemm_dgrad(yq, N, wc, h, st, R, dx, bs.OUT_BF16, status=status, recipe=recipe)
    return dict(dw=dw, y=y, dx=dx, status=status, keep=(dq, xq, wr, wc, yq))


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


@pytest.mark.parametrize("recipe", [bs.RECIPE_MX, bs.RECIPE_MX4], ids=["mxfp8", "mxfp4"])
def test_two_streams_match_sequential(recipe):
    flush(f"two streams, recipe {recipe}")
    pa = _problem(21, [900, 0, 257, 31, 1024], 256, 512, 256)
    pb = _problem(22, [1, 640, 0, 2000], 512, 256, 256)
    main = torch.cuda.current_stream()
    ref_a = _run(pa, recipe, main)
    ref_b = _run(pb, recipe, main)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    for rep in range(3):
        got_a = _run(pa, recipe, s1)
        got_b = _run(pb, recipe, s2)
        torch.cuda.synchronize()
        for name, got, ref in (("a", got_a, ref_a), ("b", got_b, ref_b)):
            assert int(got["status"].item()) == 0, (rep, name)
            for k in ("dw", "y", "dx"):
                assert torch.equal(_bits(got[k]), _bits(ref[k])), f"repeat {rep}, problem {name}: {k} differs"

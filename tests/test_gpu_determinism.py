"""Determinism stress from the DeepGEMM #365 reproducer (its stress test; the root-cause comment
traces the blow-ups to a race condition inside the GEMM kernel): the 2048 x 2048, four-expert wgrad
(one all-zero dy channel in each 128-token expert) called 10,000 times on operands cast once,
for each zero-channel scale in the page's sweep (1, 1e-4, 1e-8, 1e-30).  Every call must be
bitwise equal to the first, and no call may show the page's blow-up criterion (an expert's
output norm above max(100 x its unquantized reference norm, 1)).  The same stress runs on the
pipelined block-scaled kernels and on the 128 x 128 weight-gradient kernel of small launches, and the launches the benchmark times repeat bit for bit at the
128-expert MoE size."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_grouped_amd as bs
import workloads as W
from gpu_util import DEV, flush, gpu_quantize

pytestmark = pytest.mark.gpu

ITERS = 10000


@pytest.mark.parametrize("sf_val", [1.0, 1e-4, 1e-8, 1e-30])
def test_wgrad_10000_calls_bitwise(sf_val):
    case = W.deepgemm_case(DEV, 2048, 2048)
    splits, n, h, R = case["splits"], case["n"], case["h"], case["R"]
    E = len(splits)
    st = W.splits_tensor(splits, DEV)
    dq = gpu_quantize(case["dy"], splits, bs.RECIPE_PC, bs.COLWISE, sf_val)
    xq = gpu_quantize(case["x"], splits, bs.RECIPE_PC, bs.COLWISE, sf_val)
    # the unquantized fp32 reference norms of the page's criterion
    dyf, xf = case["dy"].float(), case["x"].float()
    ref_norms, off = [], 0
    for k in splits:
        ref_norms.append(torch.linalg.vector_norm(dyf[off:off + k].t() @ xf[off:off + k]).item())
        off += k
    thresholds = torch.tensor([max(100.0 * v, 1.0) for v in ref_norms], device=DEV)
    first = torch.empty(E, n, h, dtype=torch.float32, device=DEV)
    bs.grouped_gemm_wgrad(dq, n, xq, h, st, R, bs.RECIPE_PC, first)
    out = torch.empty_like(first)
    mismatched = torch.zeros((), dtype=torch.int64, device=DEV)
    blown = torch.zeros((), dtype=torch.int64, device=DEV)
    for it in range(ITERS):
        out.zero_()
        bs.grouped_gemm_wgrad(dq, n, xq, h, st, R, bs.RECIPE_PC, out)
        mismatched += torch.ne(out.view(torch.int32), first.view(torch.int32)).any().to(torch.int64)
        blown += (torch.linalg.vector_norm(out.view(E, -1), dim=1) > thresholds).any().to(torch.int64)
        if (it + 1) % 2500 == 0:
            torch.cuda.synchronize()
            flush(f"sf_val={sf_val}: {it + 1} calls, mismatched={int(mismatched)} blown={int(blown)}")
    torch.cuda.synchronize()
    assert int(mismatched) == 0 and int(blown) == 0
    norms = torch.linalg.vector_norm(first.view(E, -1), dim=1).cpu().numpy()
    assert np.all(norms <= np.maximum(100 * np.array(ref_norms), 1.0))
    # the zeroed channel gives an exact zero row in the 128-token experts
    assert (first[1, 0] == 0).all() and (first[2, 0] == 0).all()


# The same stress on the pipelined block-scaled kernels: the 256 x 256, 8-wave MXFP8 GEMM (next K
# step's DMA issued in the middle of the current one, E8M0 scales decoded in LDS) and the MXFP4 GEMM
# (its LDS DMAs issued as inline assembly with hand-placed waits), on the same four-expert 2048 x 2048
# shape with one all-zero dy channel in each 128-token expert.  wgrad in store mode, wgrad
# accumulating into a main_grad reset to the same fp32 contents before every call, and the m-grouped
# forward (fp32 and bf16 out) on a four-expert weight; also the MXFP8 operands on the scaled fp8 MFMA.  Every call must be bitwise equal to the first;
# the loop counts mismatching calls on the device and reports every 2,500 calls.
def _stress(run, out, label):
    run()
    torch.cuda.synchronize()
    first = out.clone()
    assert torch.isfinite(first.float()).all(), label
    mismatched = torch.zeros((), dtype=torch.int64, device=DEV)
    bits = torch.int16 if out.dtype == torch.bfloat16 else torch.int32
    for it in range(ITERS):
        run()
        mismatched += torch.ne(out.view(bits), first.view(bits)).any().to(torch.int64)
        if (it + 1) % 2500 == 0:
            torch.cuda.synchronize()
            flush(f"{label}: {it + 1} calls, mismatched={int(mismatched)}")
            assert int(mismatched) == 0, label
    torch.cuda.synchronize()
    assert int(mismatched) == 0, label
    return first


F8 = bs.RECIPE_MX | bs.GEMM_FP8_MFMA  # MXFP8 operands on the scaled fp8 MFMA


@pytest.mark.parametrize("recipe,accumulate", [(bs.RECIPE_MX, False), (bs.RECIPE_MX, True),
                                               (bs.RECIPE_MX4, False), (bs.RECIPE_MX4, True),
                                               (F8, False), (F8, True)])
def test_block_scaled_wgrad_10000_calls_bitwise(recipe, accumulate):
    case = W.deepgemm_case(DEV, 2048, 2048)
    splits, n, h, R = case["splits"], case["n"], case["h"], case["R"]
    E = len(splits)
    st = W.splits_tensor(splits, DEV)
    qrecipe = recipe & ~bs.GEMM_FP8_MFMA  # the data recipe
    dq = gpu_quantize(case["dy"], splits, qrecipe, bs.COLWISE)
    xq = gpu_quantize(case["x"], splits, qrecipe, bs.COLWISE)
    out = torch.empty(E, n, h, dtype=torch.float32, device=DEV)
    mg0 = torch.randn(E, n, h, generator=torch.Generator(device=DEV).manual_seed(7), device=DEV)

    def run():
        if accumulate:
            out.copy_(mg0)
        else:
            out.fill_(float("nan"))
        bs.grouped_gemm_wgrad(dq, n, xq, h, st, R, recipe, out, accumulate=accumulate)

    label = f"wgrad recipe={recipe} accumulate={accumulate}"
    flush(label)
    first = _stress(run, out, label)
    # the zeroed channel gives an exact zero row (store) or leaves main_grad's row as it was
    for e in (1, 2):
        assert torch.equal(first[e, 0], mg0[e, 0] if accumulate else torch.zeros_like(first[e, 0]))


@pytest.mark.parametrize("accumulate", [False, True])
def test_small_launch_wgrad_10000_calls_bitwise(accumulate):
    # TE #3484's single-group shape (1024 x 1024 over 512 tokens, padded to 768 rows with 3.0):
    # 16 tiles of 256 x 256, so the widened MXFP8 weight gradient takes its 128 x 128 kernel
    # (4 waves, two workgroups per CU)
    n = h = 1024
    live, R = 512, 768
    g = torch.Generator(device=DEV).manual_seed(1)
    x = torch.full((R, h), 3.0, dtype=torch.bfloat16, device=DEV)
    dy = torch.full((R, n), 3.0, dtype=torch.bfloat16, device=DEV)
    x[:live] = W.randn_bf16((live, h), g, DEV)
    dy[:live] = W.randn_bf16((live, n), g, DEV)
    dy[:live, 0] = 0.0
    splits = [live]
    st = W.splits_tensor(splits, DEV)
    dq = gpu_quantize(dy, splits, bs.RECIPE_MX, bs.COLWISE)
    xq = gpu_quantize(x, splits, bs.RECIPE_MX, bs.COLWISE)
    out = torch.empty(1, n, h, dtype=torch.float32, device=DEV)
    mg0 = torch.randn(1, n, h, generator=torch.Generator(device=DEV).manual_seed(7), device=DEV)

    def run():
        if accumulate:
            out.copy_(mg0)
        else:
            out.fill_(float("nan"))
        bs.grouped_gemm_wgrad(dq, n, xq, h, st, R, bs.RECIPE_MX, out, accumulate=accumulate)

    label = f"small-launch wgrad accumulate={accumulate}"
    flush(label)
    first = _stress(run, out, label)
    assert torch.equal(first[0, 0], mg0[0, 0] if accumulate else torch.zeros_like(first[0, 0]))


@pytest.mark.parametrize("recipe,out_dtype", [(bs.RECIPE_MX, bs.OUT_F32), (bs.RECIPE_MX, bs.OUT_BF16),
                                              (bs.RECIPE_MX4, bs.OUT_BF16), (F8, bs.OUT_BF16)])
def test_block_scaled_fprop_10000_calls_bitwise(recipe, out_dtype):
    case = W.deepgemm_case(DEV, 2048, 2048)
    splits, K, R = case["splits"], case["h"], case["R"]
    E, N = len(splits), 2048
    st = W.splits_tensor(splits, DEV)
    qrecipe = recipe & ~bs.GEMM_FP8_MFMA
    xq = gpu_quantize(case["x"], splits, qrecipe, bs.ROWWISE)
    w = W.randn_bf16((E * N, K), torch.Generator(device=DEV).manual_seed(8), DEV)
    wq = gpu_quantize(w, None, qrecipe, bs.ROWWISE)
    out = torch.empty(R, N, dtype=torch.float32 if out_dtype == bs.OUT_F32 else torch.bfloat16, device=DEV)

    def run():
        out.fill_(float("nan"))
        bs.grouped_gemm_fprop(xq, K, wq, N, st, R, out, out_dtype, recipe=recipe)

    label = f"fprop recipe={recipe} out_dtype={out_dtype}"
    flush(label)
    _stress(run, out, label)


# The launches the benchmark times, at full size: the 128-expert MoE layer (1,048,576 expert rows,
# hidden 7168, ffn 2048), MXFP8 wgrad accumulating into a main_grad reset before every call, the
# bf16 forward and the bf16 data gradient, each called repeatedly and compared bit for bit with
# the first call (the 128-expert shape runs 28,672 to 118,272 workgroups, over a hundred rounds of
# the chip, where the small stress shape runs one).
FULL_CALLS = 30


def _repeat(run, out, label, calls=FULL_CALLS):
    run()
    torch.cuda.synchronize()
    first = out.clone()
    bits = torch.int16 if out.dtype == torch.bfloat16 else torch.int32
    mismatched = torch.zeros((), dtype=torch.int64, device=DEV)
    for _ in range(calls):
        run()
        mismatched += torch.ne(out.view(bits), first.view(bits)).any().to(torch.int64)
    torch.cuda.synchronize()
    assert int(mismatched) == 0, f"{label}: {int(mismatched)} of {calls} calls differ from the first"
    return first


def test_moe128_launches_repeat_bitwise():
    case = W.moe128_top8(DEV)
    splits, R, T = case["splits"], case["R"], case["T"]
    n, h, K, N = case["n"], case["h"], case["K"], case["N"]
    E = len(splits)
    st = W.splits_tensor(splits, DEV)
    xq = bs.alloc_quantized(R, h, E, bs.RECIPE_MX, bs.COLWISE | bs.ROWWISE, DEV)
    dq = bs.alloc_quantized(R, n, E, bs.RECIPE_MX, bs.COLWISE | bs.ROWWISE, DEV)
    wq = bs.alloc_quantized(E * N, K, 1, bs.RECIPE_MX, bs.ROWWISE, DEV)
    wc = bs.alloc_quantized(E * N, K, E, bs.RECIPE_MX, bs.COLWISE, DEV)
    bs.grouped_quantize(case["x"], st, bs.RECIPE_MX, bs.COLWISE | bs.ROWWISE, xq)
    bs.grouped_quantize(case["dy"], st, bs.RECIPE_MX, bs.COLWISE | bs.ROWWISE, dq)
    w2 = case["W"].view(E * N, K)
    bs.grouped_quantize(w2, None, bs.RECIPE_MX, bs.ROWWISE, wq)
    bs.grouped_quantize(w2, W.splits_tensor([N] * E, DEV), bs.RECIPE_MX, bs.COLWISE, wc)
    mg0 = case["main_grad"]
    del case, w2
    mg = torch.empty_like(mg0)

    def wgrad():
        mg.copy_(mg0)
        bs.grouped_gemm_wgrad(dq, n, xq, h, st, R, bs.RECIPE_MX, mg, accumulate=True)

    flush("moe128 wgrad repeated")
    _repeat(wgrad, mg, "moe128 wgrad")
    del mg, mg0
    y = torch.empty(R, N, dtype=torch.bfloat16, device=DEV)
    flush("moe128 fprop repeated")
    _repeat(lambda: bs.grouped_gemm_fprop(xq, K, wq, N, st, R, y, bs.OUT_BF16), y, "moe128 fprop")
    del y
    dx = torch.empty(R, K, dtype=torch.bfloat16, device=DEV)
    flush("moe128 dgrad repeated")
    _repeat(lambda: bs.grouped_gemm_dgrad(dq, n, wc, K, st, R, dx, bs.OUT_BF16), dx, "moe128 dgrad")

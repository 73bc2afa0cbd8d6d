"""The binding's size checks (on device tensors, so on the GPU): a quantized buffer of another
recipe or of smaller dims than the call names, or an output too small for it, is refused with a
ValueError before the library is called, so no kernel reads or writes past a tensor's end (an
MXFP4 operand holds half the bytes per row of an MXFP8 one: handed to an MXFP8 GEMM, the kernel
would address rows twice as long).  The matching calls go through."""
import pytest
import torch

import block_scaled_fp8_grouped_amd as bs
import workloads as W
from gpu_util import DEV, gpu_quantize

pytestmark = pytest.mark.gpu


def test_recipe_and_size_mismatches_are_refused():
    splits = [100, 28]
    R, K, N, E = 160, 256, 64, 2
    st = W.splits_tensor(splits, DEV)
    g = torch.Generator(device=DEV).manual_seed(5)
    x = W.randn_bf16((R, K), g, DEV)
    w = W.randn_bf16((E * N, K), g, DEV)
    x4 = gpu_quantize(x, splits, bs.RECIPE_MX4, bs.ROWWISE | bs.COLWISE)
    w4 = gpu_quantize(w, None, bs.RECIPE_MX4, bs.ROWWISE)
    out = torch.empty(R, N, dtype=torch.float32, device=DEV)
    # MXFP4 operands named as MXFP8 (the default recipe): rows of K / 2 bytes read as K bytes
    with pytest.raises(ValueError, match=r"x_q\['row_q'\]"):
        bs.grouped_gemm_fprop(x4, K, w4, N, st, R, out, bs.OUT_F32)
    with pytest.raises(ValueError, match=r"dy_q\['col_q'\]"):
        bs.grouped_gemm_wgrad(x4, K, x4, K, st, R, bs.RECIPE_MX, torch.empty(E, K, K, device=DEV))
    # an output smaller than the call's rows x columns
    with pytest.raises(ValueError, match="out"):
        bs.grouped_gemm_fprop(x4, K, w4, N, st, R, torch.empty(R - 1, N, device=DEV), bs.OUT_F32, recipe=bs.RECIPE_MX4)
    with pytest.raises(ValueError, match="out"):
        bs.grouped_gemm_wgrad(x4, K, x4, K, st, R, bs.RECIPE_MX4, torch.empty(E, K, K // 2, device=DEV))
    # a weight quantized for fewer output channels than the dgrad call names
    dy4 = gpu_quantize(W.randn_bf16((R, N), g, DEV), splits, bs.RECIPE_MX4, bs.ROWWISE)
    wc4 = gpu_quantize(W.randn_bf16((E * N, K // 2), g, DEV), [N] * E, bs.RECIPE_MX4, bs.COLWISE)
    with pytest.raises(ValueError, match=r"w_q\['col_q'\]"):
        bs.grouped_gemm_dgrad(dy4, N, wc4, K, st, R, torch.empty(R, K, device=DEV), bs.OUT_F32, recipe=bs.RECIPE_MX4)
    # a quantize output sized for fewer rows
    small = bs.alloc_quantized(R - 32, K, E, bs.RECIPE_MX, bs.ROWWISE, DEV)
    with pytest.raises(ValueError, match=r"out\['row_q'\]"):
        bs.grouped_quantize(x, st, bs.RECIPE_MX, bs.ROWWISE, small)
    # the matching calls run
    bs.grouped_gemm_fprop(x4, K, w4, N, st, R, out, bs.OUT_F32, recipe=bs.RECIPE_MX4)
    bs.grouped_gemm_wgrad(x4, K, x4, K, st, R, bs.RECIPE_MX4, torch.empty(E, K, K, device=DEV))
    wc4 = gpu_quantize(w, [N] * E, bs.RECIPE_MX4, bs.COLWISE)
    bs.grouped_gemm_dgrad(dy4, N, wc4, K, st, R, torch.empty(R, K, device=DEV), bs.OUT_F32, recipe=bs.RECIPE_MX4)
    torch.cuda.synchronize()

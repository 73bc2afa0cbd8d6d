"""The Python binding's argument checks, which need no GPU: a tensor argument that the kernels
would read with the wrong element type (an int64 split_sizes tensor reads as sizes k_0, 0, k_1,
0, ...), or that lives in host memory (its pointer would reach the GPU), is refused with a
TypeError / ValueError before the library is called.  Raw integer addresses pass unchecked, so
each case below hands over one host tensor and fake addresses (never dereferenced) elsewhere."""
import pytest
import torch

import block_scaled_fp8_grouped_amd as bs

MX, PC = bs.RECIPE_MX, bs.RECIPE_PC
P = 1 << 20  # a fake device address


def _q(which):
    """Quantized-operand dict of fake addresses."""
    out = {}
    if which & bs.ROWWISE:
        out.update(row_q=P, row_s=P)
    if which & bs.COLWISE:
        out.update(col_q=P, col_s=P)
    return out


class _Splits:
    """A raw split-size address for E groups (the binding asks it for numel())."""

    def __init__(self, E):
        self.E = E

    def numel(self):
        return self.E

    def __int__(self):
        return P


S2 = _Splits(2)


def test_split_sizes_must_be_int32():
    st64 = torch.tensor([32, 32], dtype=torch.int64)
    q = _q(bs.COLWISE)
    with pytest.raises(TypeError, match="split_sizes"):
        bs.grouped_gemm_wgrad(q, 64, q, 64, st64, 64, MX, P)
    with pytest.raises(TypeError, match="split_sizes"):
        bs.grouped_gemm_fprop(_q(bs.ROWWISE), 64, _q(bs.ROWWISE), 64, st64, 64, P)
    with pytest.raises(TypeError, match="split_sizes"):
        bs.grouped_gemm_dgrad(_q(bs.ROWWISE), 64, _q(bs.COLWISE), 64, st64, 64, P)
    with pytest.raises(TypeError, match="split_sizes"):
        bs.grouped_quantize(P, torch.tensor([32.0, 32.0]), MX, bs.COLWISE, q, capacity_rows=64, cols=64)


def test_element_types():
    q, rq = _q(bs.COLWISE), _q(bs.ROWWISE)
    with pytest.raises(TypeError, match="out"):  # wgrad writes fp32
        bs.grouped_gemm_wgrad(q, 64, q, 64, S2, 64, MX, torch.empty(2, 64, 64, dtype=torch.float64))
    with pytest.raises(TypeError, match="out"):  # bf16 output asked, fp32 tensor given
        bs.grouped_gemm_fprop(rq, 64, rq, 64, S2, 64, torch.empty(64, 64), bs.OUT_BF16)
    with pytest.raises(TypeError, match="out"):  # fp32 output asked, bf16 tensor given
        bs.grouped_gemm_dgrad(rq, 64, q, 64, S2, 64, torch.empty(64, 64, dtype=torch.bfloat16), bs.OUT_F32)
    with pytest.raises(TypeError, match="x"):  # quantize reads bf16
        bs.grouped_quantize(torch.empty(64, 64), S2, MX, bs.COLWISE, q)
    with pytest.raises(TypeError, match="col_s"):  # per-channel scales are fp32
        bs.grouped_quantize(P, S2, PC, bs.COLWISE, dict(col_q=P, col_s=torch.empty(4, dtype=torch.uint8)),
                            capacity_rows=64, cols=64)
    with pytest.raises(TypeError, match="col_q"):  # codes are bytes
        bs.grouped_gemm_wgrad(dict(col_q=torch.empty(4, dtype=torch.int8), col_s=P), 64, q, 64, S2, 64, MX, P)
    with pytest.raises(TypeError, match="h"):  # the activation input is bf16
        bs.grouped_act_quantize(bs.ACT_SRELU, torch.empty(64, 64, dtype=torch.float16), S2, MX, bs.COLWISE, q)
    with pytest.raises(TypeError, match="status"):  # the status word is 32 bits
        bs.grouped_gemm_wgrad(q, 64, q, 64, S2, 64, MX, P, status=torch.zeros(1, dtype=torch.int64))


def test_host_tensors_are_refused():
    q = _q(bs.COLWISE)
    with pytest.raises(ValueError, match="device memory"):
        bs.grouped_gemm_wgrad(q, 64, q, 64, S2, 64, MX, torch.empty(2, 64, 64))
    with pytest.raises(ValueError, match="device memory"):
        bs.grouped_gemm_wgrad(q, 64, q, 64, torch.tensor([32, 32], dtype=torch.int32), 64, MX, P)
    with pytest.raises(ValueError, match="device memory"):
        bs.grouped_quantize(torch.empty(64, 64, dtype=torch.bfloat16), None, MX, bs.ROWWISE, _q(bs.ROWWISE))


def test_raw_addresses_pass_through():
    # integers are addresses the caller vouches for; the library's own host checks still apply
    # (here: a null split_sizes pointer for a colwise quantize) and no kernel is launched
    with pytest.raises(bs.BSFP8Error):
        bs.grouped_quantize(P, None, MX, bs.COLWISE, _q(bs.COLWISE), capacity_rows=64, cols=64, stream=0)

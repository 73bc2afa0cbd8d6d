"""The five workloads at their full sizes, in the launch configuration the benchmark uses.

1. DeepGEMM #365 shape with padding: 4 experts [256,128,128,256] + 256 rows of 3.0, n = h = 256,
   per-channel recipe, fp32 store.  Full oracle parity.
2. TE #3484 shape: one group of 512 rows, hidden 1024, MX, accumulate into zero main_grad;
   padded by 256 rows of 0.0 and of 3.0: bitwise equal to the unpadded run (the page's expected
   rel_err 0 and 0 non-finite of 1048576).  Full oracle parity.
3. DeepGEMM #365 shape: n = h = 2048, per-channel.  Full oracle parity.
4. MoE, 32 experts, 65,536 Zipf-routed rows (4 empty experts, counts not multiples of 32),
   garbage padding, hidden 4096, ffn 1536, MX; quantize bit-exact on the full tensors, wgrad on
   every expert x 64 sampled dy channels, fprop fp32 on 32 sampled output columns.
5. MoE, 128 experts, 1,048,576 rows, hidden 7168, ffn 2048, MX, wgrad accumulating into an fp32
   main_grad, fprop bf16: the full-size launches are checked on sampled experts (largest,
   smallest non-empty, one in between) against the oracle run on those experts' rows; every
   empty expert's main_grad must stay bitwise untouched.
"""
import json
import os

import numpy as np
import pytest
import torch

import block_scaled_fp8_grouped_amd as bs
import oracle
import workloads as W
from gpu_util import DEV, REL_TOL, assert_bf16_close, flush, gpu_quantize, rel_err
from test_gpu_gemm import check_fprop, check_wgrad, run_wgrad

pytestmark = pytest.mark.gpu

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_printed_values.json")))


def test_config1_deepgemm_256_padded():
    case = W.deepgemm_case(DEV, 256, 256, R=1024, pad_fill=3.0)
    check_wgrad(case["dy"], case["x"], case["splits"], bs.RECIPE_PC, label="cfg1")


def test_config2_single_group_padding_bitwise():
    exp = GOLDEN["te3484_expected"]
    outs = {}
    for R, fill in ((512, 0.0), (768, 0.0), (768, 3.0)):
        case = W.te_single_group_case(DEV, R=R, pad_fill=fill)
        flush(f"cfg2 R={R} fill={fill}")
        outs[(R, fill)] = check_wgrad(case["dy"], case["x"], case["splits"], bs.RECIPE_MX, accumulate=True,
                                      mg=case["main_grad"], label=f"cfg2 R={R} fill={fill}").double()
    ref = outs[(512, 0.0)]
    assert ref.numel() == exp["numel"]
    for key in ((768, 0.0), (768, 3.0)):
        got = outs[key]
        rel = ((got - ref).norm() / ref.norm()).item()
        assert rel == exp["rel_err"]
        assert int((~torch.isfinite(got)).sum()) == exp["non_finite"]
        assert torch.equal(got, ref)


def test_config3_deepgemm_2048():
    case = W.deepgemm_case(DEV, 2048, 2048)
    check_wgrad(case["dy"], case["x"], case["splits"], bs.RECIPE_PC, label="cfg3")


def test_config4_moe32_zipf():
    case = W.moe32_zipf(DEV)
    splits, R, T = case["splits"], case["R"], case["T"]
    assert min(splits) == 0 and any(k % 32 for k in splits)
    flush(f"cfg4 splits={splits} R={R}")
    rng = np.random.default_rng(40)
    rows = np.sort(rng.choice(case["n"], 64, replace=False)).astype(np.int32)
    check_wgrad(case["dy"], case["x"], splits, bs.RECIPE_MX, rows_sel=rows, label="cfg4 wgrad")
    cols = np.sort(rng.choice(case["N"], 32, replace=False)).astype(np.int32)
    w = case["W"].view(-1, case["K"])
    check_fprop(case["x"], w, splits, case["N"], bs.OUT_F32, cols_sel=cols, label="cfg4 fprop")


def _expert_rows(t, off, k):
    return W.bf16_bits(t[off:off + k])


def test_config5_moe128_sampled_experts():
    case = W.moe128_top8(DEV)
    splits, R, T = case["splits"], case["R"], case["T"]
    n, h, K, N = case["n"], case["h"], case["K"], case["N"]
    E = len(splits)
    st = W.splits_tensor(splits, DEV)
    flush(f"cfg5 T={T} empty={[e for e, k in enumerate(splits) if k == 0]}")
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    # the benchmark's launches
    xq = gpu_quantize(case["x"], splits, bs.RECIPE_MX, bs.COLWISE | bs.ROWWISE, status=status)
    dq = gpu_quantize(case["dy"], splits, bs.RECIPE_MX, bs.COLWISE, status=status)
    w2 = case["W"].view(E * N, K)
    wq = gpu_quantize(w2, None, bs.RECIPE_MX, bs.ROWWISE)
    mg0 = case["main_grad"]
    empty = [e for e, k in enumerate(splits) if k == 0]
    mg_empty = mg0[empty].clone()
    live = [e for e, k in enumerate(splits) if k > 0]
    sample = sorted({max(live, key=lambda e: splits[e]), min(live, key=lambda e: splits[e]), live[len(live) // 2]})
    rng = np.random.default_rng(50)
    rows = np.sort(rng.choice(n, 32, replace=False)).astype(np.int32)
    cols = np.sort(rng.choice(N, 16, replace=False)).astype(np.int32)
    mg_sample = {e: mg0[e].cpu().numpy()[None] for e in sample}
    bs.grouped_gemm_wgrad(dq, n, xq, h, st, R, bs.RECIPE_MX, mg0, accumulate=True, status=status)
    fout = torch.empty(R, N, dtype=torch.bfloat16, device=DEV)
    bs.grouped_gemm_fprop(xq, K, wq, N, st, R, fout, bs.OUT_BF16, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(mg0[empty].view(torch.int32), mg_empty.view(torch.int32)), "empty experts' main_grad touched"
    offs = np.concatenate([[0], np.cumsum(splits)])
    kps = [128 * ((k + 127) // 128) for k in splits]
    pofs = np.concatenate([[0], np.cumsum(kps)])
    for e in sample:
        k, off, P, kp = splits[e], int(offs[e]), int(pofs[e]), kps[e]
        flush(f"cfg5 expert {e} k={k}")
        ox = oracle.grouped_quantize(_expert_rows(case["x"], off, k), [k], oracle.RECIPE_MX,
                                     oracle.COLWISE | oracle.ROWWISE)
        ody = oracle.grouped_quantize(_expert_rows(case["dy"], off, k), [k], oracle.RECIPE_MX, oracle.COLWISE)
        ow = oracle.grouped_quantize(W.bf16_bits(w2[e * N:(e + 1) * N]), None, oracle.RECIPE_MX, oracle.ROWWISE)
        # quantized bytes of this expert, bit-exact
        assert np.array_equal(xq["col_q"][h * P:h * (P + kp)].cpu().numpy(), ox["col_q"])
        assert np.array_equal(xq["col_s"][h * P // 32:h * (P + kp) // 32].cpu().numpy(), ox["col_s"])
        assert np.array_equal(dq["col_q"][n * P:n * (P + kp)].cpu().numpy(), ody["col_q"])
        assert np.array_equal(dq["col_s"][n * P // 32:n * (P + kp) // 32].cpu().numpy(), ody["col_s"])
        assert np.array_equal(xq["row_q"][off:off + k].cpu().numpy(), ox["row_q"])
        assert np.array_equal(xq["row_s"][:, off:off + k].cpu().numpy(), ox["row_s"])
        assert np.array_equal(wq["row_q"][e * N:(e + 1) * N].cpu().numpy(), ow["row_q"])
        assert np.array_equal(wq["row_s"][:, e * N:(e + 1) * N].cpu().numpy(), ow["row_s"])
        # wgrad (accumulate) on sampled dy channels
        ref = oracle.grouped_wgrad(ody["col_q"], ody["col_s"], n, ox["col_q"], ox["col_s"], h, [k], k,
                                   oracle.RECIPE_MX, rows_sel=rows)
        got = mg0[e].cpu().numpy()[rows].astype(np.float64) - mg_sample[e][0][rows].astype(np.float64)
        r = rel_err(got, ref[0])
        assert r <= REL_TOL, f"cfg5 wgrad expert {e}: rel {r:.3e}"
        # fprop bf16 on sampled columns
        fref = oracle.grouped_fprop(ox["row_q"], ox["row_s"], ow["row_q"], ow["row_s"], N, [k], cols_sel=cols)
        fgot = fout[off:off + k].float().cpu().numpy().astype(np.float64)[:, cols]
        assert_bf16_close(fgot, fref, f"cfg5 fprop expert {e}")

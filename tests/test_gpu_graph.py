"""Output reuse, the quantize noop flag, and HIP-graph capture of the whole expert-layer path.

TransformerEngine PR #3224 (group_quantize output reuse): quantize can update caller-owned,
pre-allocated storage in place, and a device-resident noop flag lets a captured graph skip the
re-quantization of a cached weight on later microbatches.  TransformerEngine issue #3484 (the
graph-safe grouped linear): split sizes stay on the device, so one captured graph serves every
routing.

* noop flag set: every output byte and the status word keep what they held, even when the input
  changed or the split sizes are invalid.
* noop flag clear / NULL: in-place quantize over storage filled by an earlier call gives the same
  bytes as a call into fresh storage (which the quantize parity tests pin to the oracle).
* graph: weight quantize (behind the flag), x and dy quantize, fprop, dgrad and wgrad accumulated
  into an fp32 main_grad, captured once and replayed over several microbatches with new tokens,
  new routing (an empty expert, garbage padding) and a changed bf16 weight that the flag hides;
  between replays the program runs its own eager work and synchronizes.  Every replay is compared
  bitwise with the same calls run eagerly (the kernels are deterministic), and the first replay's
  outputs also with the oracle on sampled rows.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp8_grouped_amd as bs
import oracle
import workloads as W
from gpu_util import DEV, REL_TOL, assert_bf16_close, flush, rel_err

pytestmark = pytest.mark.gpu


def _written_views(out, splits, R, C, which):
    """The bytes a quantize call writes (its documented extents), as host arrays."""
    v = {}
    if which & bs.ROWWISE:
        T = R if splits is None else sum(splits)
        v["row_q"] = out["row_q"][:T].cpu().numpy()
        v["row_s"] = out["row_s"][:, :T].cpu().numpy()
    if which & bs.COLWISE:
        kp = sum(128 * ((k + 127) // 128) for k in splits)
        v["col_q"] = out["col_q"][:kp * C].cpu().numpy()
        s = out["col_s"].cpu().numpy().view(np.uint8)
        v["col_s"] = s[:kp * C // 32] if out["col_s"].dtype == torch.uint8 else s[:kp * C // 128 * 4]
    return v


def _alloc(R, C, E, recipe, which):
    out = bs.alloc_quantized(R, C, E, recipe, which, DEV)
    for t in out.values():
        t.view(torch.uint8).fill_(0xA5)
    return out


def _quant(x, st, recipe, which, out, noop=None, status=None):
    return bs.grouped_quantize(x, st, recipe, which, out, status=status, noop_flag=noop)


def _snapshot(out):
    return {k: v.clone() for k, v in out.items()}


def _same(a, b):
    return all(torch.equal(a[k].view(torch.uint8), b[k].view(torch.uint8)) for k in a)


@pytest.mark.parametrize("recipe,which", [(bs.RECIPE_MX, bs.ROWWISE | bs.COLWISE), (bs.RECIPE_MX, bs.COLWISE),
                                          (bs.RECIPE_PC, bs.COLWISE)])
def test_noop_flag_leaves_outputs_and_status(recipe, which):
    flush(f"noop recipe={recipe} which={which}")
    splits = [130, 0, 257, 31]
    R, C = sum(splits) + 40, 416
    g = W._gen(DEV, 11)
    x0 = W.randn_bf16((R, C), g, DEV)
    x1 = W.randn_bf16((R, C), g, DEV, scale=5.0)
    st = W.splits_tensor(splits, DEV)
    out = _alloc(R, C, len(splits), recipe, which)
    flag = torch.zeros(1, dtype=torch.float32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    _quant(x0, st, recipe, which, out, noop=flag, status=status)  # flag 0: quantizes
    torch.cuda.synchronize()
    before = _snapshot(out)
    assert int(status.item()) == 0
    flag.fill_(1.0)
    _quant(x1, st, recipe, which, out, noop=flag, status=status)  # new input, flag 1: untouched
    bad = W.splits_tensor([R, 5, -3, 0], DEV)  # invalid sizes: would set both status bits
    _quant(x1, bad, recipe, which, out, noop=flag, status=status)
    torch.cuda.synchronize()
    assert _same(out, before), "a call with the noop flag set wrote its outputs"
    assert int(status.item()) == 0, "a call with the noop flag set wrote the status word"
    flag.fill_(-2.5)  # any nonzero value counts as set
    _quant(x1, st, recipe, which, out, noop=flag, status=status)
    torch.cuda.synchronize()
    assert _same(out, before)
    # flag cleared: the same call now re-quantizes x1 in place
    flag.zero_()
    _quant(x1, bad, recipe, which, out, noop=flag, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == (bs.STATUS_NEGATIVE_SPLIT | bs.STATUS_EXCEEDS_CAPACITY)
    assert _same(out, before), "invalid split sizes must leave the outputs untouched"
    _quant(x1, st, recipe, which, out, noop=flag)
    fresh = _alloc(R, C, len(splits), recipe, which)
    _quant(x1, st, recipe, which, fresh)
    torch.cuda.synchronize()
    got, ref = _written_views(out, splits, R, C, which), _written_views(fresh, splits, R, C, which)
    old = _written_views(before, splits, R, C, which)
    for k in ref:
        assert np.array_equal(got[k], ref[k]), f"in-place re-quantize differs from a fresh call in {k}"
        assert not np.array_equal(got[k], old[k]), f"{k} was not re-quantized"


def test_in_place_reuse_with_new_routing():
    """Storage sized for the capacity is re-quantized in place for a second routing with fewer live
    rows: the bytes the second call documents as written match a fresh call, whatever the first
    call left there."""
    flush("in-place reuse, new routing")
    R, C, E = 900, 288, 3
    g = W._gen(DEV, 12)
    x = W.randn_bf16((R, C), g, DEV)
    which = bs.ROWWISE | bs.COLWISE
    out = _alloc(R, C, E, bs.RECIPE_MX, which)
    for splits in ([400, 300, 200], [0, 77, 129], [1, 0, 0]):
        st = W.splits_tensor(splits, DEV)
        _quant(x, st, bs.RECIPE_MX, which, out)
        fresh = _alloc(R, C, E, bs.RECIPE_MX, which)
        _quant(x, st, bs.RECIPE_MX, which, fresh)
        torch.cuda.synchronize()
        got, ref = _written_views(out, splits, R, C, which), _written_views(fresh, splits, R, C, which)
        for k in ref:
            assert np.array_equal(got[k], ref[k]), f"splits {splits}: {k} differs"


class _Layer:
    """Static buffers of one expert layer: everything a captured graph reads or writes."""

    def __init__(self, R, h, n, E):
        self.R, self.h, self.n, self.E = R, h, n, E
        MX = bs.RECIPE_MX
        self.x = torch.zeros((R, h), dtype=torch.bfloat16, device=DEV)
        self.dy = torch.zeros((R, n), dtype=torch.bfloat16, device=DEV)
        self.w = torch.zeros((E * n, h), dtype=torch.bfloat16, device=DEV)
        self.splits = torch.zeros(E, dtype=torch.int32, device=DEV)
        self.w_splits = W.splits_tensor([n] * E, DEV)
        self.flag = torch.zeros(1, dtype=torch.float32, device=DEV)
        self.status = torch.zeros(1, dtype=torch.int32, device=DEV)
        self.w_row = _alloc(E * n, h, 1, MX, bs.ROWWISE)
        self.w_col = _alloc(E * n, h, E, MX, bs.COLWISE)
        self.x_q = _alloc(R, h, E, MX, bs.ROWWISE | bs.COLWISE)
        self.dy_q = _alloc(R, n, E, MX, bs.ROWWISE | bs.COLWISE)
        self.y = torch.zeros((R, n), dtype=torch.bfloat16, device=DEV)
        self.dx = torch.zeros((R, h), dtype=torch.bfloat16, device=DEV)
        self.main_grad = torch.zeros((E, n, h), dtype=torch.float32, device=DEV)

    def step(self):
        """One microbatch: cached-weight quantize, forward, both backward GEMMs."""
        MX, R, h, n = bs.RECIPE_MX, self.R, self.h, self.n
        _quant(self.w, None, MX, bs.ROWWISE, self.w_row, noop=self.flag, status=self.status)
        _quant(self.w, self.w_splits, MX, bs.COLWISE, self.w_col, noop=self.flag, status=self.status)
        _quant(self.x, self.splits, MX, bs.ROWWISE | bs.COLWISE, self.x_q, status=self.status)
        bs.grouped_gemm_fprop(self.x_q, h, self.w_row, n, self.splits, R, self.y, bs.OUT_BF16, status=self.status)
        _quant(self.dy, self.splits, MX, bs.ROWWISE | bs.COLWISE, self.dy_q, status=self.status)
        bs.grouped_gemm_dgrad(self.dy_q, n, self.w_col, h, self.splits, R, self.dx, bs.OUT_BF16, status=self.status)
        bs.grouped_gemm_wgrad(self.dy_q, n, self.x_q, h, self.splits, R, MX, self.main_grad, accumulate=True,
                              status=self.status)

    def load(self, mb):
        """Eager host-side work between microbatches: new tokens, routing and flag."""
        self.x.copy_(mb["x"])
        self.dy.copy_(mb["dy"])
        self.splits.copy_(mb["splits_cpu"])
        self.w.copy_(mb["w"])
        self.flag.fill_(0.0 if mb["requant"] else 1.0)


def _microbatches(R, h, n, E, count, seed):
    rng = np.random.default_rng(seed)
    g = W._gen(DEV, seed)
    routings = [[300, 0, 411, 37], [128, 256, 1, 0], [R - 3, 0, 0, 3], [5, 900, 33, 64]][:count]
    mbs = []
    for i, splits in enumerate(routings):
        splits = [int(s) for s in splits]
        T = sum(splits)
        x = W._pad_rows(W.randn_bf16((T, h), g, DEV), R, "garbage", DEV, rng)
        dy = W._pad_rows(W.randn_bf16((T, n), g, DEV, scale=1e-3), R, "garbage", DEV, rng)
        w = W.randn_bf16((E * n, h), g, DEV, scale=0.05)  # a new weight every microbatch ...
        mbs.append(dict(x=x, dy=dy, w=w, splits=splits, splits_cpu=torch.tensor(splits, dtype=torch.int32),
                        requant=(i == 0)))  # ... that only the first one quantizes
    return mbs


def _live(t, splits):
    return t[:sum(splits)]


def test_graph_capture_replays_match_eager():
    R, h, n, E = 1024, 384, 288, 4
    mbs = _microbatches(R, h, n, E, 4, seed=21)
    eager, graphed = _Layer(R, h, n, E), _Layer(R, h, n, E)
    # eager run of the first microbatch (also loads every kernel before the capture)
    eager.load(mbs[0])
    eager.step()
    torch.cuda.synchronize()
    flush("graph: capture")
    graphed.load(mbs[0])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        graphed.step()
    # capture records the launches without running them: main_grad must still be zero
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(graphed.main_grad).item()) == 0
    for i, mb in enumerate(mbs):
        flush(f"graph: replay {i} splits={mb['splits']} requant={mb['requant']}")
        if i > 0:
            eager.load(mb)
            eager.step()
        graphed.load(mb)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert int(graphed.status.item()) == 0 and int(eager.status.item()) == 0
        sp = mb["splits"]
        assert torch.equal(_live(graphed.y, sp).view(torch.int16), _live(eager.y, sp).view(torch.int16)), \
            f"replay {i}: y differs from the eager run"
        assert torch.equal(_live(graphed.dx, sp).view(torch.int16), _live(eager.dx, sp).view(torch.int16)), \
            f"replay {i}: dx differs from the eager run"
        assert torch.equal(graphed.main_grad.view(torch.int32), eager.main_grad.view(torch.int32)), \
            f"replay {i}: main_grad differs from the eager run"
        for k in ("row_q", "row_s"):
            assert torch.equal(graphed.w_row[k], eager.w_row[k]), f"replay {i}: cached weight {k} differs"
        if i == 0:
            _check_first_replay_against_oracle(graphed, mb)
    # the cached weight is still the first microbatch's: the later bf16 weights never reached it
    fresh = _alloc(E * n, h, 1, bs.RECIPE_MX, bs.ROWWISE)
    _quant(mbs[0]["w"], None, bs.RECIPE_MX, bs.ROWWISE, fresh)
    torch.cuda.synchronize()
    assert torch.equal(fresh["row_q"], graphed.w_row["row_q"])


def _check_first_replay_against_oracle(layer, mb):
    """Sampled rows of y and dx and one expert's main_grad against the fp64 oracle."""
    splits, h, n, E = mb["splits"], layer.h, layer.n, layer.E
    offs = np.concatenate([[0], np.cumsum(splits)]).astype(np.int64)
    e = int(np.argmax(splits))
    ke, off = splits[e], int(offs[e])
    xb = W.bf16_bits(mb["x"][off:off + ke])
    dyb = W.bf16_bits(mb["dy"][off:off + ke])
    wb = W.bf16_bits(mb["w"][e * n:(e + 1) * n])
    ox = oracle.grouped_quantize(xb, [ke], oracle.RECIPE_MX, oracle.ROWWISE | oracle.COLWISE)
    ody = oracle.grouped_quantize(dyb, [ke], oracle.RECIPE_MX, oracle.ROWWISE | oracle.COLWISE)
    ow_row = oracle.grouped_quantize(wb, None, oracle.RECIPE_MX, oracle.ROWWISE)
    ow_col = oracle.grouped_quantize(wb, [n], oracle.RECIPE_MX, oracle.COLWISE)
    y_ref = oracle.grouped_fprop(ox["row_q"], ox["row_s"], ow_row["row_q"], ow_row["row_s"], n, [ke])
    dx_ref = oracle.grouped_dgrad(ody["row_q"], ody["row_s"], ow_col["col_q"], ow_col["col_s"], h, [ke])
    dw_ref = oracle.grouped_wgrad(ody["col_q"], ody["col_s"], n, ox["col_q"], ox["col_s"], h, [ke], ke,
                                  oracle.RECIPE_MX)
    y = layer.y[off:off + ke].float().cpu().numpy().astype(np.float64)
    dx = layer.dx[off:off + ke].float().cpu().numpy().astype(np.float64)
    assert_bf16_close(y, y_ref, f"first replay: y of expert {e}")
    assert_bf16_close(dx, dx_ref, f"first replay: dx of expert {e}")
    dw = layer.main_grad[e].cpu().numpy().astype(np.float64)  # 0 + dW: one exact fp32 add
    assert rel_err(dw, dw_ref[0]) <= REL_TOL, "first replay: main_grad against the oracle"
    for o in range(E):
        if splits[o] == 0:
            assert int(torch.count_nonzero(layer.main_grad[o]).item()) == 0, "an empty expert's main_grad moved"

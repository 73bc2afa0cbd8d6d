"""Seeded synthetic inputs for block-scaled FP8 grouped quantize / wgrad / fprop.

This module draws random numbers, routing counts and padding only; it holds none of the
method's arithmetic, so both the HIP path and the CPU oracle can take their inputs from it.
Shapes, value scales and structure follow the workloads of the source pages:

* DeepGEMM issue #365 (reproducer): four experts with 256/128/128/256 tokens, grad_y drawn as
  randn * 1e-7, activations as randn * 0.4, one all-zero grad_y channel in each 128-token expert.
* TransformerEngine issue #3484 (reproducer): one group of 512 live rows of randn, hidden
  1024, a buffer padded by 256 rows filled with 0.0 or with 3.0.
* Two MoE-layer shapes with routing-count skew (Zipf) and with empty experts, chosen to cover
  counts that are not multiples of 32 and garbage padding.

Every tensor is generated with ``torch`` from an explicit seed on the requested device.
"""
import numpy as np
import torch

BF16 = torch.bfloat16


def _gen(device, seed):
    return torch.Generator(device=device).manual_seed(seed)


def randn_bf16(shape, generator, device, scale=1.0, chunk_elems=1 << 28):
    """Standard normal draws in fp32, times ``scale``, rounded once to bf16.

    Drawing in fp32 keeps unit variance on every device (the CPU bf16 sampler does not: its
    standard deviation is about 0.993).  Large tensors are drawn in row chunks."""
    shape = tuple(int(d) for d in shape)
    out = torch.empty(shape, dtype=BF16, device=device)
    rows = shape[0]
    per_row = max(1, int(np.prod(shape[1:])))
    step = max(1, chunk_elems // per_row)
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        v = torch.randn((r1 - r0,) + shape[1:], dtype=torch.float32, device=device, generator=generator)
        if scale != 1.0:
            v.mul_(scale)
        out[r0:r1] = v.to(BF16)
        del v
    return out


def _pad_rows(live, R, fill, device, garbage_rng=None):
    """[R, C] buffer whose first rows are ``live`` and the rest padding.

    fill: a float constant, or "garbage" for random 16-bit patterns (NaN/Inf included).
    """
    T, C = live.shape
    if R == T:
        return live.contiguous()
    buf = torch.empty((R, C), dtype=BF16, device=device)
    buf[:T] = live
    if fill == "garbage":
        bits = garbage_rng.integers(0, 1 << 16, size=(R - T, C), dtype=np.uint16)
        buf[T:] = torch.from_numpy(bits.view(np.int16)).to(device).view(BF16)
    else:
        buf[T:] = fill
    return buf


def zipf_counts(rng, num_experts, live_experts, tokens, s=1.1):
    """Routing counts: Zipf(s) weights over ``live_experts`` ranks, mapped to experts by a random
    permutation; the remaining experts get no token."""
    perm = rng.permutation(num_experts)
    w = np.arange(1, live_experts + 1, dtype=np.float64) ** (-s)
    p = np.zeros(num_experts)
    p[perm[:live_experts]] = w / w.sum()
    return rng.multinomial(tokens, p).astype(np.int64)


def uniform_counts_with_empty(rng, num_experts, num_empty, tokens):
    empty = rng.choice(num_experts, num_empty, replace=False)
    live = np.setdiff1d(np.arange(num_experts), empty)
    p = np.zeros(num_experts)
    p[live] = 1.0 / live.size
    return rng.multinomial(tokens, p).astype(np.int64)


def deepgemm_case(device, n, h, splits=(256, 128, 128, 256), R=None, pad_fill=3.0, seed=0,
                  zero_channel_in_128=True):
    """The DeepGEMM #365 structure: dy = randn*1e-7 [T, n], x = randn*0.4 [T, h] (drawn in that
    order from one generator), dy channel 0 zeroed in every 128-token expert; the buffer is
    padded to R rows with ``pad_fill``."""
    splits = [int(k) for k in splits]
    T = sum(splits)
    R = T if R is None else R
    g = _gen(device, seed)
    dy = randn_bf16((T, n), g, device, 1e-7)
    x = randn_bf16((T, h), g, device, 0.4)
    off = 0
    for k in splits:
        if k == 128 and zero_channel_in_128:
            dy[off:off + k, 0] = 0
        off += k
    return dict(dy=_pad_rows(dy, R, pad_fill, device), x=_pad_rows(x, R, pad_fill, device),
                splits=splits, R=R, T=T, n=n, h=h)


def te_single_group_case(device, R=512, pad_fill=0.0, live=512, hidden=1024, seed=1):
    """The TE #3484 structure: one group of ``live`` randn rows (x drawn before dy), hidden x
    hidden weight gradient, the buffer padded to R rows with ``pad_fill``; main_grad zeros."""
    g = _gen(device, seed)
    x = randn_bf16((live, hidden), g, device)
    dy = randn_bf16((live, hidden), g, device)
    return dict(dy=_pad_rows(dy, R, pad_fill, device), x=_pad_rows(x, R, pad_fill, device),
                splits=[live], R=R, T=live, n=hidden, h=hidden,
                main_grad=torch.zeros(1, hidden, hidden, dtype=torch.float32, device=device))


def moe_case(device, num_experts, tokens, hidden, ffn, routing, seed, scale=1.0, pad_to=None,
             pad_fill="garbage", with_weight=True, with_main_grad=False):
    """An MoE expert layer: x [T, hidden] (fprop input and wgrad activation), dy [T, ffn] (the
    gradient at the expert output), W [E, ffn, hidden]; all bf16 (fp32 standard normal times scale, rounded once).

    routing: ("zipf", live_experts) or ("uniform_empty", num_empty).
    pad_to : None (R = T) or a row multiple; when T is already a multiple, one more block of
             that many rows is added so that padding exists.
    """
    rng = np.random.default_rng(seed)
    if routing[0] == "zipf":
        counts = zipf_counts(rng, num_experts, routing[1], tokens)
    else:
        counts = uniform_counts_with_empty(rng, num_experts, routing[1], tokens)
    T = int(counts.sum())
    if pad_to is None:
        R = T
    else:
        R = ((T + pad_to - 1) // pad_to) * pad_to
        if R == T:
            R += pad_to
    g = _gen(device, seed)
    x = randn_bf16((T, hidden), g, device, scale)
    dy = randn_bf16((T, ffn), g, device, scale)
    out = dict(splits=[int(c) for c in counts], R=R, T=T, n=ffn, h=hidden, K=hidden, N=ffn)
    out["x"] = _pad_rows(x, R, pad_fill, device, rng)
    del x
    out["dy"] = _pad_rows(dy, R, pad_fill, device, rng)
    del dy
    if with_weight:
        out["W"] = randn_bf16((num_experts, ffn, hidden), g, device, scale)
    if with_main_grad:
        out["main_grad"] = torch.randn(num_experts, ffn, hidden, dtype=torch.float32, device=device,
                                       generator=g)
    return out


def moe32_zipf(device, **kw):
    """32 experts, 65,536 routed tokens, Zipf(1.1) counts over 28 experts (4 empty), hidden 4096,
    ffn 1536, sigma 1, padded to a multiple of 128 with garbage bits."""
    return moe_case(device, 32, 65536, 4096, 1536, ("zipf", 28), seed=4, pad_to=128, **kw)


def moe128_top8(device, **kw):
    """128 experts, 131,072 tokens x top-8 = 1,048,576 expert rows, 6 empty experts, uniform
    multinomial counts over the rest, hidden 7168, ffn 2048, randn * 0.5, no padding."""
    kw.setdefault("with_main_grad", True)
    return moe_case(device, 128, 131072 * 8, 7168, 2048, ("uniform_empty", 6), seed=5, scale=0.5, **kw)


def splits_tensor(splits, device):
    return torch.tensor(list(splits), dtype=torch.int32, device=device)


def bf16_bits(t):
    """uint16 numpy view of a bf16 tensor (copied to the host)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)

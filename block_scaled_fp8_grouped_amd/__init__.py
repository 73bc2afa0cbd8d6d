"""Block-scaled FP8 grouped quantize / wgrad / fprop for MoE expert layers on MI355X (gfx950).

Thin ctypes binding of ``libbsfp8.so``.  It only marshals arguments: tensor data pointers,
sizes and torch's current HIP stream go to the C ABI declared in ``include/bsfp8.h``; every
step of the computation runs in the library's kernels.  PyTorch supplies device memory and the
stream.  If the library has not been built, importing works but every call raises.

Functions keep the C names without the ``bsfp8_`` prefix:
  grouped_quantize, grouped_gemm_wgrad, grouped_gemm_fprop, the size queries, strerror.
``alloc_quantized`` and ``alloc_*`` helpers size output tensors with the library's own size
queries.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsfp8.so")

RECIPE_MX = 1  # BSFP8_RECIPE_MX_1X32_E8M0
RECIPE_PC = 2  # BSFP8_RECIPE_PER_CHANNEL_128_F32
RECIPE_MX4 = 3  # BSFP8_RECIPE_MXFP4_1X32_E8M0
GEMM_FP8_MFMA = 0x100  # BSFP8_GEMM_FP8_MFMA: OR into RECIPE_MX for the GEMMs on the scaled fp8 MFMA
ROWWISE = 1
COLWISE = 2
ACT_SRELU = 1  # BSFP8_ACT_SRELU: y = p * max(h, 0)^2
ACT_SRELU_GRAD = 2  # BSFP8_ACT_SRELU_GRAD: g = dy * p * 2 max(h, 0)
ACT_SWIGLU = 3  # BSFP8_ACT_SWIGLU: y = p * silu(a) * b, h = (a | b)
ACT_SWIGLU_GRAD = 4  # BSFP8_ACT_SWIGLU_GRAD: (da | db) of the scaled SwiGLU
OUT_F32 = 0
OUT_BF16 = 1
STATUS_NEGATIVE_SPLIT = 1
STATUS_EXCEEDS_CAPACITY = 2
MAX_GROUPS = 1024

_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t

_lib = None


class BSFP8Error(RuntimeError):
    pass


def lib():
    """The loaded libbsfp8.so; raises when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise BSFP8Error(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                             "(or python -m block_scaled_fp8_grouped_amd._build)")
        L = ctypes.CDLL(LIB_PATH)
        L.bsfp8_colwise_rows_bound.restype = _i64
        L.bsfp8_colwise_rows_bound.argtypes = [_i64, _i32]
        L.bsfp8_colwise_data_bytes.restype = _sz
        L.bsfp8_colwise_data_bytes.argtypes = [_i64, _i64, _i32, ctypes.c_int]
        L.bsfp8_colwise_scale_bytes.restype = _sz
        L.bsfp8_colwise_scale_bytes.argtypes = [_i64, _i64, _i32, ctypes.c_int]
        L.bsfp8_rowwise_data_bytes.restype = _sz
        L.bsfp8_rowwise_data_bytes.argtypes = [_i64, _i64, ctypes.c_int]
        L.bsfp8_rowwise_scale_bytes.restype = _sz
        L.bsfp8_rowwise_scale_bytes.argtypes = [_i64, _i64]
        L.bsfp8_grouped_quantize.restype = ctypes.c_int
        L.bsfp8_grouped_quantize.argtypes = [_vp, _i64, _i64, _vp, _i32, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_float, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.bsfp8_grouped_act_quantize.restype = ctypes.c_int
        L.bsfp8_grouped_act_quantize.argtypes = [ctypes.c_int, _vp, _vp, _vp, _i64, _i64, _vp, _i32, ctypes.c_int,
                                                 ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp]
        L.bsfp8_grouped_gemm_wgrad.restype = ctypes.c_int
        L.bsfp8_grouped_gemm_wgrad.argtypes = [_vp, _vp, _i64, _vp, _vp, _i64, _vp, _i32, _i64, ctypes.c_int,
                                               _vp, ctypes.c_int, _vp, _vp]
        L.bsfp8_grouped_gemm_fprop.restype = ctypes.c_int
        L.bsfp8_grouped_gemm_fprop.argtypes = [_vp, _vp, _i64, _i64, _vp, _vp, _i64, _vp, _i32, ctypes.c_int, _vp,
                                               ctypes.c_int, _vp, _vp]
        L.bsfp8_grouped_gemm_dgrad.restype = ctypes.c_int
        L.bsfp8_grouped_gemm_dgrad.argtypes = [_vp, _vp, _i64, _i64, _vp, _vp, _i64, _vp, _i32, ctypes.c_int, _vp,
                                               ctypes.c_int, _vp, _vp]
        L.bsfp8_strerror.restype = ctypes.c_char_p
        L.bsfp8_strerror.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def strerror(code):
    return lib().bsfp8_strerror(int(code)).decode()


def _check(rc, what):
    if rc != 0:
        raise BSFP8Error(f"{what}: {strerror(rc)} ({rc})")


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        return int(t)  # a raw address
    return t.data_ptr()


_U8 = (torch.uint8,)
_BF16 = (torch.bfloat16, torch.int16)  # bf16 data, or its bits viewed as int16
_F32 = (torch.float32,)
_I32 = (torch.int32,)
_F32_BITS = (torch.float32, torch.int32)


def _dev(t, what, dtypes):
    """Pointer of an argument that the kernels read or write: a contiguous device tensor of one
    of ``dtypes`` (checked in that order, so a wrong type is reported before a wrong device), a
    raw device address (int, not checked), or None.  A host tensor would hand the GPU a host
    pointer, and a tensor of another element type would be read with the wrong layout (an int64
    split_sizes tensor reads as sizes k_0, 0, k_1, 0, ...)."""
    if t is None or not isinstance(t, torch.Tensor):
        return _ptr(t)
    if t.dtype not in dtypes:
        raise TypeError(f"{what}: dtype {t.dtype}, expected {' or '.join(str(d) for d in dtypes)}")
    if t.device.type != "cuda":
        raise ValueError(f"{what}: a {t.device.type} tensor; the library takes device memory")
    if not t.is_contiguous():
        raise ValueError(f"{what}: not contiguous")
    return t.data_ptr()


def _quant(q, key, what, dtypes=_U8):
    return _dev(q.get(key), f"{what}[{key!r}]", dtypes)


def _need(t, nbytes, what):
    """A tensor argument must hold at least the bytes the kernels address for the given sizes and
    recipe (a buffer quantized with another recipe, or sized for other dims, would be read or
    written past its end); raw addresses are not checked."""
    if isinstance(t, torch.Tensor) and nbytes > 0 and t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{what}: {t.numel() * t.element_size()} bytes, the call addresses {nbytes}")


def _need_quant(q, recipe, rows, cols, num_groups, which, what):
    """The quantized buffers of ``q`` against the layouts ``which`` of a [rows, cols] operand with
    ``num_groups`` groups: at least the size queries' bytes (alloc_quantized's sizes; a colwise
    buffer holds up to that bound, depending on the device split sizes).  With no rows nothing is
    addressed."""
    if rows == 0:
        return
    r = recipe & ~GEMM_FP8_MFMA
    if which & ROWWISE:
        _need(q.get("row_q"), rowwise_data_bytes(rows, cols, r), f"{what}['row_q']")
        _need(q.get("row_s"), rowwise_scale_bytes(rows, cols), f"{what}['row_s']")
    if which & COLWISE:
        _need(q.get("col_q"), colwise_data_bytes(rows, cols, num_groups, r), f"{what}['col_q']")
        _need(q.get("col_s"), colwise_scale_bytes(rows, cols, num_groups, r), f"{what}['col_s']")


def _col_s_types(recipe):
    return _F32 if (recipe & ~GEMM_FP8_MFMA) == RECIPE_PC else _U8


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


# ------------------------------------------------------------------------------------------
# size queries
# ------------------------------------------------------------------------------------------

def colwise_rows_bound(capacity_rows, num_groups):
    return int(lib().bsfp8_colwise_rows_bound(capacity_rows, num_groups))


def colwise_data_bytes(capacity_rows, cols, num_groups, recipe=RECIPE_MX):
    return int(lib().bsfp8_colwise_data_bytes(capacity_rows, cols, num_groups, recipe))


def colwise_scale_bytes(capacity_rows, cols, num_groups, recipe):
    return int(lib().bsfp8_colwise_scale_bytes(capacity_rows, cols, num_groups, recipe))


def rowwise_data_bytes(rows, cols, recipe=RECIPE_MX):
    return int(lib().bsfp8_rowwise_data_bytes(rows, cols, recipe))


def rowwise_scale_bytes(rows, cols):
    return int(lib().bsfp8_rowwise_scale_bytes(rows, cols))


def alloc_quantized(capacity_rows, cols, num_groups, recipe, which, device="cuda"):
    """Output tensors for grouped_quantize, sized by the library's size queries.

    Returns a dict with row_q uint8 [R, C] (MXFP4: [R, C/2]), row_s uint8 [C/32, R], col_q uint8
    [bytes], col_s uint8 [bytes] (MX recipes) or float32 [bytes/4] (per-channel), for the
    requested layouts."""
    out = {}
    if which & ROWWISE:
        per = 2 if recipe == RECIPE_MX4 else 1
        out["row_q"] = torch.empty((capacity_rows, cols // per), dtype=torch.uint8, device=device)
        out["row_s"] = torch.empty((cols // 32, capacity_rows), dtype=torch.uint8, device=device)
    if which & COLWISE:
        out["col_q"] = torch.empty(colwise_data_bytes(capacity_rows, cols, num_groups, recipe), dtype=torch.uint8,
                                   device=device)
        nb = colwise_scale_bytes(capacity_rows, cols, num_groups, recipe)
        if recipe != RECIPE_PC:
            out["col_s"] = torch.empty(nb, dtype=torch.uint8, device=device)
        else:
            out["col_s"] = torch.empty(nb // 4, dtype=torch.float32, device=device)
    return out


# ------------------------------------------------------------------------------------------
# entry points
# ------------------------------------------------------------------------------------------

def grouped_quantize(x, split_sizes, recipe, which, out, zero_amax_scale=1e-30, status=None, stream=None,
                     capacity_rows=None, cols=None, noop_flag=None):
    """bsfp8_grouped_quantize on a bf16 [R, C] tensor; ``out`` holds the output tensors
    (see alloc_quantized), overwritten in place.  split_sizes: int32 device tensor, or None
    (rowwise, all rows live).  noop_flag: None, or a float32 device scalar; when it holds a
    nonzero value at run time the call leaves ``out`` (and ``status``) as they are."""
    if isinstance(x, torch.Tensor):
        R, C = x.shape if capacity_rows is None else (capacity_rows, cols)
    else:
        R, C = capacity_rows, cols
    E = 0 if split_sizes is None else int(split_sizes.numel())
    args = (_dev(x, "x", _BF16), R, C, _dev(split_sizes, "split_sizes", _I32), E, recipe, which,
            float(zero_amax_scale), _quant(out, "row_q", "out"), _quant(out, "row_s", "out"),
            _quant(out, "col_q", "out"), _quant(out, "col_s", "out", _col_s_types(recipe)),
            _dev(noop_flag, "noop_flag", _F32), _dev(status, "status", _I32), _stream(stream))
    _need(x, R * C * 2, "x")
    _need_quant(out, recipe, R, C, max(E, 1), which, "out")
    rc = lib().bsfp8_grouped_quantize(*args)
    _check(rc, "grouped_quantize")
    return out


def grouped_act_quantize(activation, h, split_sizes, recipe, which, out, probs=None, dy=None, status=None,
                         stream=None):
    """bsfp8_grouped_act_quantize: the scaled squared ReLU (ACT_SRELU) of the bf16 [R, C] tensor
    h, or its gradient (ACT_SRELU_GRAD, with the bf16 gradient dy [R, C]); or the scaled SwiGLU
    (ACT_SWIGLU) of h = (a | b) [R, 2F], or its gradient (ACT_SWIGLU_GRAD, dy [R, F]); times the
    float32 per-row probs (None: 1), quantized into ``out`` with an MX recipe.  ``out`` comes
    from alloc_quantized for [R, C], [R, F] (ACT_SWIGLU) or [R, 2F] (ACT_SWIGLU_GRAD)."""
    R, C = h.shape
    if activation in (ACT_SWIGLU, ACT_SWIGLU_GRAD):
        if C % 2:
            raise ValueError("grouped_act_quantize: a GLU input has an even number of columns")
        C //= 2
    E = int(split_sizes.numel())
    args = (activation, _dev(h, "h", _BF16), _dev(probs, "probs", _F32), _dev(dy, "dy", _BF16), R, C,
            _dev(split_sizes, "split_sizes", _I32), E, recipe, which, _quant(out, "row_q", "out"),
            _quant(out, "row_s", "out"), _quant(out, "col_q", "out"), _quant(out, "col_s", "out"),
            _dev(status, "status", _I32), _stream(stream))
    _need_quant(out, recipe, R, 2 * C if activation == ACT_SWIGLU_GRAD else C, E, which, "out")
    rc = lib().bsfp8_grouped_act_quantize(*args)
    _check(rc, "grouped_act_quantize")
    return out


def grouped_gemm_wgrad(dy_q, n, x_q, h, split_sizes, capacity_rows, recipe, out, accumulate=False, status=None,
                       stream=None):
    """bsfp8_grouped_gemm_wgrad: dy_q / x_q are the colwise dicts of grouped_quantize; out is
    fp32 [E, n, h] (overwritten, or accumulated into with ``accumulate``).  recipe: the data
    recipe, or RECIPE_MX | GEMM_FP8_MFMA for the MXFP8 operands on the scaled fp8 MFMA."""
    E = int(split_sizes.numel())
    cs = _col_s_types(recipe)
    args = (_quant(dy_q, "col_q", "dy_q"), _quant(dy_q, "col_s", "dy_q", cs), n, _quant(x_q, "col_q", "x_q"),
            _quant(x_q, "col_s", "x_q", cs), h, _dev(split_sizes, "split_sizes", _I32), E, capacity_rows, recipe,
            _dev(out, "out", _F32_BITS), 1 if accumulate else 0, _dev(status, "status", _I32), _stream(stream))
    _need_quant(dy_q, recipe, capacity_rows, n, E, COLWISE, "dy_q")
    _need_quant(x_q, recipe, capacity_rows, h, E, COLWISE, "x_q")
    _need(out, E * n * h * 4, "out")
    rc = lib().bsfp8_grouped_gemm_wgrad(*args)
    _check(rc, "grouped_gemm_wgrad")
    return out


def grouped_gemm_fprop(x_q, k, w_q, n, split_sizes, capacity_rows, out, out_dtype=OUT_F32, status=None,
                       stream=None, recipe=RECIPE_MX):
    """bsfp8_grouped_gemm_fprop: x_q is the rowwise dict of x [R, k], w_q the rowwise dict of the
    weight [E*n, k], both of ``recipe`` (MX or MX4; RECIPE_MX | GEMM_FP8_MFMA multiplies MX
    operands on the scaled fp8 MFMA); out is [R, n] fp32 or bf16 (rows past
    sum(split_sizes) untouched)."""
    E = int(split_sizes.numel())
    args = (_quant(x_q, "row_q", "x_q"), _quant(x_q, "row_s", "x_q"), capacity_rows, k, _quant(w_q, "row_q", "w_q"),
            _quant(w_q, "row_s", "w_q"), n, _dev(split_sizes, "split_sizes", _I32), E, recipe,
            _dev(out, "out", _F32_BITS if out_dtype == OUT_F32 else _BF16), out_dtype,
            _dev(status, "status", _I32), _stream(stream))
    _need_quant(x_q, recipe, capacity_rows, k, E, ROWWISE, "x_q")
    _need_quant(w_q, recipe, E * n, k, 1, ROWWISE, "w_q")
    _need(out, capacity_rows * n * (4 if out_dtype == OUT_F32 else 2), "out")
    rc = lib().bsfp8_grouped_gemm_fprop(*args)
    _check(rc, "grouped_gemm_fprop")
    return out


def grouped_gemm_dgrad(dy_q, n, w_q, k, split_sizes, capacity_rows, out, out_dtype=OUT_F32, status=None,
                       stream=None, recipe=RECIPE_MX):
    """bsfp8_grouped_gemm_dgrad: dy_q is the rowwise dict of dy [R, n]; w_q the colwise dict of the
    weight viewed as [E*n, k] quantized with split sizes [n] * E (blocks of 32 along n inside each
    expert); out is [R, k] fp32 or bf16: out[off_e + t] = dy[off_e + t] @ W_e (rows past
    sum(split_sizes) untouched)."""
    E = int(split_sizes.numel())
    args = (_quant(dy_q, "row_q", "dy_q"), _quant(dy_q, "row_s", "dy_q"), capacity_rows, n,
            _quant(w_q, "col_q", "w_q"), _quant(w_q, "col_s", "w_q"), k, _dev(split_sizes, "split_sizes", _I32), E,
            recipe, _dev(out, "out", _F32_BITS if out_dtype == OUT_F32 else _BF16), out_dtype,
            _dev(status, "status", _I32), _stream(stream))
    _need_quant(dy_q, recipe, capacity_rows, n, E, ROWWISE, "dy_q")
    # the weight [E*n, k] quantized colwise with split sizes n: E groups of 128 * ceil(n / 128) rows
    np_ = 128 * ((n + 127) // 128)
    per = 2 if (recipe & ~GEMM_FP8_MFMA) == RECIPE_MX4 else 1
    _need(w_q.get("col_q"), k * E * np_ // per, "w_q['col_q']")
    _need(w_q.get("col_s"), k * E * np_ // 32, "w_q['col_s']")
    _need(out, capacity_rows * k * (4 if out_dtype == OUT_F32 else 2), "out")
    rc = lib().bsfp8_grouped_gemm_dgrad(*args)
    _check(rc, "grouped_gemm_dgrad")
    return out

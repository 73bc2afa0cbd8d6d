"""ctypes binding of the plain CPU oracle in ``oracle.c``.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` are the only callers.  The product library never imports, links or runs anything
here, and this module imports nothing from the product package.

All arrays are numpy arrays on the host.  bf16 inputs are passed as their uint16 bit patterns.
Every function documents the layout it produces; the layouts are derived in ``oracle.c`` on
their own (see its header).
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

RECIPE_MX = 1  # MXFP8: e4m3 data, one E8M0 power-of-two scale per 32 elements
RECIPE_PC = 2  # per channel: e4m3 data, one fp32 scale per 128 rows
RECIPE_MX4 = 3  # MXFP4: e2m1 data packed two per byte, one E8M0 power-of-two scale per 32 elements
ROWWISE = 1
COLWISE = 2

_lib = None

_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_vp = ctypes.c_void_p


def build():
    """Compile oracle.c with plain IEEE settings (no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
           "-std=c11", "-Wall", _SRC, "-o", LIB_PATH + ".tmp", "-lm"]
    subprocess.check_call(cmd)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e4m3_encode_array.argtypes = [_vp, _vp, _i64]
        L.oracle_e4m3_decode_array.argtypes = [_vp, _vp, _i64]
        L.oracle_e8m0_exponent.restype = ctypes.c_int
        L.oracle_e8m0_exponent.argtypes = [ctypes.c_float]
        L.oracle_e8m0_exponent_array.argtypes = [_vp, _vp, _i64]
        L.oracle_e2m1_decode.restype = ctypes.c_double
        L.oracle_e2m1_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e2m1_encode.restype = ctypes.c_uint8
        L.oracle_e2m1_encode.argtypes = [ctypes.c_float]
        L.oracle_e2m1_encode_array.argtypes = [_vp, _vp, _i64]
        L.oracle_e8m0_exponent_fp4.restype = ctypes.c_int
        L.oracle_e8m0_exponent_fp4.argtypes = [ctypes.c_float]
        L.oracle_e8m0_exponent_fp4_array.argtypes = [_vp, _vp, _i64]
        L.oracle_padded_rows.restype = _i64
        L.oracle_padded_rows.argtypes = [_vp, _i32]
        L.oracle_grouped_quantize.restype = ctypes.c_int
        L.oracle_grouped_quantize.argtypes = [_vp, _i64, _i64, _vp, _i32, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_float, _vp, _vp, _vp, _vp]
        L.oracle_act_values.argtypes = [ctypes.c_int, _vp, _vp, _vp, _i64, _vp]
        L.oracle_exp2_spec.restype = ctypes.c_float
        L.oracle_exp2_spec.argtypes = [ctypes.c_float]
        L.oracle_glu_values.argtypes = [ctypes.c_int, _vp, _vp, _vp, _vp, _i64, _vp, _vp]
        L.oracle_grouped_act_quantize.restype = ctypes.c_int
        L.oracle_grouped_act_quantize.argtypes = [ctypes.c_int, _vp, _vp, _vp, _i64, _i64, _vp, _i32, ctypes.c_int,
                                                  ctypes.c_int, _vp, _vp, _vp, _vp]
        L.oracle_grouped_wgrad.restype = ctypes.c_int
        L.oracle_grouped_wgrad.argtypes = [_vp, _vp, _i64, _vp, _vp, _i64, _vp, _i32, _i64, ctypes.c_int,
                                           _vp, _i32, ctypes.c_int, _vp, _vp]
        L.oracle_grouped_fprop.restype = ctypes.c_int
        L.oracle_grouped_fprop.argtypes = [_vp, _vp, _i64, _i64, _vp, _vp, _i64, _vp, _i32, ctypes.c_int, _vp, _i32,
                                           _vp]
        L.oracle_grouped_dgrad.restype = ctypes.c_int
        L.oracle_grouped_dgrad.argtypes = [_vp, _vp, _i64, _i64, _vp, _vp, _i64, _vp, _i32, ctypes.c_int, _vp, _i32,
                                           _vp]
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_num_threads.argtypes = []
        L.oracle_wgrad_unquantized.restype = ctypes.c_int
        L.oracle_wgrad_unquantized.argtypes = [_vp, _i64, _vp, _i64, _vp, _i32, _i64, _vp]
        _lib = L
    return _lib


def num_threads():
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().oracle_num_threads())


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def e4m3_encode(v):
    """Nearest-even OCP E4M3FN code of every float32 in ``v`` (magnitudes >= 448 give 448)."""
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().oracle_e4m3_encode_array(_p(v), _p(out), v.size)
    return out


def e4m3_decode(q):
    """Exact value (float64) of every e4m3 code in ``q``."""
    q = _c(q, np.uint8)
    out = np.empty(q.shape, np.float64)
    lib().oracle_e4m3_decode_array(_p(q), _p(out), q.size)
    return out


def e8m0_exponent(amax):
    """MXFP8 block exponent e (int32) for every float32 block amax."""
    a = _c(amax, np.float32)
    out = np.empty(a.shape, np.int32)
    lib().oracle_e8m0_exponent_array(_p(a), _p(out), a.size)
    return out


def e2m1_encode(v):
    """Nearest-even OCP FP4 E2M1 code (0..15) of every float32 in ``v`` (magnitudes >= 6 give 6)."""
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().oracle_e2m1_encode_array(_p(v), _p(out), v.size)
    return out


def e2m1_decode(q):
    """Exact value (float64) of every e2m1 code (low 4 bits) in ``q``."""
    q = _c(q, np.uint8)
    return np.array([lib().oracle_e2m1_decode(int(c)) for c in q.ravel()], np.float64).reshape(q.shape)


def e8m0_exponent_fp4(amax):
    """MXFP4 block exponent e (int32) for every float32 block amax."""
    a = _c(amax, np.float32)
    out = np.empty(a.shape, np.int32)
    lib().oracle_e8m0_exponent_fp4_array(_p(a), _p(out), a.size)
    return out


def padded_rows(splits):
    s = _c(splits, np.int32)
    return int(lib().oracle_padded_rows(_p(s), s.size))


def grouped_quantize(x_bits, splits, recipe, which, zero_amax_scale=1e-30):
    """Quantize a bf16 [R, C] buffer (uint16 bit patterns).

    Returns a dict with, for the requested layouts:
      row_q uint8 [R, C] and row_s uint8 [C/32, R]   (rows not live are left 0)
      col_q uint8 [C * sum(Kp_e)] and col_s uint8 [C * sum(Kp_e) / 32] (MX) or
      float32 [C * sum(Kp_e) / 128] (per-channel).
    MXFP4 (RECIPE_MX4) packs two e2m1 codes per byte: row_q is uint8 [R, C/2] and col_q has
    C * sum(Kp_e) / 2 bytes; the scales are as for MX.
    ``splits`` may be None for rowwise-only quantization of a fully live buffer.
    """
    x = _c(x_bits, np.uint16)
    R, C = x.shape
    out = {}
    s = None if splits is None else _c(splits, np.int32)
    E = 0 if s is None else s.size
    row_q = row_s = col_q = col_s = None
    per = 2 if recipe == RECIPE_MX4 else 1  # elements per data byte
    if which & ROWWISE:
        row_q = np.zeros((R, C // per), np.uint8)
        row_s = np.zeros((C // 32, R), np.uint8)
        out["row_q"], out["row_s"] = row_q, row_s
    if which & COLWISE:
        rows = padded_rows(s)
        col_q = np.zeros(C * rows // per, np.uint8)
        if recipe != RECIPE_PC:
            col_s = np.zeros(C * rows // 32, np.uint8)
        else:
            col_s = np.zeros(C * rows // 128, np.float32)
        out["col_q"], out["col_s"] = col_q, col_s
    rc = lib().oracle_grouped_quantize(_p(x), R, C, _p(s), E, recipe, which, float(zero_amax_scale),
                                       _p(row_q), _p(row_s), _p(col_q), _p(col_s))
    if rc != 0:
        raise ValueError(f"oracle_grouped_quantize failed ({rc})")
    return out


ACT_SRELU_FWD = 1  # y = p * relu(h)^2
ACT_SRELU_BWD = 2  # g = dy * p * 2 relu(h)
ACT_SWIGLU_FWD = 3  # y = silu(a) * b * p, (a | b) the halves of fc1's output row
ACT_SWIGLU_BWD = 4  # (da | db) from dy * p


def exp2_spec(x):
    """The stated fp32 2^x of the GLU activations (see oracle.c), element by element."""
    x = np.asarray(x, np.float32)
    return np.array([lib().oracle_exp2_spec(float(v)) for v in x.ravel()], np.float32).reshape(x.shape)


def glu_values(act, a_bits, b_bits, p, dy_bits=None):
    """SwiGLU values (act 3: y; act 4: (da, db)) of bf16 a, b (and dy) with float32 p."""
    a = _c(a_bits, np.uint16)
    b = _c(b_bits, np.uint16)
    pp = _c(p, np.float32)
    d = None if dy_bits is None else _c(dy_bits, np.uint16)
    o0 = np.empty(a.shape, np.float32)
    o1 = np.empty(a.shape, np.float32) if act == ACT_SWIGLU_BWD else None
    lib().oracle_glu_values(act, _p(a), _p(b), _p(pp), _p(d), a.size, _p(o0), _p(o1))
    return o0 if act == ACT_SWIGLU_FWD else (o0, o1)


def act_values(act, h_bits, p, dy_bits=None):
    """The fp32 activation values (act 1: (r r) p; act 2: ((2 r) p) dy; r = max(h, 0)) of bf16
    h (and dy) with float32 p, element by element (all arrays of one shape)."""
    h = _c(h_bits, np.uint16)
    pp = _c(p, np.float32)
    d = None if dy_bits is None else _c(dy_bits, np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().oracle_act_values(act, _p(h), _p(pp), _p(d), h.size, _p(out))
    return out


def grouped_act_quantize(act, h_bits, probs, dy_bits, splits, recipe, which):
    """Scaled squared ReLU (act 1) or its gradient (act 2) in fp32 on the live rows of the bf16
    [R, C] buffer(s), or scaled SwiGLU (act 3, h [R, 2F] -> y [R, F]) and its gradient (act 4,
    h [R, 2F] and dy [R, F] -> (da | db) [R, 2F]), then the grouped quantize of those values (MX
    recipes).  probs: float32 [R] or None (p = 1).  Returns the same dict as grouped_quantize."""
    h = _c(h_bits, np.uint16)
    R, C = h.shape
    if act >= ACT_SWIGLU_FWD:
        C //= 2  # the GLU width F
    Cout = 2 * C if act == ACT_SWIGLU_BWD else C
    s = _c(splits, np.int32)
    p = None if probs is None else _c(probs, np.float32)
    d = None if dy_bits is None else _c(dy_bits, np.uint16)
    per = 2 if recipe == RECIPE_MX4 else 1
    out = {}
    row_q = row_s = col_q = col_s = None
    if which & ROWWISE:
        row_q = np.zeros((R, Cout // per), np.uint8)
        row_s = np.zeros((Cout // 32, R), np.uint8)
        out["row_q"], out["row_s"] = row_q, row_s
    if which & COLWISE:
        rows = padded_rows(s)
        col_q = np.zeros(Cout * rows // per, np.uint8)
        col_s = np.zeros(Cout * rows // 32, np.uint8)
        out["col_q"], out["col_s"] = col_q, col_s
    rc = lib().oracle_grouped_act_quantize(act, _p(h), _p(p), _p(d), R, C, _p(s), s.size, recipe, which,
                                           _p(row_q), _p(row_s), _p(col_q), _p(col_s))
    if rc != 0:
        raise ValueError(f"oracle_grouped_act_quantize failed ({rc})")
    return out


def grouped_wgrad(dy_col_q, dy_col_s, n, x_col_q, x_col_s, h, splits, R, recipe,
                  rows_sel=None, accumulate=False, mg_in=None):
    """fp64 dW[e][i][j] = sum_t dy_e[t][i] x_e[t][j] over the dequantized colwise operands.

    Returns float64 [E, len(rows_sel) or n, h].  With ``accumulate`` the result is
    ``mg_in + sum`` (mg_in float32 [E, n, h]); an empty group returns mg_in unchanged.
    """
    s = _c(splits, np.int32)
    E = s.size
    sel = None if rows_sel is None else _c(rows_sel, np.int32)
    ns = n if sel is None else sel.size
    out = np.empty((E, ns, h), np.float64)
    mg = None if mg_in is None else _c(mg_in, np.float32)
    rc = lib().oracle_grouped_wgrad(_p(_c(dy_col_q, np.uint8)), _p(np.ascontiguousarray(dy_col_s)), n,
                                    _p(_c(x_col_q, np.uint8)), _p(np.ascontiguousarray(x_col_s)), h,
                                    _p(s), E, R, recipe, _p(sel), 0 if sel is None else sel.size,
                                    1 if accumulate else 0, _p(mg), _p(out))
    if rc != 0:
        raise ValueError(f"oracle_grouped_wgrad failed ({rc})")
    return out


def grouped_fprop(x_row_q, x_row_s, w_q, w_s, N, splits, cols_sel=None, recipe=RECIPE_MX):
    """fp64 out[off_e + t][j] = sum_k x[off_e + t][k] W[e][j][k] over dequantized rowwise data.

    x_row_q uint8 [R, K], x_row_s uint8 [K/32, R], w_q uint8 [E*N, K], w_s uint8 [K/32, E*N]
    (MXFP4: the data arrays are [R, K/2] and [E*N, K/2], two codes per byte).
    Returns float64 [R, len(cols_sel) or N]; rows not in any group hold NaN.
    """
    xq = _c(x_row_q, np.uint8)
    R, K = xq.shape
    if recipe == RECIPE_MX4:
        K *= 2
    s = _c(splits, np.int32)
    sel = None if cols_sel is None else _c(cols_sel, np.int32)
    ns = N if sel is None else sel.size
    out = np.full((R, ns), np.nan, np.float64)
    rc = lib().oracle_grouped_fprop(_p(xq), _p(_c(x_row_s, np.uint8)), R, K, _p(_c(w_q, np.uint8)),
                                    _p(_c(w_s, np.uint8)), N, _p(s), s.size, recipe, _p(sel),
                                    0 if sel is None else sel.size, _p(out))
    if rc != 0:
        raise ValueError(f"oracle_grouped_fprop failed ({rc})")
    return out


def grouped_dgrad(dy_row_q, dy_row_s, w_col_q, w_col_s, k, splits, cols_sel=None, recipe=RECIPE_MX):
    """fp64 out[off_e + t][j] = sum_c dy[off_e + t][c] W[e][c][j] over the dequantized rowwise dy
    [R, n] (scales [n/32, R]) and the colwise-quantized weight (grouped_quantize of W viewed as
    [E*n, k] with splits [n] * E).  Returns float64 [R, len(cols_sel) or k]; rows not in any group
    hold NaN.  MXFP4: dy_row_q is [R, n/2] (two codes per byte)."""
    yq = _c(dy_row_q, np.uint8)
    R, n = yq.shape
    if recipe == RECIPE_MX4:
        n *= 2
    s = _c(splits, np.int32)
    sel = None if cols_sel is None else _c(cols_sel, np.int32)
    ns = k if sel is None else sel.size
    out = np.full((R, ns), np.nan, np.float64)
    rc = lib().oracle_grouped_dgrad(_p(yq), _p(_c(dy_row_s, np.uint8)), R, n, _p(_c(w_col_q, np.uint8)),
                                    _p(_c(w_col_s, np.uint8)), k, _p(s), s.size, recipe, _p(sel),
                                    0 if sel is None else sel.size, _p(out))
    if rc != 0:
        raise ValueError(f"oracle_grouped_dgrad failed ({rc})")
    return out


def wgrad_unquantized(dy_bits, x_bits, splits, R):
    """fp64 sum_t dy[off_e+t][i] x[off_e+t][j] from the bf16 values themselves (tiny inputs)."""
    dy = _c(dy_bits, np.uint16)
    x = _c(x_bits, np.uint16)
    n, h = dy.shape[1], x.shape[1]
    s = _c(splits, np.int32)
    out = np.empty((s.size, n, h), np.float64)
    rc = lib().oracle_wgrad_unquantized(_p(dy), n, _p(x), h, _p(s), s.size, R, _p(out))
    if rc != 0:
        raise ValueError(f"oracle_wgrad_unquantized failed ({rc})")
    return out

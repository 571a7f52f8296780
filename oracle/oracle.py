"""numpy front end of the C oracle (test infrastructure only).

Every array crosses as a contiguous numpy array; element values of bfloat16 /
float16 tensors are passed as float32 (an exact widening), and results of type
T come back as float32 arrays holding values exactly representable in T.
"""
import ctypes
import os

import numpy as np

from . import build as _build

F32, F16, BF16 = 0, 1, 2
DTYPE_CODES = {"f32": F32, "f16": F16, "bf16": BF16}

MUT_NONE = 0
MUT_DROP_GW = 1
MUT_DROP_GX = 2
MUT_GW_ON_SUM = 3
MUT_AMAX6_BF16 = 4
MUT_ENC_ORDER = 5
MUT_E8M0_NEAREST = 6

MX_BITS = {"mxfp4": 4, "mxfp8": 8}

_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_F = ctypes.c_float
_INT = ctypes.c_int


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        L.orc_e2m1_value.restype = ctypes.c_double
        L.orc_e2m1_value.argtypes = [ctypes.c_uint]
        L.orc_e2m1_encode.restype = ctypes.c_uint
        L.orc_e2m1_encode.argtypes = [_F]
        L.orc_e4m3_value.restype = ctypes.c_double
        L.orc_e4m3_value.argtypes = [ctypes.c_uint]
        L.orc_e4m3_encode.restype = ctypes.c_uint
        L.orc_e4m3_encode.argtypes = [_F]
        L.orc_round_ieee.restype = ctypes.c_double
        L.orc_round_ieee.argtypes = [ctypes.c_double, _INT, _INT, _INT]
        L.orc_round_to.restype = _F
        L.orc_round_to.argtypes = [_F, _INT]
        L.orc_tensor_amax.restype = _F
        L.orc_tensor_amax.argtypes = [_P, _I64]
        L.orc_quantize.restype = None
        L.orc_quantize.argtypes = [_P, _I64, _I64, _INT, _F, _P, _P]
        L.orc_dequantize.restype = None
        L.orc_dequantize.argtypes = [_P, _P, _I64, _I64, _INT, _F, _INT, _P]
        L.orc_quant_dequant.restype = None
        L.orc_quant_dequant.argtypes = [_P, _I64, _I64, _INT, _F, _INT, _P]
        L.orc_qqmm_subset.restype = None
        L.orc_qqmm_subset.argtypes = [_P, _INT, _I64, _I64, _INT, _F, _F, _P, _P, _I64,
                                      _P, _I64, _P, _I64, _P, _INT]
        L.orc_gather_qmm_subset.restype = None
        L.orc_gather_qmm_subset.argtypes = [_P, _INT, _I64, _I64, _P, _P, _P, _I64, _I64,
                                            _P, _I64, _P, _P, _I64, _P, _I64, _P, _INT]
        L.orc_gather_qmm_indexed_subset.restype = None
        L.orc_gather_qmm_indexed_subset.argtypes = [_P, _INT, _I64, _I64, _I64, _P, _P, _P, _I64, _I64,
                                                    _INT, _P, _P, _I64, _P, _I64, _P, _I64, _P, _INT]
        L.orc_moe_route.restype = _INT
        L.orc_moe_route.argtypes = [_P, _I64, _I64, _I64, _P, _P]
        L.orc_e8m0_value.restype = ctypes.c_double
        L.orc_e8m0_value.argtypes = [ctypes.c_uint]
        L.orc_e8m0_encode_up.restype = ctypes.c_uint
        L.orc_e8m0_encode_up.argtypes = [_F]
        L.orc_mx_quantize.restype = None
        L.orc_mx_quantize.argtypes = [_P, _I64, _I64, _INT, _P, _P]
        L.orc_mx_dequantize.restype = None
        L.orc_mx_dequantize.argtypes = [_P, _P, _I64, _I64, _INT, _INT, _P]
        L.orc_mx_quant_dequant.restype = None
        L.orc_mx_quant_dequant.argtypes = [_P, _I64, _I64, _INT, _INT, _P]
        L.orc_mx_qqmm_subset.restype = None
        L.orc_mx_qqmm_subset.argtypes = [_P, _INT, _I64, _I64, _INT, _P, _P, _I64, _P, _I64,
                                         _P, _I64, _P, _INT]
        L.orc_mx_gather_qmm_subset.restype = None
        L.orc_mx_gather_qmm_subset.argtypes = [_P, _INT, _I64, _INT, _P, _P, _I64, _I64, _P, _I64,
                                               _P, _P, _I64, _P, _I64, _P, _INT]
        L.orc_set_mutant.restype = None
        L.orc_set_mutant.argtypes = [_INT]
        L.orc_get_mutant.restype = _INT
        L.orc_get_mutant.argtypes = []
        _lib = L
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _dt(dtype):
    return DTYPE_CODES[dtype] if isinstance(dtype, str) else int(dtype)


def default_threads():
    return max(1, os.cpu_count() or 1)


class mutant:
    """Context manager that plants one of the oracle's test-only mistakes."""

    def __init__(self, which):
        self.which = which

    def __enter__(self):
        self.prev = lib().orc_get_mutant()
        lib().orc_set_mutant(self.which)
        return self

    def __exit__(self, *exc):
        lib().orc_set_mutant(self.prev)
        return False


# ----------------------------------------------------------------- formats

def e2m1_value(code):
    return lib().orc_e2m1_value(int(code))


def e2m1_encode(v):
    return lib().orc_e2m1_encode(float(v))


def e4m3_value(b):
    return lib().orc_e4m3_value(int(b))


def e4m3_encode(v):
    return lib().orc_e4m3_encode(float(v))


def round_ieee(v, p, emin, emax):
    return lib().orc_round_ieee(float(v), p, emin, emax)


def round_to(v, dtype):
    return lib().orc_round_to(float(v), _dt(dtype))


# ----------------------------------------------------------------- ops

def tensor_amax(x):
    x = _f32(x)
    return float(lib().orc_tensor_amax(_ptr(x), x.size))


def quantize(x, global_scale=None):
    """x [rows, k] float values -> (codes uint8 [rows, k/2], scales uint8 [rows, k/16])."""
    x = _f32(x)
    rows, k = x.shape
    assert k % 16 == 0
    codes = np.empty((rows, k // 2), np.uint8)
    scales = np.empty((rows, k // 16), np.uint8)
    has_g = global_scale is not None
    lib().orc_quantize(_ptr(x), rows, k, int(has_g), float(global_scale or 0.0),
                       _ptr(codes), _ptr(scales))
    return codes, scales


def dequantize(codes, scales, global_scale=None, dtype="bf16"):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows = codes.shape[0]
    k = codes.shape[1] * 2
    out = np.empty((rows, k), np.float32)
    has_g = global_scale is not None
    lib().orc_dequantize(_ptr(codes), _ptr(scales), rows, k, int(has_g),
                         float(global_scale or 0.0), _dt(dtype), _ptr(out))
    return out


def quant_dequant(x, global_scale=None, dtype="bf16"):
    x = _f32(x)
    rows, k = x.shape
    out = np.empty((rows, k), np.float32)
    has_g = global_scale is not None
    lib().orc_quant_dequant(_ptr(x), rows, k, int(has_g), float(global_scale or 0.0),
                            _dt(dtype), _ptr(out))
    return out


def qqmm(x, w_codes, w_scales, global_scale_x=None, global_scale_w=None, dtype="bf16",
         rows=None, cols=None, nthreads=None):
    """out[rows][:, cols] of T(x_hat @ w^T), x_hat = quant_dequant(x, g_x)."""
    x = _f32(x)
    m, k = x.shape
    w_codes = np.ascontiguousarray(w_codes, dtype=np.uint8)
    w_scales = np.ascontiguousarray(w_scales, dtype=np.uint8)
    n = w_codes.shape[0]
    assert w_codes.shape[1] * 2 == k and w_scales.shape[1] * 16 == k
    if (global_scale_x is None) != (global_scale_w is None):
        raise ValueError("both global scales or neither")
    has_g = global_scale_x is not None
    mi = np.arange(m, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, np.int64)
    ni = np.arange(n, dtype=np.int64) if cols is None else np.ascontiguousarray(cols, np.int64)
    out = np.empty((mi.size, ni.size), np.float32)
    lib().orc_qqmm_subset(_ptr(x), _dt(dtype), m, k, int(has_g),
                          float(global_scale_x or 0.0), float(global_scale_w or 0.0),
                          _ptr(w_codes), _ptr(w_scales), n, _ptr(mi), mi.size, _ptr(ni),
                          ni.size, _ptr(out), int(nthreads or default_threads()))
    return out


def gather_qmm(x, w_codes, w_scales, idx, global_scale=None, dtype="bf16", pairs=None,
               cols=None, nthreads=None):
    """Rows of out[t, j, cols] for the (t, j) pairs given (all pairs by default).

    Returns an array [len(pairs), len(cols)]; with pairs=None the result is
    reshaped to [t, top_k, len(cols)].
    """
    x = _f32(x)
    t_count, k = x.shape
    w_codes = np.ascontiguousarray(w_codes, dtype=np.uint8)
    w_scales = np.ascontiguousarray(w_scales, dtype=np.uint8)
    e_count, n = w_codes.shape[0], w_codes.shape[1]
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    top_k = idx.shape[1]
    g = None if global_scale is None else _f32(np.reshape(global_scale, (-1,)))
    if pairs is None:
        tt, jj = np.meshgrid(np.arange(t_count), np.arange(top_k), indexing="ij")
        pt, pj = tt.reshape(-1).astype(np.int64), jj.reshape(-1).astype(np.int64)
    else:
        pt = np.ascontiguousarray([p[0] for p in pairs], np.int64)
        pj = np.ascontiguousarray([p[1] for p in pairs], np.int64)
    ni = np.arange(n, dtype=np.int64) if cols is None else np.ascontiguousarray(cols, np.int64)
    out = np.empty((pt.size, ni.size), np.float32)
    lib().orc_gather_qmm_subset(_ptr(x), _dt(dtype), t_count, k, _ptr(w_codes),
                                _ptr(w_scales), None if g is None else _ptr(g), e_count, n,
                                _ptr(idx), top_k, _ptr(pt), _ptr(pj), pt.size, _ptr(ni),
                                ni.size, _ptr(out), int(nthreads or default_threads()))
    if pairs is None:
        out = out.reshape(t_count, top_k, ni.size)
    return out


def gather_qmm_indexed(x, w_codes, w_scales, rhs, lhs=None, global_scale=None, transpose=True,
                       dtype="bf16", rows=None, cols=None, nthreads=None):
    """gather_qmm in its indexed form: x [b, mr, k] (or [b, k], mr = 1),
    pair p takes x entry lhs[p] (p if lhs is None) and expert rhs[p]; returns
    out rows q = p * mr + r ([len(rhs) * mr, n], or the `rows` / `cols`
    subset).  transpose=True: w_codes [e, n, k/2] (quantized along k);
    transpose=False: w_codes [e, k, n/2] (quantized along n), out = x @ w."""
    x = _f32(x)
    if x.ndim == 2:
        x = x[:, None, :]
    b, mr, k = x.shape
    w_codes = np.ascontiguousarray(w_codes, dtype=np.uint8)
    w_scales = np.ascontiguousarray(w_scales, dtype=np.uint8)
    e_count = w_codes.shape[0]
    if transpose:
        n = w_codes.shape[1]
        assert w_codes.shape[2] * 2 == k and w_scales.shape[2] * 16 == k
    else:
        n = w_codes.shape[2] * 2
        assert w_codes.shape[1] == k and w_scales.shape[2] * 16 == n
    rhs = np.ascontiguousarray(np.reshape(rhs, (-1,)), dtype=np.int32)
    L = rhs.size
    lhs_a = None if lhs is None else np.ascontiguousarray(np.reshape(lhs, (-1,)), dtype=np.int32)
    g = None if global_scale is None else _f32(np.reshape(global_scale, (-1,)))
    qi = np.arange(L * mr, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, np.int64)
    ni = np.arange(n, dtype=np.int64) if cols is None else np.ascontiguousarray(cols, np.int64)
    out = np.empty((qi.size, ni.size), np.float32)
    lib().orc_gather_qmm_indexed_subset(_ptr(x), _dt(dtype), b, mr, k, _ptr(w_codes), _ptr(w_scales),
                                        None if g is None else _ptr(g), e_count, n, int(bool(transpose)),
                                        None if lhs_a is None else _ptr(lhs_a), _ptr(rhs), L, _ptr(qi),
                                        qi.size, _ptr(ni), ni.size, _ptr(out),
                                        int(nthreads or default_threads()))
    return out


def moe_route(idx, e_count):
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    t_count, top_k = idx.shape
    offsets = np.empty(e_count + 1, np.int32)
    perm = np.empty(t_count * top_k, np.int32)
    rc = lib().orc_moe_route(_ptr(idx), t_count, top_k, e_count, _ptr(offsets), _ptr(perm))
    if rc != 0:
        raise ValueError("expert index out of range")
    return offsets, perm


# ----------------------------------------------------------------- backward

def quantize_columnwise(x, global_scale=None):
    """Encode x [rows, cols] along its first axis: the rowwise encode of x^T,
    codes [cols, rows/2] and scales [cols, rows/16] ("mlx 0.30.7.2 -> 0.30.7.6"
    diff page 7, fp_quantize_columnwise: an M-major [M, K] tensor quantized in
    groups along K, the scale and code steps those of fp_quantize_rowwise)."""
    return quantize(np.ascontiguousarray(_f32(x).T), global_scale)


def quant_dequant_columnwise(x, global_scale=None, dtype="bf16"):
    """The round trip of x^T: [cols, rows] values of type T."""
    return quant_dequant(np.ascontiguousarray(_f32(x).T), global_scale, dtype)


def qqmm_vjp(x, w, dy, global_scale_x=None, global_scale_w=None, dtype="bf16", nthreads=None,
             dx_rows=None, dw_rows=None):
    """Gradients of y = qqmm(x, w) for the cotangent dy ("mlx 0.30.7.2 ->
    0.30.7.6" diff page 8, primitives.cpp QQMatmul::vjp):
      g_dy = float32(max |dy|) when the primal global scales are given, else none;
      dx = qqmm(dy, w^T)   with w^T [k, n] quantized along n under g_w;
      dw = qqmm(dy^T, x^T) with x^T [k, m] quantized along m under g_x;
    each qqmm round-trips its first operand under g_dy.  Returns (dx [m, k],
    dw [n, k], g_dy); with dx_rows / dw_rows, only those rows of dx / dw (the
    same values, fewer of them)."""
    x, w, dy = _f32(x), _f32(w), _f32(dy)
    if (global_scale_x is None) != (global_scale_w is None):
        raise ValueError("both global scales or neither")
    g_dy = tensor_amax(dy) if global_scale_x is not None else None
    wt_codes, wt_scales = quantize_columnwise(w, global_scale_w)   # w^T [k, n]
    dx = qqmm(dy, wt_codes, wt_scales, g_dy, global_scale_w, dtype=dtype, nthreads=nthreads,
              rows=dx_rows)
    xt_codes, xt_scales = quantize_columnwise(x, global_scale_x)   # x^T [k, m]
    dw = qqmm(np.ascontiguousarray(dy.T), xt_codes, xt_scales, g_dy, global_scale_x, dtype=dtype,
              nthreads=nthreads, rows=dw_rows)
    return dx, dw, g_dy


# ----------------------------------------------------------------- mx modes

def _bits(mode):
    if mode not in MX_BITS:
        raise ValueError(f"mx mode must be 'mxfp4' or 'mxfp8', not {mode!r}")
    return MX_BITS[mode]


def e8m0_value(b):
    return lib().orc_e8m0_value(int(b))


def e8m0_encode_up(v):
    return lib().orc_e8m0_encode_up(float(v))


def mx_code_bytes(k, mode):
    """Bytes of one quantized row of k elements."""
    return k if _bits(mode) == 8 else k // 2


def mx_quantize(x, mode):
    """x [rows, k] (k % 32 == 0) -> (codes uint8 [rows, k/2] for mxfp4 or [rows, k]
    for mxfp8, E8M0 scales uint8 [rows, k/32])."""
    bits = _bits(mode)
    x = _f32(x)
    rows, k = x.shape
    assert k % 32 == 0
    codes = np.empty((rows, mx_code_bytes(k, mode)), np.uint8)
    scales = np.empty((rows, k // 32), np.uint8)
    lib().orc_mx_quantize(_ptr(x), rows, k, bits, _ptr(codes), _ptr(scales))
    return codes, scales


def mx_dequantize(codes, scales, mode, dtype="bf16"):
    bits = _bits(mode)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows = codes.shape[0]
    k = scales.shape[1] * 32
    assert codes.shape[1] == mx_code_bytes(k, mode)
    out = np.empty((rows, k), np.float32)
    lib().orc_mx_dequantize(_ptr(codes), _ptr(scales), rows, k, bits, _dt(dtype), _ptr(out))
    return out


def mx_quant_dequant(x, mode, dtype="bf16"):
    bits = _bits(mode)
    x = _f32(x)
    rows, k = x.shape
    assert k % 32 == 0
    out = np.empty((rows, k), np.float32)
    lib().orc_mx_quant_dequant(_ptr(x), rows, k, bits, _dt(dtype), _ptr(out))
    return out


def mx_qqmm(x, w_codes, w_scales, mode, dtype="bf16", rows=None, cols=None, nthreads=None):
    """out[rows][:, cols] of T(x_hat @ w_hat^T) in an mx mode: x goes through
    its own mx encode, w is given quantized; products of the float32 decodes
    summed in double, one rounding to T."""
    bits = _bits(mode)
    x = _f32(x)
    m, k = x.shape
    w_codes = np.ascontiguousarray(w_codes, dtype=np.uint8)
    w_scales = np.ascontiguousarray(w_scales, dtype=np.uint8)
    n = w_codes.shape[0]
    assert w_codes.shape[1] == mx_code_bytes(k, mode) and w_scales.shape[1] * 32 == k
    mi = np.arange(m, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, np.int64)
    ni = np.arange(n, dtype=np.int64) if cols is None else np.ascontiguousarray(cols, np.int64)
    out = np.empty((mi.size, ni.size), np.float32)
    lib().orc_mx_qqmm_subset(_ptr(x), _dt(dtype), m, k, bits, _ptr(w_codes), _ptr(w_scales), n,
                             _ptr(mi), mi.size, _ptr(ni), ni.size, _ptr(out),
                             int(nthreads or default_threads()))
    return out


def mx_gather_qmm(x, w_codes, w_scales, idx, mode, dtype="bf16", pairs=None, cols=None,
                  nthreads=None):
    """gather_qmm in an mx mode: rows of out[t, j, cols] = T(x[t] @ w_hat[e]^T),
    e = idx[t, j], for the (t, j) pairs given (all by default); x as given,
    w_codes [e, n, row bytes] and E8M0 w_scales [e, n, k/32].  Returns
    [len(pairs), len(cols)], or [t, top_k, len(cols)] with pairs=None."""
    bits = _bits(mode)
    x = _f32(x)
    t_count, k = x.shape
    w_codes = np.ascontiguousarray(w_codes, dtype=np.uint8)
    w_scales = np.ascontiguousarray(w_scales, dtype=np.uint8)
    e_count, n = w_codes.shape[0], w_codes.shape[1]
    assert w_codes.shape[2] == mx_code_bytes(k, mode) and w_scales.shape[2] * 32 == k
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    top_k = idx.shape[1]
    if pairs is None:
        tt, jj = np.meshgrid(np.arange(t_count), np.arange(top_k), indexing="ij")
        pt, pj = tt.reshape(-1).astype(np.int64), jj.reshape(-1).astype(np.int64)
    else:
        pt = np.ascontiguousarray([p[0] for p in pairs], np.int64)
        pj = np.ascontiguousarray([p[1] for p in pairs], np.int64)
    ni = np.arange(n, dtype=np.int64) if cols is None else np.ascontiguousarray(cols, np.int64)
    out = np.empty((pt.size, ni.size), np.float32)
    lib().orc_mx_gather_qmm_subset(_ptr(x), _dt(dtype), k, bits, _ptr(w_codes), _ptr(w_scales),
                                   e_count, n, _ptr(idx), top_k, _ptr(pt), _ptr(pj), pt.size,
                                   _ptr(ni), ni.size, _ptr(out), int(nthreads or default_threads()))
    if pairs is None:
        out = out.reshape(t_count, top_k, ni.size)
    return out


__all__ = [
    "MUT_E8M0_NEAREST", "MX_BITS", "e8m0_value", "e8m0_encode_up", "mx_code_bytes",
    "mx_quantize", "mx_dequantize", "mx_quant_dequant", "mx_qqmm", "mx_gather_qmm",
    "F32", "F16", "BF16", "MUT_NONE", "MUT_DROP_GW", "MUT_DROP_GX", "MUT_GW_ON_SUM",
    "MUT_AMAX6_BF16", "MUT_ENC_ORDER", "mutant", "quantize_columnwise", "quant_dequant_columnwise",
    "qqmm_vjp", "gather_qmm_indexed", "e2m1_value", "e2m1_encode", "e4m3_value",
    "e4m3_encode", "round_ieee", "round_to", "tensor_amax", "quantize", "dequantize",
    "quant_dequant", "qqmm", "gather_qmm", "moe_route", "lib", "default_threads",
]

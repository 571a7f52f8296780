"""Python binding of libnvfp4.so: NVFP4 block-scaled quantize / dequantize /
qmv / qqmm / gather_qmm on AMD Instinct MI355X (gfx950).

This module only marshals arguments: torch supplies device memory and the
current stream, every computation runs in the HIP kernels of libnvfp4.so.
There is no CPU fallback: without the built library (or without a GPU) the
calls raise.

The functions carry the C entry points' names (see include/nvfp4.h):
    nvfp4_tensor_amax(x)                              -> float32 [1]
    nvfp4_quantize(x, global_scale=None)              -> (codes, scales)
    nvfp4_dequantize(codes, scales, global_scale=None, dtype=torch.bfloat16)
    nvfp4_quant_dequant(x, global_scale=None)         -> x_hat
    nvfp4_qmv(x, w_codes, w_scales, global_scale_x=None, global_scale_w=None)
    nvfp4_qqmm(x, w_codes, w_scales, global_scale_x=None, global_scale_w=None)
    nvfp4_qmm(x, w_codes, w_scales, global_scale_w=None)   (x not quantized)
    nvfp4_gather_qmm(x, w_codes, w_scales, expert_idx, global_scale_w=None)
    nvfp4_moe_route(expert_idx, num_experts)          -> (offsets, perm)
    nvfp4_mfma_pack(w_codes, w_scales)                -> MfmaPacked (packed copy)
    nvfp4_qqmm_packed / nvfp4_qmm_packed / nvfp4_gather_qmm_packed
                                                      (same, on the packed copy)
    nvfp4_mx_quantize / _dequantize / _quant_dequant / _pack / _qqmm / _qqmm_packed
                                                      (the mxfp4 / mxfp8 modes)
Global scales are float32 device tensors with one element (per expert: e
elements, any shape such as [e, 1, 1]), as the pages' validate_global_scale
requires ("mlx 0.30.7.2 -> 0.30.7.6" diff, page 8).
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")

NVFP4_OK, NVFP4_ERR_INVALID_ARGUMENT, NVFP4_ERR_UNSUPPORTED, NVFP4_ERR_DEVICE = 0, 1, 2, 3
_DT = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}

_lib = None


class NVFP4Error(RuntimeError):
    def __init__(self, status, message):
        super().__init__(message)
        self.status = status


def load_library():
    """Load libnvfp4.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libnvfp4.so not built at {LIB_PATH}; run nvfp4_block_scaled_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, SZ, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
    sig = {
        "nvfp4_last_error": (ctypes.c_char_p, []),
        "nvfp4_version": (I, []),
        "nvfp4_debug_set_arch_override": (None, [ctypes.c_char_p]),
        "nvfp4_tensor_amax": (I, [P, I, I64, P, P]),
        "nvfp4_quantize": (I, [P, I, I64, I64, P, P, P, P]),
        "nvfp4_dequantize": (I, [P, P, I64, I64, P, P, I, P]),
        "nvfp4_quant_dequant": (I, [P, I, I64, I64, P, P, P]),
        "nvfp4_qmv": (I, [P, I, P, P, P, P, I64, I64, P, P]),
        "nvfp4_qqmm_workspace_size": (SZ, [I64, I64, I64, I]),
        "nvfp4_qqmm": (I, [P, I, P, P, P, P, I64, I64, I64, P, P, SZ, P]),
        "nvfp4_qmm": (I, [P, I, P, P, P, I64, I64, I64, P, P]),
        "nvfp4_gather_qmm_workspace_size": (SZ, [I64, I64, I64, I64, I64]),
        "nvfp4_gather_qmm": (I, [P, I, P, P, P, P, I64, I64, I64, I64, I64, P, P, SZ, P]),
        "nvfp4_gather_qmm_noalloc": (I, [P, I, P, P, P, P, I64, I64, I64, I64, I64, P, P]),
        "nvfp4_moe_route_workspace_size": (SZ, [I64, I64, I64]),
        "nvfp4_moe_route": (I, [P, I64, I64, I64, P, P, P, SZ, P]),
        "nvfp4_mfma_pack_size": (I, [I64, I64, ctypes.POINTER(SZ), ctypes.POINTER(SZ)]),
        "nvfp4_mfma_pack": (I, [P, P, I64, I64, P, P, P]),
        "nvfp4_qqmm_packed": (I, [P, I, P, P, P, P, I64, I64, I64, P, P, SZ, P]),
        "nvfp4_qmm_packed": (I, [P, I, P, P, P, I64, I64, I64, P, P]),
        "nvfp4_gather_qmm_packed": (I, [P, I, P, P, P, P, I64, I64, I64, I64, I64, P, P, SZ, P]),
        "nvfp4_quantize_columnwise": (I, [P, I, I64, I64, P, P, P, P]),
        "nvfp4_quant_dequant_columnwise": (I, [P, I, I64, I64, P, P, P]),
        "nvfp4_qqmm_vjp_workspace_size": (SZ, [I64, I64, I64, I]),
        "nvfp4_qqmm_vjp": (I, [P, P, P, I, P, P, I64, I64, I64, P, P, P, P, SZ, P]),
        "nvfp4_gather_qmm_indexed_workspace_size": (SZ, [I64, I64, I64, I]),
        "nvfp4_gather_qmm_indexed": (I, [P, I, I64, I64, P, P, P, P, P, I64, I64, I64, I64, I, I, P, P,
                                         SZ, P]),
        "nvfp4_mx_quantize": (I, [P, I, I, I64, I64, P, P, P]),
        "nvfp4_mx_dequantize": (I, [P, P, I, I64, I64, P, I, P]),
        "nvfp4_mx_quant_dequant": (I, [P, I, I, I64, I64, P, P]),
        "nvfp4_mx_pack_size": (I, [I, I64, I64, ctypes.POINTER(SZ), ctypes.POINTER(SZ)]),
        "nvfp4_mx_pack": (I, [P, P, I, I64, I64, P, P, P]),
        "nvfp4_mx_quantize_packed": (I, [P, I, I, I64, I64, P, P, P]),
        "nvfp4_mx_mm_packed": (I, [P, P, P, P, I, I64, I64, I64, P, I, P]),
        "nvfp4_mx_qqmm_workspace_size": (SZ, [I, I64, I64, I64, I]),
        "nvfp4_mx_qqmm": (I, [P, I, I, P, P, I64, I64, I64, P, P, SZ, P]),
        "nvfp4_mx_qqmm_packed": (I, [P, I, I, P, P, I64, I64, I64, P, P, SZ, P]),
        "nvfp4_mx_gather_qmm": (I, [P, I, I, P, P, P, I64, I64, I64, I64, I64, P, P, SZ, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(status):
    if status != NVFP4_OK:
        msg = load_library().nvfp4_last_error().decode()
        if status == NVFP4_ERR_INVALID_ARGUMENT:
            raise ValueError(msg)
        raise NVFP4Error(status, msg)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _dtype_code(t, name):
    if t.dtype not in _DT:
        raise ValueError(f"{name}: unsupported dtype {t.dtype} (float32, float16, bfloat16 only)")
    return _DT[t.dtype]


def _gscale(g, name, numel=1):
    """Device float32 global scale with `numel` elements, or None."""
    if g is None:
        return None
    if not isinstance(g, torch.Tensor):
        raise ValueError(f"{name} must be a float32 device tensor")
    if g.numel() != numel:
        raise ValueError(f"{name} must have {numel} element(s) but got shape {tuple(g.shape)}.")
    if g.dtype != torch.float32:
        raise ValueError(f"{name} must have dtype float32 but got {g.dtype}.")
    return _dev(g, name)


def _rows_k(x):
    if x.dim() == 0:
        raise ValueError("input must have at least one dimension")
    k = x.shape[-1]
    return x.numel() // k if k else 0, k


# ------------------------------------------------------------------ codec

def nvfp4_tensor_amax(x, out=None):
    L = load_library()
    _dev(x, "x")
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=x.device)
    _check(L.nvfp4_tensor_amax(_ptr(x), _dtype_code(x, "x"), x.numel(), _ptr(out), _stream()))
    return out


def nvfp4_quantize(x, global_scale=None, codes=None, scales=None):
    L = load_library()
    _dev(x, "x")
    rows, k = _rows_k(x)
    g = _gscale(global_scale, "global_scale")
    shape = tuple(x.shape[:-1])
    if codes is None:
        codes = torch.empty(shape + (k // 2,), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(shape + (k // 16,), dtype=torch.uint8, device=x.device)
    _check(L.nvfp4_quantize(_ptr(x), _dtype_code(x, "x"), rows, k, _ptr(g), _ptr(codes),
                            _ptr(scales), _stream()))
    return codes, scales


def nvfp4_dequantize(codes, scales, global_scale=None, dtype=torch.bfloat16, out=None):
    L = load_library()
    _dev(codes, "codes")
    _dev(scales, "scales")
    if codes.dtype != torch.uint8 or scales.dtype != torch.uint8:
        raise ValueError("codes and scales must be uint8")
    k = codes.shape[-1] * 2
    rows = codes.numel() // codes.shape[-1] if codes.shape[-1] else 0
    if scales.numel() * 16 != rows * k:
        raise ValueError("scales do not match codes")
    g = _gscale(global_scale, "global_scale")
    if out is None:
        out = torch.empty(tuple(codes.shape[:-1]) + (k,), dtype=dtype, device=codes.device)
    _check(L.nvfp4_dequantize(_ptr(codes), _ptr(scales), rows, k, _ptr(g), _ptr(out),
                              _dtype_code(out, "out"), _stream()))
    return out


def nvfp4_quant_dequant(x, global_scale=None, out=None):
    L = load_library()
    _dev(x, "x")
    rows, k = _rows_k(x)
    g = _gscale(global_scale, "global_scale")
    if out is None:
        out = torch.empty_like(x)
    _check(L.nvfp4_quant_dequant(_ptr(x), _dtype_code(x, "x"), rows, k, _ptr(g), _ptr(out),
                                 _stream()))
    return out


# ------------------------------------------------------------------ backward

def _rows_cols(x):
    if x.dim() != 2:
        raise ValueError("x must be 2-D [rows, cols]")
    return x.shape[0], x.shape[1]


def nvfp4_quantize_columnwise(x, global_scale=None, codes=None, scales=None):
    """Quantize x [rows, cols] along its first axis (the encode of x^T):
    codes [cols, rows/2], scales [cols, rows/16]."""
    L = load_library()
    _dev(x, "x")
    rows, cols = _rows_cols(x)
    g = _gscale(global_scale, "global_scale")
    if codes is None:
        codes = torch.empty(cols, rows // 2, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(cols, rows // 16, dtype=torch.uint8, device=x.device)
    _check(L.nvfp4_quantize_columnwise(_ptr(x), _dtype_code(x, "x"), rows, cols, _ptr(g),
                                       _ptr(codes), _ptr(scales), _stream()))
    return codes, scales


def nvfp4_quant_dequant_columnwise(x, global_scale=None, out=None):
    """The NVFP4 round trip of x^T: [cols, rows] of x's dtype."""
    L = load_library()
    _dev(x, "x")
    rows, cols = _rows_cols(x)
    g = _gscale(global_scale, "global_scale")
    if out is None:
        out = torch.empty(cols, rows, dtype=x.dtype, device=x.device)
    _check(L.nvfp4_quant_dequant_columnwise(_ptr(x), _dtype_code(x, "x"), rows, cols, _ptr(g),
                                            _ptr(out), _stream()))
    return out


def nvfp4_qqmm_vjp(x, w, dy, global_scale_x=None, global_scale_w=None, want_dx=True,
                   want_dw=True, workspace=None):
    """Gradients of y = nvfp4_qqmm(x, w) for the cotangent dy [m, n]:
    returns (dx [m, k] or None, dw [n, k] or None, g_dy (device float, or
    None without global scales))."""
    L = load_library()
    for t, name in ((x, "x"), (w, "w"), (dy, "dy")):
        _dev(t, name)
    m, k = _rows_cols(x)
    n = w.shape[0]
    if w.shape != (n, k) or dy.shape != (m, n):
        raise ValueError(f"[qqmm_vjp] shapes x {tuple(x.shape)}, w {tuple(w.shape)}, dy {tuple(dy.shape)}")
    if not (x.dtype == w.dtype == dy.dtype):
        raise ValueError("[qqmm_vjp] x, w and dy must share one dtype")
    gx, gw = _gscale(global_scale_x, "global_scale_x"), _gscale(global_scale_w, "global_scale_w")
    dt = _dtype_code(x, "x")
    dx = torch.empty(m, k, dtype=x.dtype, device=x.device) if want_dx else None
    dw = torch.empty(n, k, dtype=x.dtype, device=x.device) if want_dw else None
    gdy = torch.empty(1, dtype=torch.float32, device=x.device) if gx is not None else None
    if workspace is None:
        nbytes = L.nvfp4_qqmm_vjp_workspace_size(m, n, k, dt)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    else:
        nbytes = workspace.numel() * workspace.element_size()
    _check(L.nvfp4_qqmm_vjp(_ptr(x), _ptr(w), _ptr(dy), dt, _ptr(gx), _ptr(gw), m, n, k,
                            _ptr(dx), _ptr(dw), _ptr(gdy), _ptr(workspace), nbytes, _stream()))
    return dx, dw, gdy


# ------------------------------------------------------------------ contractions

def _w_shapes(w_codes, w_scales, k):
    _dev(w_codes, "w_codes")
    _dev(w_scales, "w_scales")
    if w_codes.dtype != torch.uint8 or w_scales.dtype != torch.uint8:
        raise ValueError("w_codes and w_scales must be uint8")
    if w_codes.shape[-1] * 2 != k or w_scales.shape[-1] * 16 != k:
        raise ValueError(f"weights of inner size {w_codes.shape[-1] * 2} do not match x's {k}")


def nvfp4_qmv(x, w_codes, w_scales, global_scale_x=None, global_scale_w=None, out=None):
    L = load_library()
    _dev(x, "x")
    k = x.shape[-1]
    if x.numel() != k:
        raise ValueError("qmv takes a single row x")
    _w_shapes(w_codes, w_scales, k)
    n = w_codes.shape[0]
    gx, gw = _gscale(global_scale_x, "global_scale_x"), _gscale(global_scale_w, "global_scale_w")
    if out is None:
        out = torch.empty(tuple(x.shape[:-1]) + (n,), dtype=x.dtype, device=x.device)
    _check(L.nvfp4_qmv(_ptr(x), _dtype_code(x, "x"), _ptr(gx), _ptr(w_codes), _ptr(w_scales),
                       _ptr(gw), n, k, _ptr(out), _stream()))
    return out


def qqmm_workspace(m, n, k, dtype, device):
    nbytes = load_library().nvfp4_qqmm_workspace_size(m, n, k, _DT[dtype])
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device), nbytes


def nvfp4_qqmm(x, w_codes, w_scales, global_scale_x=None, global_scale_w=None, out=None,
               workspace=None):
    """out = x_hat @ w^T with x [m, k] (at most 2-D, as the pages' qqmm)."""
    L = load_library()
    _dev(x, "x")
    if x.dim() > 2 or w_codes.dim() > 2:
        raise ValueError("[qqmm] Only 2D inputs are supported.")
    x2 = x.reshape(-1, x.shape[-1])
    m, k = x2.shape
    _w_shapes(w_codes, w_scales, k)
    n = w_codes.shape[0]
    gx, gw = _gscale(global_scale_x, "global_scale_x"), _gscale(global_scale_w, "global_scale_w")
    if out is None:
        out = torch.empty(tuple(x.shape[:-1]) + (n,), dtype=x.dtype, device=x.device)
    if workspace is None:
        workspace, nbytes = qqmm_workspace(m, n, k, x.dtype, x.device)
    else:
        nbytes = workspace.numel() * workspace.element_size()
    _check(L.nvfp4_qqmm(_ptr(x2), _dtype_code(x, "x"), _ptr(gx), _ptr(w_codes), _ptr(w_scales),
                        _ptr(gw), m, n, k, _ptr(out), _ptr(workspace), nbytes, _stream()))
    return out


def nvfp4_qmm(x, w_codes, w_scales, global_scale_w=None, out=None):
    """out = x @ dequant(w)^T with x used as given (the pages' quantized_matmul)."""
    L = load_library()
    _dev(x, "x")
    x2 = x.reshape(-1, x.shape[-1])
    m, k = x2.shape
    _w_shapes(w_codes, w_scales, k)
    n = w_codes.shape[0]
    gw = _gscale(global_scale_w, "global_scale_w")
    if out is None:
        out = torch.empty(tuple(x.shape[:-1]) + (n,), dtype=x.dtype, device=x.device)
    _check(L.nvfp4_qmm(_ptr(x2), _dtype_code(x, "x"), _ptr(w_codes), _ptr(w_scales), _ptr(gw),
                       m, n, k, _ptr(out), _stream()))
    return out


def gather_workspace(t, top_k, e, n, k, device):
    nbytes = load_library().nvfp4_gather_qmm_workspace_size(t, top_k, e, n, k)
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device), nbytes


def nvfp4_gather_qmm(x, w_codes, w_scales, expert_idx, global_scale_w=None, out=None,
                     workspace=None):
    """out[t, j, :] = x[t] @ dequant(w[expert_idx[t, j]])^T with per-expert g."""
    L = load_library()
    _dev(x, "x")
    _dev(expert_idx, "expert_idx")
    if expert_idx.dtype != torch.int32 or expert_idx.dim() != 2:
        raise ValueError("expert_idx must be int32 [t, top_k]")
    t, k = x.shape
    top_k = expert_idx.shape[1]
    if expert_idx.shape[0] != t:
        raise ValueError("expert_idx rows must match x rows")
    _w_shapes(w_codes, w_scales, k)
    e, n = w_codes.shape[0], w_codes.shape[1]
    g = _gscale(global_scale_w, "global_scale_w", numel=e)
    if out is None:
        out = torch.empty((t, top_k, n), dtype=x.dtype, device=x.device)
    if workspace is None:
        workspace, nbytes = gather_workspace(t, top_k, e, n, k, x.device)
    else:
        nbytes = workspace.numel() * workspace.element_size()
    _check(L.nvfp4_gather_qmm(_ptr(x), _dtype_code(x, "x"), _ptr(w_codes), _ptr(w_scales), _ptr(g),
                              _ptr(expert_idx), t, top_k, e, n, k, _ptr(out), _ptr(workspace),
                              nbytes, _stream()))
    return out


def nvfp4_gather_qmm_noalloc(x, w_codes, w_scales, expert_idx, global_scale_w=None, out=None):
    """nvfp4_gather_qmm without a workspace: the routing tables live in the
    library's fixed device scratch (overlapping calls on one GPU race)."""
    L = load_library()
    _dev(x, "x")
    _dev(expert_idx, "expert_idx")
    if expert_idx.dtype != torch.int32 or expert_idx.dim() != 2:
        raise ValueError("expert_idx must be int32 [t, top_k]")
    t, k = x.shape
    top_k = expert_idx.shape[1]
    if expert_idx.shape[0] != t:
        raise ValueError("expert_idx rows must match x rows")
    _w_shapes(w_codes, w_scales, k)
    e, n = w_codes.shape[0], w_codes.shape[1]
    g = _gscale(global_scale_w, "global_scale_w", numel=e)
    if out is None:
        out = torch.empty((t, top_k, n), dtype=x.dtype, device=x.device)
    _check(L.nvfp4_gather_qmm_noalloc(_ptr(x), _dtype_code(x, "x"), _ptr(w_codes), _ptr(w_scales),
                                      _ptr(g), _ptr(expert_idx), t, top_k, e, n, k, _ptr(out),
                                      _stream()))
    return out


def nvfp4_gather_qmm_indexed(x, w_codes, w_scales, rhs_indices, lhs_indices=None,
                             global_scale_w=None, transpose=True, sorted_indices=False, out=None,
                             workspace=None):
    """Indexed gather_qmm: x [entries, rows_per_entry, k] (or [entries, k]);
    pair p multiplies x entry lhs_indices[p] (p without lhs_indices) by expert
    rhs_indices[p]; out [pairs, rows_per_entry, n] (or [pairs, n]).
    transpose=True: w_codes [e, n, k/2] (x @ w^T); transpose=False: w_codes
    [e, k, n/2] quantized along n (x @ w)."""
    L = load_library()
    _dev(x, "x")
    _dev(w_codes, "w_codes")
    _dev(w_scales, "w_scales")
    _dev(rhs_indices, "rhs_indices")
    if x.dim() not in (2, 3) or w_codes.dim() != 3:
        raise ValueError("x must be [entries, k] or [entries, rows, k] and w_codes [e, ., .]")
    entries, mr, k = (x.shape[0], 1, x.shape[1]) if x.dim() == 2 else tuple(x.shape)
    e = w_codes.shape[0]
    if transpose:
        n = w_codes.shape[1]
        if w_codes.shape[2] * 2 != k or tuple(w_scales.shape) != (e, n, k // 16):
            raise ValueError("w_codes / w_scales do not match x's inner size (transpose=True)")
    else:
        n = w_codes.shape[2] * 2
        if w_codes.shape[1] != k or tuple(w_scales.shape) != (e, k, n // 16):
            raise ValueError("w_codes / w_scales do not match x's inner size (transpose=False)")
    if rhs_indices.dtype != torch.int32:
        raise ValueError("rhs_indices must be int32")
    pairs = rhs_indices.numel()
    if lhs_indices is not None:
        _dev(lhs_indices, "lhs_indices")
        if lhs_indices.dtype != torch.int32 or lhs_indices.numel() != pairs:
            raise ValueError("lhs_indices must be int32 with one entry per pair")
    g = _gscale(global_scale_w, "global_scale", numel=e)
    if out is None:
        shape = (pairs, n) if x.dim() == 2 else (pairs, mr, n)
        out = torch.empty(shape, dtype=x.dtype, device=x.device)
    if workspace is None:
        nbytes = L.nvfp4_gather_qmm_indexed_workspace_size(pairs, mr, e, int(lhs_indices is not None))
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    nbytes = workspace.numel() * workspace.element_size()
    _check(L.nvfp4_gather_qmm_indexed(_ptr(x), _dtype_code(x, "x"), entries, mr, _ptr(w_codes),
                                      _ptr(w_scales), _ptr(g), _ptr(lhs_indices), _ptr(rhs_indices), pairs,
                                      e, n, k, int(bool(transpose)), int(bool(sorted_indices)), _ptr(out),
                                      _ptr(workspace), nbytes, _stream()))
    return out


def nvfp4_moe_route(expert_idx, num_experts):
    L = load_library()
    _dev(expert_idx, "expert_idx")
    t, top_k = expert_idx.shape
    offsets = torch.empty(num_experts + 1, dtype=torch.int32, device=expert_idx.device)
    perm = torch.empty(t * top_k, dtype=torch.int32, device=expert_idx.device)
    nbytes = L.nvfp4_moe_route_workspace_size(t, top_k, num_experts)
    workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=expert_idx.device)
    _check(L.nvfp4_moe_route(_ptr(expert_idx), t, top_k, num_experts, _ptr(offsets), _ptr(perm),
                             _ptr(workspace), nbytes, _stream()))
    return offsets, perm


# ------------------------------------------------------------------ packed weights

class MfmaPacked:
    """The packed copy of an NVFP4 weight ([rows, k] or stacked experts
    [e, n, k]) for the matrix-core contractions: codes and scales as flat uint8
    device tensors in the order include/nvfp4.h describes."""

    def __init__(self, codes, scales, shape):
        self.codes, self.scales, self.shape = codes, scales, tuple(shape)

    @property
    def k(self):
        return self.shape[-1]


def nvfp4_mfma_pack(w_codes, w_scales):
    L = load_library()
    _dev(w_codes, "w_codes")
    _dev(w_scales, "w_scales")
    k = w_codes.shape[-1] * 2
    if w_scales.shape[-1] * 16 != k or w_codes.shape[:-1] != w_scales.shape[:-1]:
        raise ValueError("w_codes and w_scales describe different shapes")
    rows = w_codes.numel() // w_codes.shape[-1]
    cb, sb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(L.nvfp4_mfma_pack_size(rows, k, ctypes.byref(cb), ctypes.byref(sb)))
    pc = torch.empty(cb.value, dtype=torch.uint8, device=w_codes.device)
    ps = torch.empty(sb.value, dtype=torch.uint8, device=w_codes.device)
    _check(L.nvfp4_mfma_pack(_ptr(w_codes), _ptr(w_scales), rows, k, _ptr(pc), _ptr(ps), _stream()))
    return MfmaPacked(pc, ps, tuple(w_codes.shape[:-1]) + (k,))


def nvfp4_qqmm_packed(x, w, global_scale_x=None, global_scale_w=None, out=None, workspace=None):
    """nvfp4_qqmm with w an MfmaPacked [n, k]."""
    L = load_library()
    _dev(x, "x")
    if x.dim() > 2 or len(w.shape) != 2:
        raise ValueError("[qqmm] Only 2D inputs are supported.")
    x2 = x.reshape(-1, x.shape[-1])
    m, k = x2.shape
    n = w.shape[0]
    if w.k != k:
        raise ValueError(f"weights of inner size {w.k} do not match x's {k}")
    gx, gw = _gscale(global_scale_x, "global_scale_x"), _gscale(global_scale_w, "global_scale_w")
    if out is None:
        out = torch.empty(tuple(x.shape[:-1]) + (n,), dtype=x.dtype, device=x.device)
    if workspace is None:
        workspace, nbytes = qqmm_workspace(max(m, 2), n, k, x.dtype, x.device)
    else:
        nbytes = workspace.numel() * workspace.element_size()
    _check(L.nvfp4_qqmm_packed(_ptr(x2), _dtype_code(x, "x"), _ptr(gx), _ptr(w.codes), _ptr(w.scales),
                               _ptr(gw), m, n, k, _ptr(out), _ptr(workspace), nbytes, _stream()))
    return out


def nvfp4_qmm_packed(x, w, global_scale_w=None, out=None):
    """nvfp4_qmm with w an MfmaPacked [n, k]."""
    L = load_library()
    _dev(x, "x")
    x2 = x.reshape(-1, x.shape[-1])
    m, k = x2.shape
    n = w.shape[0]
    if len(w.shape) != 2 or w.k != k:
        raise ValueError("weights must be a packed [n, k] with x's k")
    gw = _gscale(global_scale_w, "global_scale_w")
    if out is None:
        out = torch.empty(tuple(x.shape[:-1]) + (n,), dtype=x.dtype, device=x.device)
    _check(L.nvfp4_qmm_packed(_ptr(x2), _dtype_code(x, "x"), _ptr(w.codes), _ptr(w.scales), _ptr(gw),
                              m, n, k, _ptr(out), _stream()))
    return out


def nvfp4_gather_qmm_packed(x, w, expert_idx, global_scale_w=None, out=None, workspace=None):
    """nvfp4_gather_qmm with w an MfmaPacked of stacked experts [e, n, k]."""
    L = load_library()
    _dev(x, "x")
    _dev(expert_idx, "expert_idx")
    if expert_idx.dtype != torch.int32 or expert_idx.dim() != 2:
        raise ValueError("expert_idx must be int32 [t, top_k]")
    t, k = x.shape
    top_k = expert_idx.shape[1]
    if len(w.shape) != 3 or w.k != k:
        raise ValueError("weights must be a packed [e, n, k] with x's k")
    e, n = w.shape[0], w.shape[1]
    g = _gscale(global_scale_w, "global_scale_w", numel=e)
    if out is None:
        out = torch.empty((t, top_k, n), dtype=x.dtype, device=x.device)
    if workspace is None:
        workspace, nbytes = gather_workspace(t, top_k, e, n, k, x.device)
    else:
        nbytes = workspace.numel() * workspace.element_size()
    _check(L.nvfp4_gather_qmm_packed(_ptr(x), _dtype_code(x, "x"), _ptr(w.codes), _ptr(w.scales), _ptr(g),
                                     _ptr(expert_idx), t, top_k, e, n, k, _ptr(out), _ptr(workspace),
                                     nbytes, _stream()))
    return out


# ------------------------------------------------------------------ mx modes

MX_MODES = {"mxfp4": 4, "mxfp8": 8}


def _mx_mode(mode):
    if mode not in MX_MODES:
        raise ValueError(f"mx mode must be 'mxfp4' or 'mxfp8', not {mode!r}")
    return MX_MODES[mode]


def _mx_code_cols(k, mode):
    return k if MX_MODES[mode] == 8 else k // 2


def nvfp4_mx_quantize(x, mode, codes=None, scales=None):
    """(codes uint8 [..., k/2] (mxfp4) or [..., k] (mxfp8), E8M0 scales uint8 [..., k/32])."""
    L = load_library()
    bits = _mx_mode(mode)
    _dev(x, "x")
    rows, k = _rows_k(x)
    if codes is None:
        codes = torch.empty(tuple(x.shape[:-1]) + (_mx_code_cols(k, mode),), dtype=torch.uint8,
                            device=x.device)
    if scales is None:
        scales = torch.empty(tuple(x.shape[:-1]) + (k // 32,), dtype=torch.uint8, device=x.device)
    _check(L.nvfp4_mx_quantize(_ptr(x), _dtype_code(x, "x"), bits, rows, k, _ptr(codes), _ptr(scales),
                               _stream()))
    return codes, scales


def nvfp4_mx_dequantize(codes, scales, mode, dtype=torch.bfloat16, out=None):
    L = load_library()
    bits = _mx_mode(mode)
    _dev(codes, "codes")
    _dev(scales, "scales")
    k = scales.shape[-1] * 32
    if codes.shape[-1] != _mx_code_cols(k, mode) or codes.shape[:-1] != scales.shape[:-1]:
        raise ValueError("codes and scales describe different shapes")
    rows = scales.numel() // scales.shape[-1] if scales.shape[-1] else 0
    if out is None:
        out = torch.empty(tuple(codes.shape[:-1]) + (k,), dtype=dtype, device=codes.device)
    _check(L.nvfp4_mx_dequantize(_ptr(codes), _ptr(scales), bits, rows, k, _ptr(out),
                                 _dtype_code(out, "out"), _stream()))
    return out


def nvfp4_mx_quant_dequant(x, mode, out=None):
    L = load_library()
    bits = _mx_mode(mode)
    _dev(x, "x")
    rows, k = _rows_k(x)
    if out is None:
        out = torch.empty_like(x)
    _check(L.nvfp4_mx_quant_dequant(_ptr(x), _dtype_code(x, "x"), bits, rows, k, _ptr(out), _stream()))
    return out


class MxPacked:
    """The packed copy of an mx weight [rows, k] for the block-scaled
    matrix-core product: flat uint8 device tensors in the order include/nvfp4.h
    describes."""

    def __init__(self, codes, scales, shape, mode):
        self.codes, self.scales, self.shape, self.mode = codes, scales, tuple(shape), mode

    @property
    def k(self):
        return self.shape[-1]


def nvfp4_mx_pack(w_codes, w_scales, mode):
    L = load_library()
    bits = _mx_mode(mode)
    _dev(w_codes, "w_codes")
    _dev(w_scales, "w_scales")
    k = w_scales.shape[-1] * 32
    if w_codes.shape[-1] != _mx_code_cols(k, mode) or w_codes.shape[:-1] != w_scales.shape[:-1]:
        raise ValueError("w_codes and w_scales describe different shapes")
    rows = w_scales.numel() // w_scales.shape[-1]
    cb, sb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(L.nvfp4_mx_pack_size(bits, rows, k, ctypes.byref(cb), ctypes.byref(sb)))
    pc = torch.empty(cb.value, dtype=torch.uint8, device=w_codes.device)
    ps = torch.empty(sb.value, dtype=torch.uint8, device=w_codes.device)
    _check(L.nvfp4_mx_pack(_ptr(w_codes), _ptr(w_scales), bits, rows, k, _ptr(pc), _ptr(ps),
                           _stream()))
    return MxPacked(pc, ps, tuple(w_codes.shape[:-1]) + (k,), mode)


def nvfp4_mx_quantize_packed(x, mode, out=None):
    """x [rows, k] quantized in an mx mode straight into the packed layout
    (into `out`, an MxPacked of the same shape and mode, when given)."""
    L = load_library()
    bits = _mx_mode(mode)
    _dev(x, "x")
    rows, k = _rows_k(x)
    if out is None:
        cb, sb = ctypes.c_size_t(0), ctypes.c_size_t(0)
        _check(L.nvfp4_mx_pack_size(bits, rows, k, ctypes.byref(cb), ctypes.byref(sb)))
        out = MxPacked(torch.empty(cb.value, dtype=torch.uint8, device=x.device),
                       torch.empty(sb.value, dtype=torch.uint8, device=x.device), (rows, k), mode)
    elif out.mode != mode or out.shape != (rows, k):
        raise ValueError("out has another mode or shape")
    _check(L.nvfp4_mx_quantize_packed(_ptr(x), _dtype_code(x, "x"), bits, rows, k, _ptr(out.codes),
                                      _ptr(out.scales), _stream()))
    return out


def nvfp4_mx_mm_packed(x, w, dtype=torch.bfloat16, out=None):
    """out [m, n] = x_hat @ w_hat^T for two MxPacked operands of one mode."""
    L = load_library()
    if x.mode != w.mode or x.k != w.k:
        raise ValueError("the packed operands differ in mode or inner size")
    m, n, k = x.shape[0], w.shape[0], x.k
    if out is None:
        out = torch.empty(m, n, dtype=dtype, device=x.codes.device)
    _check(L.nvfp4_mx_mm_packed(_ptr(x.codes), _ptr(x.scales), _ptr(w.codes), _ptr(w.scales),
                                _mx_mode(x.mode), m, n, k, _ptr(out), _dtype_code(out, "out"),
                                _stream()))
    return out


def mx_qqmm_workspace(mode, m, n, k, packed_w, device):
    nbytes = load_library().nvfp4_mx_qqmm_workspace_size(_mx_mode(mode), m, n, k, int(bool(packed_w)))
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device), nbytes


def nvfp4_mx_qqmm(x, w_codes, w_scales, mode, out=None, workspace=None):
    """out [m, n] = x_hat @ w_hat^T in an mx mode (x quantized in the kernel
    path; w given quantized, row-major)."""
    L = load_library()
    bits = _mx_mode(mode)
    _dev(x, "x")
    _dev(w_codes, "w_codes")
    _dev(w_scales, "w_scales")
    if x.dim() > 2 or w_codes.dim() != 2:
        raise ValueError("[qqmm] Only 2D inputs are supported.")
    m, k = x.shape if x.dim() == 2 else (1, x.shape[0])
    n = w_codes.shape[0]
    if w_scales.shape != (n, k // 32) or w_codes.shape[1] != _mx_code_cols(k, mode):
        raise ValueError("w_codes / w_scales do not match x's inner size")
    if out is None:
        out = torch.empty(tuple(x.shape[:-1]) + (n,), dtype=x.dtype, device=x.device)
    if workspace is None:
        workspace, nbytes = mx_qqmm_workspace(mode, m, n, k, False, x.device)
    else:
        nbytes = workspace.numel() * workspace.element_size()
    _check(L.nvfp4_mx_qqmm(_ptr(x), _dtype_code(x, "x"), bits, _ptr(w_codes), _ptr(w_scales), m, n, k,
                           _ptr(out), _ptr(workspace), nbytes, _stream()))
    return out


def nvfp4_mx_qqmm_packed(x, w, out=None, workspace=None):
    """nvfp4_mx_qqmm with w an MxPacked [n, k]."""
    L = load_library()
    bits = _mx_mode(w.mode)
    _dev(x, "x")
    if x.dim() > 2 or len(w.shape) != 2:
        raise ValueError("[qqmm] Only 2D inputs are supported.")
    m, k = x.shape if x.dim() == 2 else (1, x.shape[0])
    n = w.shape[0]
    if w.k != k:
        raise ValueError(f"weights of inner size {w.k} do not match x's {k}")
    if out is None:
        out = torch.empty(tuple(x.shape[:-1]) + (n,), dtype=x.dtype, device=x.device)
    if workspace is None:
        workspace, nbytes = mx_qqmm_workspace(w.mode, m, n, k, True, x.device)
    else:
        nbytes = workspace.numel() * workspace.element_size()
    _check(L.nvfp4_mx_qqmm_packed(_ptr(x), _dtype_code(x, "x"), bits, _ptr(w.codes), _ptr(w.scales), m,
                                  n, k, _ptr(out), _ptr(workspace), nbytes, _stream()))
    return out


# ------------------------------------------------------------------ MLX-style names

def _mode_check(group_size, bits, mode, global_scales=()):
    """The pages' mode table: nvfp4 = group 16, bits 4; mxfp4 = 32, 4; mxfp8 =
    32, 8; global scales only with nvfp4 ("mlx 0.30.7.2 -> 0.30.7.6" diff page
    8, fp_quantize and validate_global_scale)."""
    want = {"nvfp4": (16, 4), "mxfp4": (32, 4), "mxfp8": (32, 8)}
    if mode not in want:
        raise ValueError(f"[quantize] unsupported mode {mode!r} (nvfp4, mxfp4, mxfp8)")
    gs, b = want[mode]
    if group_size not in (None, gs) or bits not in (None, b):
        raise ValueError(f"[quantize] mode {mode!r} needs group_size={gs} and bits={b}")
    if mode != "nvfp4" and any(g is not None for g in global_scales):
        raise ValueError("[quantize] Global scale is only supported for 'nvfp4' quantization mode.")


def quantize(w, group_size=None, bits=None, mode="nvfp4", global_scale=None):
    _mode_check(group_size, bits, mode, (global_scale,))
    if mode != "nvfp4":
        return nvfp4_mx_quantize(w, mode)
    return nvfp4_quantize(w, global_scale)


def dequantize(w, scales, group_size=None, bits=None, mode="nvfp4", global_scale=None,
               dtype=torch.bfloat16):
    _mode_check(group_size, bits, mode, (global_scale,))
    if mode != "nvfp4":
        return nvfp4_mx_dequantize(w, scales, mode, dtype)
    return nvfp4_dequantize(w, scales, global_scale, dtype)


def nvfp4_mx_gather_qmm(x, w_codes, w_scales, expert_idx, mode, out=None, workspace=None):
    """out[t, j, :] = x[t] @ w_hat[expert_idx[t, j]]^T with mx weights
    (codes [e, n, k/2] for mxfp4 or [e, n, k] for mxfp8, scales [e, n, k/32])."""
    L = load_library()
    bits = _mx_mode(mode)
    _dev(x, "x")
    _dev(expert_idx, "expert_idx")
    _dev(w_codes, "w_codes")
    _dev(w_scales, "w_scales")
    if expert_idx.dtype != torch.int32 or expert_idx.dim() != 2:
        raise ValueError("expert_idx must be int32 [t, top_k]")
    if x.dim() != 2:
        raise ValueError("x must be [t, k]")
    t, k = x.shape
    top_k = expert_idx.shape[1]
    if expert_idx.shape[0] != t:
        raise ValueError("expert_idx rows must match x rows")
    if w_codes.dtype != torch.uint8 or w_scales.dtype != torch.uint8 or w_codes.dim() != 3:
        raise ValueError("w_codes and w_scales must be uint8 [e, n, .]")
    e, n = w_codes.shape[0], w_codes.shape[1]
    if w_codes.shape[2] != _mx_code_cols(k, mode) or tuple(w_scales.shape) != (e, n, k // 32):
        raise ValueError("w_codes / w_scales do not match x's inner size")
    if out is None:
        out = torch.empty((t, top_k, n), dtype=x.dtype, device=x.device)
    if workspace is None:
        workspace, nbytes = gather_workspace(t, top_k, e, n, k, x.device)
    else:
        nbytes = workspace.numel() * workspace.element_size()
    _check(L.nvfp4_mx_gather_qmm(_ptr(x), _dtype_code(x, "x"), bits, _ptr(w_codes), _ptr(w_scales),
                                 _ptr(expert_idx), t, top_k, e, n, k, _ptr(out), _ptr(workspace),
                                 nbytes, _stream()))
    return out


def qqmm(x, w, scales, group_size=None, bits=None, mode="nvfp4", global_scale_x=None,
         global_scale_w=None):
    _mode_check(group_size, bits, mode, (global_scale_x, global_scale_w))
    if mode != "nvfp4":
        return nvfp4_mx_qqmm(x, w, scales, mode)
    return nvfp4_qqmm(x, w, scales, global_scale_x, global_scale_w)


def gather_qmm(x, w, scales, rhs_indices, global_scale=None, lhs_indices=None, transpose=True,
               sorted_indices=False, group_size=None, bits=None, mode="nvfp4"):
    """The MoE form (x [t, k], rhs_indices [t, top_k]) by default; with
    lhs_indices, transpose=False or sorted_indices the indexed form.  The mx
    modes take the MoE form."""
    _mode_check(group_size, bits, mode, (global_scale,))
    if mode != "nvfp4":
        if lhs_indices is not None or not transpose or x.dim() != 2 or rhs_indices.dim() != 2:
            raise ValueError(f"[gather_qmm] mode {mode!r}: only x [t, k] with rhs_indices "
                             "[t, top_k] and transpose=True")
        return nvfp4_mx_gather_qmm(x, w, scales, rhs_indices, mode)
    if lhs_indices is None and transpose and not sorted_indices and x.dim() == 2 \
            and rhs_indices.dim() == 2 and rhs_indices.shape[0] == x.shape[0]:
        return nvfp4_gather_qmm(x, w, scales, rhs_indices, global_scale)
    return nvfp4_gather_qmm_indexed(x, w, scales, rhs_indices.reshape(-1), lhs_indices, global_scale,
                                    transpose, sorted_indices)


__all__ = [
    "load_library", "NVFP4Error", "nvfp4_tensor_amax", "nvfp4_quantize", "nvfp4_dequantize",
    "nvfp4_quant_dequant", "nvfp4_qmv", "nvfp4_qqmm", "nvfp4_qmm", "nvfp4_gather_qmm", "nvfp4_moe_route",
    "qqmm_workspace", "gather_workspace", "quantize", "dequantize", "qqmm", "gather_qmm",
    "MX_MODES", "MxPacked", "nvfp4_mx_quantize", "nvfp4_mx_dequantize", "nvfp4_mx_quant_dequant",
    "nvfp4_mx_pack", "mx_qqmm_workspace", "nvfp4_mx_qqmm", "nvfp4_mx_qqmm_packed",
    "nvfp4_mx_quantize_packed", "nvfp4_mx_mm_packed", "nvfp4_gather_qmm_indexed",
    "nvfp4_mx_gather_qmm",
]

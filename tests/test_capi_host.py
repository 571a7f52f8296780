"""Host-only checks of the C ABI (no GPU needed, no kernel is launched).

The library must load and export every entry point that include/nvfp4.h
declares, and every argument error must be reported on the host, before any
HIP call, with the pages' "[op] message" convention ("mlx 0.30.7.2 ->
0.30.7.6" diff page 8: validate_global_scale, validate_qqmm_inputs).
Addresses passed here are fake; validation rejects the call before anything
dereferences them, and the architecture override stops every call that
passes validation before it reaches the device.
"""
import ctypes
import os
import re

import pytest

import nvfp4_block_scaled_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")

INV, UNSUP = nv.NVFP4_ERR_INVALID_ARGUMENT, nv.NVFP4_ERR_UNSUPPORTED
F32, F16, BF16 = 0, 1, 2
A = 0x10000  # a fake, 256-byte aligned "device address"
B = 0x20000
C = 0x30000
G = 0x40000
W = 0x50000


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(nv.LIB_PATH):
        from nvfp4_block_scaled_amd import build
        build.build()
    lib = nv.load_library()
    lib.nvfp4_debug_set_arch_override(b"gfx942")  # nothing reaches a device
    yield lib
    lib.nvfp4_debug_set_arch_override(None)


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(L, n), n
        assert ctypes.cast(getattr(L, n), ctypes.c_void_p).value


def test_ceiling_library_exports_its_header():
    """libnvfp4_ceiling.so (the benchmark's read / copy / MFMA-loop kernels)
    loads and exports every function include/nvfp4_ceiling.h declares; its
    argument checks reject bad sizes before anything is enqueued."""
    path = os.path.join(ROOT, "nvfp4_block_scaled_amd", "libnvfp4_ceiling.so")
    if not os.path.exists(path):
        from nvfp4_block_scaled_amd import build
        build.build()
    lib = ctypes.CDLL(path)
    names = declared_functions(os.path.join(ROOT, "include", "nvfp4_ceiling.h"))
    assert names == ["nvfp4_ceiling_copy", "nvfp4_ceiling_mfma", "nvfp4_ceiling_read"]
    for n in names:
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value
    lib.nvfp4_ceiling_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
    lib.nvfp4_ceiling_mfma.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p]
    bad = 1  # hipErrorInvalidValue
    assert lib.nvfp4_ceiling_read(A, 24, B, None) == bad      # not a multiple of 16
    assert lib.nvfp4_ceiling_read(None, 32, B, None) == bad
    assert lib.nvfp4_ceiling_mfma(0, 4, B, C, None) == bad
    assert lib.nvfp4_ceiling_mfma(10, 0, B, C, None) == bad


def test_version(L):
    assert L.nvfp4_version() >= 100


def err(L):
    return L.nvfp4_last_error().decode()


def test_quantize_argument_errors(L):
    q = L.nvfp4_quantize
    assert q(A, BF16, 4, 24, None, B, C, None) == INV and "group size 16" in err(L)
    assert q(A, BF16, 4, 0, None, B, C, None) == INV
    assert q(A, 7, 4, 32, None, B, C, None) == INV and "Unsupported dtype" in err(L)
    assert q(A, BF16, -1, 32, None, B, C, None) == INV
    assert q(None, BF16, 4, 32, None, B, C, None) == INV and "NULL" in err(L)
    assert q(A, BF16, 4, 32, None, None, C, None) == INV
    assert q(A + 2, BF16, 4, 32, None, B, C, None) == INV and "aligned" in err(L)
    # valid arguments stop at the (overridden) architecture check
    assert q(A, BF16, 4, 32, G, B, C, None) == UNSUP and "gfx950" in err(L)


def test_dequantize_and_quant_dequant_errors(L):
    assert L.nvfp4_dequantize(A, B, 4, 40, None, C, BF16, None) == INV
    assert L.nvfp4_dequantize(None, B, 4, 32, None, C, BF16, None) == INV
    assert L.nvfp4_dequantize(A, B, 4, 32, None, C, 3, None) == INV
    assert L.nvfp4_quant_dequant(A, F16, 4, 32, None, None, None) == INV
    assert L.nvfp4_quant_dequant(A, F16, 4, 32, None, C + 8, None) == INV
    assert L.nvfp4_quant_dequant(A, F16, 4, 32, None, C, None) == UNSUP


def test_qqmm_global_scales_both_or_neither(L):
    ws = L.nvfp4_qqmm_workspace_size(8, 16, 32, BF16)
    assert ws >= 8 * 32 * 2 and ws % 256 == 0
    args = (A, BF16, G, W, B, None, 8, 16, 32, C, 0x60000, ws, None)
    assert L.nvfp4_qqmm(*args) == INV
    assert "both global_scale_x and global_scale_w" in err(L)
    args = (A, BF16, None, W, B, G, 8, 16, 32, C, 0x60000, ws, None)
    assert L.nvfp4_qqmm(*args) == INV
    assert L.nvfp4_qmv(A, BF16, G, W, B, None, 16, 32, C, None) == INV
    assert L.nvfp4_qmv(A, BF16, G, W, B, G, 16, 32, C, None) == UNSUP
    assert L.nvfp4_qmv(A, BF16, None, W, B, None, 16, 32, C, None) == UNSUP


def test_qqmm_shapes_and_workspace(L):
    ws = L.nvfp4_qqmm_workspace_size(8, 16, 32, BF16)
    assert L.nvfp4_qqmm(A, BF16, G, W, B, G, 8, 16, 20, C, 0x60000, ws, None) == INV
    assert L.nvfp4_qqmm(A, BF16, G, W, B, G, 0, 16, 32, C, 0x60000, ws, None) == INV
    assert L.nvfp4_qqmm(A, BF16, G, W, B, G, 8, 16, 32, C, 0x60000, ws - 1, None) == INV
    assert "workspace" in err(L)
    assert L.nvfp4_qqmm(A, BF16, G, W, B, G, 8, 16, 32, C, 0x60010, ws, None) == INV
    assert L.nvfp4_qqmm(A, BF16, G, W, B, G, 8, 16, 32, C, 0x60000, ws, None) == UNSUP
    # m == 1 needs no workspace
    assert L.nvfp4_qqmm_workspace_size(1, 16, 32, BF16) == 0
    assert L.nvfp4_qqmm(A, BF16, G, W, B, G, 1, 16, 32, C, None, 0, None) == UNSUP
    assert L.nvfp4_qmv(A, BF16, None, W, B, None, 16, 65536, C, None) == UNSUP


def test_gather_qmm_errors(L):
    ws = L.nvfp4_gather_qmm_workspace_size(10, 2, 4, 16, 32)
    assert ws >= (5 + 20) * 4
    ok = (A, BF16, W, B, G, 0x70000, 10, 2, 4, 16, 32, C, 0x60000, ws, None)
    assert L.nvfp4_gather_qmm(*ok) == UNSUP
    bad = list(ok)
    bad[10] = 24
    assert L.nvfp4_gather_qmm(*bad) == INV
    bad = list(ok)
    bad[13] = ws - 4
    assert L.nvfp4_gather_qmm(*bad) == INV
    bad = list(ok)
    bad[5] = None
    assert L.nvfp4_gather_qmm(*bad) == INV
    bad = list(ok)
    bad[8] = 2000
    assert L.nvfp4_gather_qmm(*bad) == UNSUP
    rws = L.nvfp4_moe_route_workspace_size(10, 2, 4)
    assert rws > 0 and rws % 256 == 0
    assert L.nvfp4_moe_route(0x70000, 10, 2, 0, A, B, 0x60000, rws, None) == INV
    assert L.nvfp4_moe_route(0x70000, 10, 2, 4, A, B, None, rws, None) == INV
    assert L.nvfp4_moe_route(0x70000, 10, 2, 4, A, B, 0x60000, rws - 1, None) == INV
    assert L.nvfp4_moe_route(0x70000, 10, 2, 4, A, B, 0x60010, rws, None) == INV
    assert L.nvfp4_moe_route(0x70000, 10, 2, 4, A, B, 0x60000, rws, None) == UNSUP
    # the gather workspace holds the routing's counts as well
    assert ws >= 256 + 256 + rws


def test_gather_noalloc_limits(L):
    """The allocation-free gather takes no workspace; tables beyond its fixed
    5 MiB scratch are refused on the host with the sizes in the message."""
    ok = (A, BF16, W, B, G, 0x70000, 1 << 19, 2, 256, 64, 32, C, None)
    assert L.nvfp4_gather_qmm_noalloc(*ok) == UNSUP and "gfx950" in err(L)  # fits: 2^20 pairs
    big = list(ok)
    big[6] = 1 << 20  # 2^21 pairs
    assert L.nvfp4_gather_qmm_noalloc(*big) == UNSUP and "scratch" in err(L) and "2097152" in err(L)
    big = list(ok)
    big[8] = 1024  # 1024 experts with 2^20 pairs
    assert L.nvfp4_gather_qmm_noalloc(*big) == UNSUP and "scratch" in err(L)
    bad = list(ok)
    bad[10] = 24
    assert L.nvfp4_gather_qmm_noalloc(*bad) == INV and "group size 16" in err(L)
    bad = list(ok)
    bad[5] = None
    assert L.nvfp4_gather_qmm_noalloc(*bad) == INV


def test_contraction_offset_limits(L):
    """The matrix-core contractions address x and the weight's codes with
    32-bit offsets: 2 GB or more of either is refused on the host (m > 1)."""
    big = 1 << 40  # a workspace size that never limits
    # x of 2^31 bytes: m * k * 2 = 2^31
    m, k = 1 << 15, 1 << 15
    assert L.nvfp4_qqmm(A, BF16, G, W, B, G, m, 64, k, C, 0x60000, big, None) == UNSUP
    assert "2 GB" in err(L)
    assert L.nvfp4_qmm(A, BF16, W, B, G, m, 64, k, C, None) == UNSUP and "2 GB" in err(L)
    # just below: validation passes and the architecture check stops the call
    assert L.nvfp4_qqmm(A, BF16, G, W, B, G, m - 1, 64, k, C, 0x60000, big, None) == UNSUP
    assert "gfx950" in err(L)
    # the weight's codes: n * k / 2 = 2^31
    n = 1 << 17
    assert L.nvfp4_qqmm(A, BF16, G, W, B, G, 64, n, k, C, 0x60000, big, None) == UNSUP
    assert "2 GB" in err(L)
    assert L.nvfp4_qqmm_packed(A, BF16, G, W, B, G, 64, n, k, C, 0x60000, big, None) == UNSUP
    assert "2 GB" in err(L)
    # one row of x streams with 64-bit addressing: no such limit
    assert L.nvfp4_qmv(A, BF16, None, W, B, None, n, 32768, C, None) == UNSUP
    assert "gfx950" in err(L)
    # gather: x rows (t) and one expert's codes
    gws = L.nvfp4_gather_qmm_workspace_size(1 << 16, 2, 8, 64, 1 << 14)
    assert L.nvfp4_gather_qmm(A, BF16, W, B, G, 0x70000, 1 << 16, 2, 8, 64, 1 << 14, C, 0x60000, gws,
                              None) == UNSUP and "2 GB" in err(L)
    gws = L.nvfp4_gather_qmm_workspace_size(64, 2, 8, n, k)
    assert L.nvfp4_gather_qmm(A, BF16, W, B, G, 0x70000, 64, 2, 8, n, k, C, 0x60000, gws,
                              None) == UNSUP and "2 GB" in err(L)
    assert L.nvfp4_gather_qmm_packed(A, BF16, W, B, G, 0x70000, 64, 2, 8, n, k, C, 0x60000, gws,
                                     None) == UNSUP and "2 GB" in err(L)


def test_tensor_amax_errors(L):
    assert L.nvfp4_tensor_amax(A, BF16, -1, B, None) == INV
    assert L.nvfp4_tensor_amax(A, BF16, 10, None, None) == INV
    assert L.nvfp4_tensor_amax(A, 9, 10, B, None) == INV
    assert L.nvfp4_tensor_amax(A, BF16, 10, B, None) == UNSUP


def test_python_binding_rejects_host_tensors_and_bad_modes():
    import torch
    x = torch.zeros(4, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        nv.nvfp4_quantize(x)
    with pytest.raises(ValueError):
        nv.quantize(x, group_size=32, mode="nvfp4")
    with pytest.raises(ValueError):
        nv.quantize(x, mode="mxfp6")
    with pytest.raises(ValueError):
        nv.quantize(x, mode="mxfp4", global_scale=torch.ones(1))
    with pytest.raises(ValueError):
        nv.quantize(x, group_size=16, mode="mxfp8")
    with pytest.raises(ValueError):
        nv.nvfp4_mx_quantize(x, "mxfp4")  # host tensor


def test_mx_argument_errors(L):
    cb, sb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    # 100 rows -> 4 tiles; k = 96 -> 2 steps, padded to one quad of 4
    assert L.nvfp4_mx_pack_size(4, 100, 96, ctypes.byref(cb), ctypes.byref(sb)) == 0
    assert cb.value == 4 * 4 * 2 * 512 and sb.value == 4 * 1 * 256
    assert L.nvfp4_mx_pack_size(8, 100, 320, ctypes.byref(cb), ctypes.byref(sb)) == 0
    assert cb.value == 4 * 8 * 4 * 512 and sb.value == 4 * 2 * 256
    assert L.nvfp4_mx_pack_size(6, 100, 96, ctypes.byref(cb), ctypes.byref(sb)) == INV
    assert "mx mode" in err(L) and cb.value == 0
    assert L.nvfp4_mx_pack_size(4, 100, 48, ctypes.byref(cb), ctypes.byref(sb)) == INV
    assert "multiple of 32" in err(L)
    assert L.nvfp4_mx_quantize(A, BF16, 4, 4, 48, B, C, None) == INV and "group size 32" in err(L)
    assert L.nvfp4_mx_quantize(A, BF16, 5, 4, 64, B, C, None) == INV and "[mx_quantize]" in err(L)
    assert L.nvfp4_mx_quantize(A + 8, BF16, 8, 4, 64, B, C, None) == INV and "aligned" in err(L)
    assert L.nvfp4_mx_quantize(A, 7, 8, 4, 64, B, C, None) == INV
    assert L.nvfp4_mx_quantize(A, BF16, 8, 4, 64, B, C, None) == UNSUP  # validation passed
    assert L.nvfp4_mx_dequantize(A, B, 4, 4, 64, None, BF16, None) == INV
    assert L.nvfp4_mx_quant_dequant(A, F16, 4, 4, 64, B + 4, None) == INV and "aligned" in err(L)
    need = L.nvfp4_mx_qqmm_workspace_size(4, 300, 520, 192, 0)
    need_p = L.nvfp4_mx_qqmm_workspace_size(4, 300, 520, 192, 1)
    assert need > need_p > 0 and need % 256 == 0 and need_p % 256 == 0
    assert L.nvfp4_mx_qqmm_workspace_size(4, 300, 520, 100, 0) == 0
    assert L.nvfp4_mx_qqmm(A, BF16, 4, B, C, 300, 520, 192, G, W, need - 1, None) == INV
    assert "workspace" in err(L)
    assert L.nvfp4_mx_qqmm(A, BF16, 4, B, C, 300, 520, 192, G, W + 16, need, None) == INV
    assert L.nvfp4_mx_qqmm(A, BF16, 4, B, C, 0, 520, 192, G, W, need, None) == INV
    assert L.nvfp4_mx_qqmm(A, BF16, 4, None, C, 300, 520, 192, G, W, need, None) == INV
    assert L.nvfp4_mx_qqmm(A, BF16, 4, B, C, 300, 520, 192, G, W, need, None) == UNSUP
    # one row of x with up to 8 KB of codes per row: the matrix-vector kernel,
    # no workspace (NULL accepted); longer rows take the matrix-core kernel
    assert L.nvfp4_mx_qqmm_workspace_size(4, 1, 14336, 4096, 0) == 0
    assert L.nvfp4_mx_qqmm_workspace_size(8, 1, 14336, 4096, 0) == 0
    assert L.nvfp4_mx_qqmm_workspace_size(8, 1, 14336, 4096, 1) > 0
    assert L.nvfp4_mx_qqmm_workspace_size(4, 1, 300, 2048, 0) == 0
    assert L.nvfp4_mx_qqmm_workspace_size(4, 1, 300, 32, 0) == 0
    assert L.nvfp4_mx_qqmm_workspace_size(4, 1, 300, 16384, 0) == 0
    assert L.nvfp4_mx_qqmm_workspace_size(4, 1, 300, 16416, 0) > 0
    assert L.nvfp4_mx_qqmm_workspace_size(8, 1, 300, 8192, 0) == 0
    assert L.nvfp4_mx_qqmm_workspace_size(8, 1, 300, 8224, 0) > 0
    assert L.nvfp4_mx_qqmm_workspace_size(4, 2, 300, 2048, 0) > 0
    assert L.nvfp4_mx_qqmm(A, BF16, 8, B, C, 1, 14336, 4096, G, None, 0, None) == UNSUP
    need_p8 = L.nvfp4_mx_qqmm_workspace_size(8, 300, 520, 192, 1)
    assert need_p8 > need_p  # mxfp8 codes take twice the bytes
    assert L.nvfp4_mx_qqmm_packed(A, BF16, 8, B, C, 300, 520, 192, G, W, need_p8 - 1, None) == INV
    assert L.nvfp4_mx_qqmm_packed(A, BF16, 8, B, C, 300, 520, 192, G, W, need_p8, None) == UNSUP
    # a packed operand of 2 GB or more is refused before the device
    assert L.nvfp4_mx_qqmm_packed(A, BF16, 8, B, C, 2048, 1 << 21, 1024, G, W, 1 << 40, None) == UNSUP
    assert "too large" in err(L)


def test_mfma_pack_sizes_and_errors(L):
    cb, sb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    # 100 rows -> 4 tiles of 32 rows; k = 256 -> 4 k-steps of 64
    assert L.nvfp4_mfma_pack_size(100, 256, ctypes.byref(cb), ctypes.byref(sb)) == 0
    assert cb.value == 4 * 4 * 1024 and sb.value == 4 * 4 * 128
    assert L.nvfp4_mfma_pack_size(100, 96, ctypes.byref(cb), ctypes.byref(sb)) == INV
    assert "multiple of 64" in err(L) and cb.value == 0 and sb.value == 0
    assert L.nvfp4_mfma_pack_size(0, 64, ctypes.byref(cb), ctypes.byref(sb)) == INV
    assert L.nvfp4_mfma_pack(A, B, 100, 96, C, G, None) == INV and "[mfma_pack]" in err(L)
    assert L.nvfp4_mfma_pack(A + 4, B, 100, 64, C, G, None) == INV and "aligned" in err(L)
    assert L.nvfp4_mfma_pack(A, B, 100, 64, None, G, None) == INV
    assert L.nvfp4_mfma_pack(A, B, 100, 64, C, G, None) == UNSUP


def test_packed_matmul_errors(L):
    ws = L.nvfp4_qqmm_workspace_size(8, 16, 64, BF16)
    ok = (A, BF16, G, W, B, G, 8, 16, 64, C, 0x60000, ws, None)
    assert L.nvfp4_qqmm_packed(*ok) == UNSUP
    bad = list(ok)
    bad[1] = F32
    assert L.nvfp4_qqmm_packed(*bad) == INV and "float16 or bfloat16" in err(L)
    bad = list(ok)
    bad[8] = 32
    assert L.nvfp4_qqmm_packed(*bad) == INV and "multiple of 64" in err(L)
    bad = list(ok)
    bad[7] = 18
    assert L.nvfp4_qqmm_packed(*bad) == INV and "multiple of 4" in err(L)
    bad = list(ok)
    bad[5] = None
    assert L.nvfp4_qqmm_packed(*bad) == INV and "both global_scale_x" in err(L)
    # m == 1 still runs the matrix-core path, so it needs the workspace
    assert L.nvfp4_qqmm_packed(A, BF16, G, W, B, G, 1, 16, 64, C, None, 0, None) == INV
    assert L.nvfp4_qmm_packed(A, F16, W, B, G, 8, 16, 64, C, None) == UNSUP
    assert L.nvfp4_qmm_packed(A, F16, W, B, G, 8, 16, 80, C, None) == INV
    gws = L.nvfp4_gather_qmm_workspace_size(10, 2, 4, 64, 64)
    gok = (A, BF16, W, B, G, 0x70000, 10, 2, 4, 64, 64, C, 0x60000, gws, None)
    assert L.nvfp4_gather_qmm_packed(*gok) == UNSUP
    bad = list(gok)
    bad[9] = 48
    assert L.nvfp4_gather_qmm_packed(*bad) == INV and "multiple of 32" in err(L)
    bad = list(gok)
    bad[13] = gws - 4
    assert L.nvfp4_gather_qmm_packed(*bad) == INV and "workspace" in err(L)


def test_columnwise_errors(L):
    q = L.nvfp4_quantize_columnwise
    assert q(A, BF16, 24, 16, None, B, C, None) == INV and "group size 16" in err(L)
    assert q(A, BF16, 32, 12, None, B, C, None) == INV and "multiple of 8" in err(L)
    assert q(A, F32, 32, 12, None, B, C, None) == UNSUP  # float32 needs cols % 4 only
    assert q(A, BF16, 32, 16, None, B + 4, C, None) == INV and "aligned" in err(L)
    assert q(None, BF16, 32, 16, None, B, C, None) == INV
    assert q(A, BF16, 32, 16, None, B, C, None) == UNSUP
    qd = L.nvfp4_quant_dequant_columnwise
    assert qd(A, F16, 32, 16, None, None, None) == INV
    assert qd(A, F16, 32, 16, None, C + 8, None) == INV
    assert qd(A, F16, 32, 16, None, C, None) == UNSUP


def test_vjp_errors(L):
    ws = L.nvfp4_qqmm_vjp_workspace_size(32, 64, 48, BF16)
    assert ws % 256 == 0 and ws >= 64 * 48 // 2 + 32 * 64 * 2 * 2 + 48 * 32 // 2
    D = 0x70000
    vjp = L.nvfp4_qqmm_vjp
    ok = (A, W, B, BF16, G, G, 32, 64, 48, C, D, None, 0x80000, ws, None)
    assert vjp(*ok) == UNSUP
    bad_m = ok[:6] + (24,) + ok[7:]
    assert vjp(*bad_m) == INV and "multiples of 16" in err(L)
    one_g = ok[:4] + (G, None) + ok[6:]
    assert vjp(*one_g) == INV and "both global_scale_x and global_scale_w" in err(L)
    none_out = ok[:9] + (None, None) + ok[11:]
    assert vjp(*none_out) == INV and "both NULL" in err(L)
    small_ws = ok[:13] + (ws - 1,) + ok[14:]
    assert vjp(*small_ws) == INV and "workspace" in err(L)
    # dx alone needs no x, dw alone no w
    assert vjp(None, W, B, BF16, G, G, 32, 64, 48, C, None, None, 0x80000, ws, None) == UNSUP
    assert vjp(A, None, B, BF16, G, G, 32, 64, 48, None, D, None, 0x80000, ws, None) == UNSUP
    assert vjp(None, W, B, BF16, G, G, 32, 64, 48, C, D, None, 0x80000, ws, None) == INV


def test_gather_indexed_errors(L):
    need = L.nvfp4_gather_qmm_indexed_workspace_size(70, 1, 4, 1)
    assert need > L.nvfp4_gather_qmm_indexed_workspace_size(70, 1, 4, 0) > 0 and need % 256 == 0
    assert L.nvfp4_gather_qmm_indexed_workspace_size(0, 1, 4, 1) == 0
    args = lambda **kw: dict(dict(x=A, dt=BF16, entries=40, mr=1, wc=B, ws=C, g=None, lhs=G, rhs=W,
                                  pairs=70, e=4, n=160, k=96, tr=1, srt=0, out=A, wsp=W + 0x1000,
                                  nb=need), **kw)
    call = lambda a: L.nvfp4_gather_qmm_indexed(a["x"], a["dt"], a["entries"], a["mr"], a["wc"], a["ws"],
                                                a["g"], a["lhs"], a["rhs"], a["pairs"], a["e"], a["n"],
                                                a["k"], a["tr"], a["srt"], a["out"], a["wsp"], a["nb"], None)
    assert call(args()) == UNSUP  # validation passed
    assert call(args(k=100)) == INV and "group size 16" in err(L)
    assert call(args(tr=0, k=96, n=100)) == INV and "quantized along n" in err(L)
    assert call(args(tr=0, k=100)) == INV and "multiple of 8" in err(L)
    assert call(args(tr=0, k=100, n=160)) == INV
    assert call(args(lhs=None)) == INV and "must not exceed entries" in err(L)
    assert call(args(rhs=None)) == INV
    assert call(args(x=A + 8)) == INV and "aligned" in err(L)
    assert call(args(nb=need - 1)) == INV and "workspace" in err(L)
    assert call(args(e=2000)) == UNSUP
    assert call(args(dt=7)) == INV


def test_mx_gather_qmm_errors(L):
    ws = L.nvfp4_gather_qmm_workspace_size(10, 2, 4, 16, 64)
    ok = (A, BF16, 4, W, B, 0x70000, 10, 2, 4, 16, 64, C, 0x60000, ws, None)
    assert L.nvfp4_mx_gather_qmm(*ok) == UNSUP and "gfx950" in err(L)  # validation passed
    for i, v, what in ((2, 6, "mx mode"), (1, 7, "dtype"), (10, 48, "group size 32"),
                       (10, 0, "group size 32"), (13, ws - 4, "workspace"), (12, 0x60010, "aligned"),
                       (5, None, "NULL"), (3, W + 8, "aligned"), (0, A + 8, "aligned"),
                       (6, 0, "positive"), (9, 0, "positive")):
        bad = list(ok)
        bad[i] = v
        assert L.nvfp4_mx_gather_qmm(*bad) == INV, (i, v)
        assert "[mx_gather_qmm]" in err(L) and what in err(L), err(L)
    bad = list(ok)
    bad[8] = 2000
    assert L.nvfp4_mx_gather_qmm(*bad) == UNSUP and "1024 experts" in err(L)
    # one expert's mxfp8 codes of 2 GB or more (n * k bytes) are refused; the
    # same sizes in mxfp4 (half the bytes) pass validation
    gws = L.nvfp4_gather_qmm_workspace_size(64, 2, 8, 1 << 17, 1 << 14)
    big = (A, BF16, 8, W, B, 0x70000, 64, 2, 8, 1 << 17, 1 << 14, C, 0x60000, gws, None)
    assert L.nvfp4_mx_gather_qmm(*big) == UNSUP and "2 GB" in err(L)
    big = list(big)
    big[2] = 4
    assert L.nvfp4_mx_gather_qmm(*big) == UNSUP and "gfx950" in err(L)

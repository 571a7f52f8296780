"""GPU parity of the backward path: columnwise quantize / round trip and the
vjp of qqmm (nvfp4_qqmm_vjp) against the oracle.

Bars: codes and scales bit for bit; round-tripped values equal; on the
doubly-grid operands of the oracle's vjp pin the gradients equal the exact
products rounded once (bit for bit); on general data the norm-wise 1e-2 bar
and the matrix-core regression guard (the decoded weights are rounded to the
16-bit type before the products)."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_amd as nv
import workloads as W
from _parity import (O, assert_bytes_equal, assert_close, assert_values_equal, host,
                     oracle_dtype, say, scalar)

pytestmark = pytest.mark.gpu

MFMA_FRO_GUARD = 5e-3
G_X = 2688.0 * 2.0 ** -20
G_W = 2688.0 * 2.0 ** 10


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    nv.load_library()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("rows,cols", [(16, 8), (272, 200), (512, 64)])
@pytest.mark.parametrize("with_g", [True, False])
def test_columnwise_quantize_and_round_trip(dtype, rows, cols, with_g):
    """Ragged tiles in both directions (256 x 64 tiles)."""
    say(f"columnwise {dtype} {rows}x{cols} g={with_g}")
    x = W.normal((rows, cols), 1.0, 400 + rows + cols, oracle_dtype(dtype), outlier_frac=0.01,
                 outlier_mult=30.0)
    g = O.tensor_amax(host(x)) if with_g else None
    xd = x.cuda()
    codes, scales = nv.nvfp4_quantize_columnwise(xd, scalar(g))
    xt_hat = nv.nvfp4_quant_dequant_columnwise(xd, scalar(g))
    torch.cuda.synchronize()
    oc, os_ = O.quantize_columnwise(host(x), g)
    assert_bytes_equal(codes.cpu().numpy(), oc, "columnwise codes")
    assert_bytes_equal(scales.cpu().numpy(), os_, "columnwise scales")
    assert_values_equal(host(xt_hat), O.quant_dequant_columnwise(host(x), g, dtype=oracle_dtype(dtype)),
                        "columnwise round trip")


def test_columnwise_quantize_weight_14336x4096():
    """The weight of the prefill shape quantized along its rows (as the vjp
    does for dx), g = amax(w)."""
    say("columnwise 14336x4096")
    w = W.normal((14336, 4096), 0.02, 410, "bf16")
    g = O.tensor_amax(host(w))
    codes, scales = nv.nvfp4_quantize_columnwise(w.cuda(), scalar(g))
    torch.cuda.synchronize()
    oc, os_ = O.quantize_columnwise(host(w), g)
    assert_bytes_equal(scales.cpu().numpy(), os_, "scales")
    assert_bytes_equal(codes.cpu().numpy(), oc, "codes")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("m,n,k", [(32, 64, 48), (16, 128, 64)])
def test_vjp_exact_on_grid_operands(dtype, m, n, k):
    """The oracle pin's operands: dx = dy @ w and dw = dy^T @ x exactly,
    g_dy = max|dy| (the second shape takes the small-batch kernel for dx)."""
    say(f"vjp grid {dtype} {m}x{n}x{k}")
    x = W.doubly_grid(m, k, seed=1, scale=2.0 ** -20, col_exponent_period=4)
    w = W.doubly_grid(n, k, seed=2, scale=2.0 ** 10, col_exponent_period=4)
    dy = W.doubly_grid(m, n, seed=3, scale=2.0 ** -8)
    od = oracle_dtype(dtype)
    dx, dw, gdy = nv.nvfp4_qqmm_vjp(x.to(dtype).cuda(), w.to(dtype).cuda(), dy.to(dtype).cuda(),
                                    scalar(G_X), scalar(G_W))
    torch.cuda.synchronize()
    assert float(gdy.item()) == 6.0 * 2.0 ** -8
    x64, w64, dy64 = (t.double().numpy() for t in (x, w, dy))
    round_t = lambda a: np.array([[O.round_to(float(v), od) for v in row] for row in a], np.float32)
    assert_values_equal(host(dx), round_t(dy64 @ w64), "dx")
    assert_values_equal(host(dw), round_t(dy64.T @ x64), "dw")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("m,n,k,with_g", [(64, 320, 192, True), (128, 256, 128, False),
                                          (16, 256, 384, True)])
def test_vjp_general(dtype, m, n, k, with_g):
    say(f"vjp general {dtype} {m}x{n}x{k} g={with_g}")
    od = oracle_dtype(dtype)
    x = W.normal((m, k), 1.0, 420 + m, od)
    w = W.normal((n, k), 0.02, 421 + n, od)
    dy = W.normal((m, n), 0.01, 422 + k, od)
    gx = O.tensor_amax(host(x)) if with_g else None
    gw = O.tensor_amax(host(w)) if with_g else None
    dx, dw, gdy = nv.nvfp4_qqmm_vjp(x.cuda(), w.cuda(), dy.cuda(), scalar(gx), scalar(gw))
    torch.cuda.synchronize()
    rdx, rdw, rg = O.qqmm_vjp(host(x), host(w), host(dy), gx, gw, dtype=od)
    if with_g:
        assert float(gdy.item()) == rg
    else:
        assert gdy is None
    for got, ref, what in ((dx, rdx, "dx"), (dw, rdw, "dw")):
        fro, _ = assert_close(host(got), ref, what=what)
        assert fro <= MFMA_FRO_GUARD


def test_vjp_one_gradient_at_a_time():
    """dx alone and dw alone give the same values as both together."""
    say("vjp dx / dw alone")
    m, n, k = 64, 128, 192
    x = W.normal((m, k), 1.0, 430, "bf16").cuda()
    w = W.normal((n, k), 0.02, 431, "bf16").cuda()
    dy = W.normal((m, n), 0.01, 432, "bf16").cuda()
    gx, gw = nv.nvfp4_tensor_amax(x), nv.nvfp4_tensor_amax(w)
    dx, dw, _ = nv.nvfp4_qqmm_vjp(x, w, dy, gx, gw)
    dx1, none1, _ = nv.nvfp4_qqmm_vjp(x, w, dy, gx, gw, want_dw=False)
    none2, dw2, _ = nv.nvfp4_qqmm_vjp(x, w, dy, gx, gw, want_dx=False)
    torch.cuda.synchronize()
    assert none1 is None and none2 is None
    assert torch.equal(dx.view(torch.int16), dx1.view(torch.int16))
    assert torch.equal(dw.view(torch.int16), dw2.view(torch.int16))

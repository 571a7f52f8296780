"""Pins of the oracle's backward functions (columnwise quantize, QQMatmul's
vjp) against what the mathematics fixes, independent of the oracle's code.

The vjp pin uses "doubly grid" operands: values on the e2m1 grid with a +6
and a -6 in every group of 16 along both axes, scaled by powers of two, and
global scales for which the encode and decode factors are exact.  On such
data every quantization along the intended axis is exact, so the gradients
equal plain float64 products:
    dx = dy @ w,   dw = dy^T @ x     (y = x @ w^T).
Each operand carries its own power of two, so that encoding an operand with
another operand's global scale either underflows its block scales to zero or
saturates its codes; and x and w carry a factor that varies along their
columns (2^(c % 4)), so that only the grouping along their rows (m for x, n
for w -- the axis the vjp quantizes them along) is exact.  A swapped global
scale, a wrong grouping axis or a transposed operand fails the pin (the
mutants below show it; a missing transpose also changes the output shape)."""
import numpy as np
import pytest

import workloads as W
from oracle import oracle as O

M, N, K = 32, 64, 48


def _operands():
    x = W.doubly_grid(M, K, seed=1, scale=2.0 ** -20, col_exponent_period=4).numpy()
    w = W.doubly_grid(N, K, seed=2, scale=2.0 ** 10, col_exponent_period=4).numpy()
    dy = W.doubly_grid(M, N, seed=3, scale=2.0 ** -8).numpy()
    return x, w, dy


G_X = 2688.0 * 2.0 ** -20  # encode factor 2^20, decode factor 2^-20, both exact
G_W = 2688.0 * 2.0 ** 10


def test_doubly_grid_structure():
    x = W.doubly_grid(48, 64, seed=5).numpy()
    grid = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0}
    assert set(np.abs(x).ravel().tolist()) <= grid
    for axis in (0, 1):
        g = np.moveaxis(x, axis, 1).reshape(x.shape[1 - axis], -1, 16)
        assert (g.max(axis=2) == 6).all() and (g.min(axis=2) == -6).all()


def test_vjp_exact_on_grid_operands():
    """dx = dy @ w and dw = dy^T @ x exactly (float32 outputs), g_dy = max|dy|."""
    x, w, dy = _operands()
    dx, dw, g_dy = O.qqmm_vjp(x, w, dy, G_X, G_W, dtype="f32")
    assert dx.shape == (M, K) and dw.shape == (N, K)
    assert g_dy == float(np.abs(dy).max()) == 6.0 * 2.0 ** -8
    np.testing.assert_array_equal(dx, (dy.astype(np.float64) @ w.astype(np.float64)).astype(np.float32))
    np.testing.assert_array_equal(dw, (dy.T.astype(np.float64) @ x.astype(np.float64)).astype(np.float32))


def test_vjp_exact_without_global_scales():
    x = W.doubly_grid(M, K, seed=6).numpy()
    w = W.doubly_grid(N, K, seed=7).numpy()
    dy = W.doubly_grid(M, N, seed=8).numpy()
    dx, dw, g_dy = O.qqmm_vjp(x, w, dy, None, None, dtype="f32")
    assert g_dy is None
    np.testing.assert_array_equal(dx, (dy.astype(np.float64) @ w.astype(np.float64)).astype(np.float32))
    np.testing.assert_array_equal(dw, (dy.T.astype(np.float64) @ x.astype(np.float64)).astype(np.float32))


def test_vjp_bf16_output_is_one_rounding_of_the_exact_product():
    x, w, dy = _operands()
    dx, dw, _ = O.qqmm_vjp(x, w, dy, G_X, G_W, dtype="bf16")
    exact = (dy.astype(np.float64) @ w.astype(np.float64))
    ref = np.array([[O.round_to(float(v), "bf16") for v in row] for row in exact], np.float32)
    np.testing.assert_array_equal(dx, ref)


@pytest.mark.parametrize("mistake", ["x with g_w", "w with g_x", "w grouped along k",
                                     "x grouped along k", "dy with g_x instead of its amax"])
def test_vjp_pin_catches_mistakes(mistake):
    """Plausible implementation mistakes, built from the oracle's own pieces,
    each move a gradient away from the float64 product."""
    x, w, dy = _operands()
    g_dy = O.tensor_amax(dy)
    dx_ref = (dy.astype(np.float64) @ w.astype(np.float64)).astype(np.float32)
    dw_ref = (dy.T.astype(np.float64) @ x.astype(np.float64)).astype(np.float32)
    if mistake == "x with g_w":
        dw = O.qqmm(dy.T.copy(), *O.quantize_columnwise(x, G_W), g_dy, G_W, dtype="f32")
        assert not np.array_equal(dw, dw_ref)
    elif mistake == "w with g_x":
        dx = O.qqmm(dy, *O.quantize_columnwise(w, G_X), g_dy, G_X, dtype="f32")
        assert not np.array_equal(dx, dx_ref)
    elif mistake == "w grouped along k":
        # w decoded from a rowwise encode (groups along k), then used as w^T
        w_hat = O.dequantize(*O.quantize(w, G_W), G_W, dtype="f32")
        dx = O.qqmm(dy, *O.quantize(np.ascontiguousarray(w_hat.T), G_W), g_dy, G_W, dtype="f32")
        assert not np.array_equal(dx, dx_ref)
    elif mistake == "x grouped along k":
        x_hat = O.dequantize(*O.quantize(x, G_X), G_X, dtype="f32")
        dw = O.qqmm(dy.T.copy(), *O.quantize(np.ascontiguousarray(x_hat.T), G_X), g_dy, G_X,
                    dtype="f32")
        assert not np.array_equal(dw, dw_ref)
    else:
        dx = O.qqmm(dy, *O.quantize_columnwise(w, G_W), G_X, G_W, dtype="f32")
        assert not np.array_equal(dx, dx_ref)


def test_columnwise_round_trip_exact():
    """Doubly-grid x with g = 2688: every column group has amax 6, so the
    scales are all 1.0 (0x38) and the decode gives x^T back exactly."""
    x = W.doubly_grid(64, 48, seed=9).numpy()
    codes, scales = O.quantize_columnwise(x, 2688.0)
    assert codes.shape == (48, 32) and scales.shape == (48, 4)
    assert (scales == 0x38).all()
    np.testing.assert_array_equal(O.dequantize(codes, scales, 2688.0, dtype="f32"), x.T)
    np.testing.assert_array_equal(O.quant_dequant_columnwise(x, 2688.0, dtype="f32"), x.T)


def test_columnwise_invariants_on_general_data():
    """With g = amax: the largest scale byte is 0x7E and sits in the column
    group holding the amax; no byte is 0x7F or has its sign bit; in groups
    with scale >= 2^-6 every element of magnitude amax_b encodes to +-6."""
    x = W.normal((96, 40), 1.0, seed=10, dtype="bf16").float().numpy()
    g = O.tensor_amax(x)
    codes, scales = O.quantize_columnwise(x, g)
    assert scales.max() == 0x7E and not (scales & 0x80).any() and not (scales == 0x7F).any()
    r, c = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert scales[c, r // 16] == 0x7E
    nib = np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(40, 96)
    xt = x.T
    for col in range(40):
        for grp in range(6):
            seg = np.abs(xt[col, 16 * grp: 16 * grp + 16])
            if O.e4m3_value(int(scales[col, grp])) >= 2.0 ** -6:
                top = np.nonzero(seg == seg.max())[0]
                assert all((nib[col, 16 * grp + t] & 7) == 7 for t in top)

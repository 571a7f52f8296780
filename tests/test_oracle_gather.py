"""Pins of the oracle's indexed gather_qmm (the cells of the pages' gather_qmm
test loops: float32 / float16 / bfloat16, transpose True and False, per-expert
global scales of shape [E, 1, 1] -- "[Metal] global scale for qmm" (PR 4458)
test hunk; the op's lhs_indices / rhs_indices arguments).

The transpose pin uses doubly-grid experts: values on the e2m1 grid with +6
and -6 in every 16-group along both axes, times a per-expert power of two, and
per-expert global scales whose encode and decode factors are exact.  Such a
weight quantizes exactly along either axis, so transpose=True (w [n, k]
quantized along k) and transpose=False (w^T [k, n] quantized along n) must both
give the float64 product, and reading one layout as the other does not."""
import numpy as np
import pytest

import workloads as W
from oracle import oracle as O

E, N, K = 3, 48, 64


def _experts(square=False):
    n = K if square else N
    ws = [W.doubly_grid(n, K, seed=20 + e, scale=2.0 ** (3 * e - 2)).numpy() for e in range(E)]
    g = np.array([2688.0 * 2.0 ** (3 * e - 2) for e in range(E)], np.float32).reshape(E, 1, 1)
    return ws, g


def _quantized(ws, g, transpose):
    codes, scales = [], []
    for e, w in enumerate(ws):
        src = w if transpose else np.ascontiguousarray(w.T)
        c, s = O.quantize(src, float(g[e, 0, 0]))
        codes.append(c)
        scales.append(s)
    return np.stack(codes), np.stack(scales)


def _exact(x, ws, lhs, rhs, mr, dtype):
    x3 = x.reshape(-1, mr, K).astype(np.float64)
    out = []
    for p in range(len(rhs)):
        ent = p if lhs is None else lhs[p]
        out.append(x3[ent] @ ws[rhs[p]].astype(np.float64).T)
    y = np.concatenate(out, axis=0)
    return np.array([[O.round_to(float(v), dtype) for v in row] for row in y], np.float32)


@pytest.mark.parametrize("transpose", [True, False])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_exact_on_doubly_grid_experts(transpose, dtype):
    ws, g = _experts()
    codes, scales = _quantized(ws, g, transpose)
    rng = np.random.default_rng(3)
    x = W.grid_tensor(10, K, seed=4).numpy()
    rhs = rng.integers(0, E, 16).astype(np.int32)
    lhs = rng.integers(0, 10, 16).astype(np.int32)
    y = O.gather_qmm_indexed(x, codes, scales, rhs, lhs, g, transpose=transpose, dtype=dtype)
    np.testing.assert_array_equal(y, _exact(x, ws, lhs, rhs, 1, dtype))


def test_reading_one_layout_as_the_other_fails_the_pin():
    """Square experts: the [k, n] codes passed as if they were [n, k] give
    the product with w instead of w^T."""
    ws, g = _experts(square=True)
    codes, scales = _quantized(ws, g, transpose=False)
    x = W.grid_tensor(4, K, seed=5).numpy()
    rhs = np.array([0, 1, 2, 1], np.int32)
    wrong = O.gather_qmm_indexed(x, codes, scales, rhs, None, g, transpose=True, dtype="f32")
    assert not np.array_equal(wrong, _exact(x, ws, None, rhs, 1, "f32"))
    right = O.gather_qmm_indexed(x, codes, scales, rhs, None, g, transpose=False, dtype="f32")
    np.testing.assert_array_equal(right, _exact(x, ws, None, rhs, 1, "f32"))


def test_swapped_expert_scales_fail_the_pin():
    ws, g = _experts()
    codes, scales = _quantized(ws, g, transpose=True)
    x = W.grid_tensor(6, K, seed=6).numpy()
    rhs = np.array([0, 1, 2, 2, 1, 0], np.int32)
    y = O.gather_qmm_indexed(x, codes, scales, rhs, None, g[::-1].copy(), dtype="f32")
    assert not np.array_equal(y, _exact(x, ws, None, rhs, 1, "f32"))


def test_rows_per_entry_equal_the_flattened_call():
    """x [b, mr, k] with pair (lhs[p], rhs[p]) equals x [b * mr, k] with the
    pairs expanded row by row."""
    ws, g = _experts()
    codes, scales = _quantized(ws, g, transpose=True)
    rng = np.random.default_rng(7)
    b, mr = 5, 3
    x = W.normal((b * mr, K), 1.0, 8, "f32").numpy()
    lhs = rng.integers(0, b, 7).astype(np.int32)
    rhs = rng.integers(0, E, 7).astype(np.int32)
    y = O.gather_qmm_indexed(x.reshape(b, mr, K), codes, scales, rhs, lhs, g, dtype="f32")
    lhs2 = np.array([lhs[p] * mr + r for p in range(7) for r in range(mr)], np.int32)
    rhs2 = np.repeat(rhs, mr)
    y2 = O.gather_qmm_indexed(x, codes, scales, rhs2, lhs2, g, dtype="f32")
    np.testing.assert_array_equal(y, y2)


def test_moe_form_is_lhs_p_over_top_k():
    """The MoE call (x [t, k], idx [t, top_k]) is the indexed call with
    lhs[p] = p // top_k and rhs = idx flattened; the subset arguments select
    rows and columns of the whole."""
    ws, g = _experts()
    codes, scales = _quantized(ws, g, transpose=True)
    rng = np.random.default_rng(9)
    t, top_k = 8, 2
    x = W.normal((t, K), 1.0, 10, "bf16").float().numpy()
    idx = np.stack([rng.permutation(E)[:top_k] for _ in range(t)]).astype(np.int32)
    ref = O.gather_qmm(x, codes, scales, idx, g, dtype="bf16").reshape(t * top_k, N)
    lhs = (np.arange(t * top_k) // top_k).astype(np.int32)
    y = O.gather_qmm_indexed(x, codes, scales, idx.reshape(-1), lhs, g, dtype="bf16")
    np.testing.assert_array_equal(y, ref)
    sub = O.gather_qmm_indexed(x, codes, scales, idx.reshape(-1), lhs, g, dtype="bf16", rows=[1, 9],
                               cols=[0, 47])
    np.testing.assert_array_equal(sub, ref[[1, 9]][:, [0, 47]])

"""Pins of the oracle's encode / decode / contraction against what the pages fix
and against the mathematics (CPU only).

Each pin is chosen so that a plausible mistake in the oracle (a dropped global
factor, the factor on the sum, a wrong nibble order, a transposed operand, a
bfloat16 intermediate) fails at least one of them; the mutant tests plant such
mistakes in the oracle and check that the pins notice.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def read_kv(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                out[k] = float(v)
    return out


def read_cases():
    rows = {}
    with open(os.path.join(GOLDEN, "grid_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                c, gx, gw, dt, wscale, wdec, factor = line.split()
                rows[c] = dict(gx=None if gx == "none" else float(gx),
                               gw=None if gw == "none" else float(gw), dtype=dt,
                               wscale=float(wscale), wdec=float(wdec), factor=float(factor))
    return rows


def f32np(t):
    return t.to(torch.float32).numpy()


# ------------------------------------------------------------- worked example

def test_worked_example_of_the_global_scale_pull_request():
    """"[Metal] global scale for qmm" (ml-explore/mlx PR 4458), "Example":
    q = 6, block scale 0.5 (e4m3 byte 0x30), decode factor 0.1."""
    ex = read_kv("worked_example.txt")
    K = int(ex["K"])
    # a global scale g whose decode factor g/2688 is float32 0.1 up to one ulp
    g = float(np.float32(ex["global_factor"] * 2688.0))
    codes = np.full((1, K // 2), 0x77, np.uint8)  # every element e2m1 code 7 (= 6)
    scales = np.full((1, K // 16), 0x30, np.uint8)  # e4m3 0.5
    assert O.e2m1_value(7) == ex["q"] and O.e4m3_value(0x30) == ex["block_scale"]

    w_with = O.dequantize(codes, scales, global_scale=g, dtype="bf16")
    w_without = O.dequantize(codes, scales, global_scale=None, dtype="bf16")
    assert np.all(w_with == ex["w_with_global"])
    assert np.all(w_without == ex["w_without_global"])

    # ones @ W with bfloat16 weights and float32 sums
    inside = np.float32(0.0)
    for v in w_with[0]:
        inside = np.float32(inside + np.float32(v))
    after_mm = np.float32(0.0)
    for v in w_without[0]:
        after_mm = np.float32(after_mm + np.float32(v))
    after = np.float32(after_mm * np.float32(ex["global_factor"]))
    assert float(inside) == ex["scale_inside"]
    assert float(after) == ex["scale_after"]
    assert float(after - inside) == ex["difference"]

    # the oracle's qmv with x = ones (g_x = amax(x) = 1 reproduces x exactly)
    x = np.ones((1, K), np.float32)
    assert np.array_equal(O.quant_dequant(x, global_scale=1.0, dtype="bf16"), x)
    y = O.qqmm(x, codes, scales, global_scale_x=1.0, global_scale_w=g, dtype="bf16")
    assert y[0, 0] == ex["scale_inside"]
    # with a float32 output the float32 contraction keeps g inside the weights:
    # 4096 * float32(6 * float32(0.5 * dec)) summed exactly
    y32 = O.qqmm(x, codes, scales, global_scale_x=1.0, global_scale_w=g, dtype="f32")
    dec = np.float32(np.float32(g) / np.float32(2688.0))
    assert y32[0, 0] == np.float32(K * float(np.float32(6.0 * np.float32(0.5 * dec))))


# ------------------------------------------------------------- grid cases A-D

def _case(name):
    c = W.grid_case(name)
    spec = read_cases()[name]
    assert c["g_x"] == spec["gx"] and c["g_w"] == spec["gw"] and c["dtype"] == spec["dtype"]
    return c, spec


def _exact_product(x, w, dtype):
    y = x.astype(np.float64) @ w.astype(np.float64).T
    return np.array([[O.round_to(float(v), dtype) for v in row] for row in y], np.float32)


@pytest.mark.parametrize("name", ["A", "B", "C", "D"])
def test_grid_case_scales_roundtrip_and_exact_product(name):
    c, spec = _case(name)
    x, w, dt = f32np(c["x"]), f32np(c["w"]), c["dtype"]
    wc, ws = O.quantize(w, c["g_w"])
    # w's block scales are the value the page names for the case
    assert np.all(ws == O.e4m3_encode(spec["wscale"]))
    assert O.e4m3_value(ws[0, 0]) == spec["wscale"]
    # and w decodes back exactly, with the page's decode factor
    assert np.array_equal(O.dequantize(wc, ws, c["g_w"], dt), w)
    if c["g_w"] is not None:
        assert np.float32(c["g_w"]) / np.float32(2688.0) == np.float32(spec["wdec"])
    # x's round trip is exact (its block scales are 1.0)
    xc, xs = O.quantize(x, c["g_x"])
    assert np.all(xs == 0x38)
    assert np.array_equal(O.quant_dequant(x, c["g_x"], dt), x)
    # the product equals a plain fp64 triple loop of the raw operands
    y = O.qqmm(x, wc, ws, c["g_x"], c["g_w"], dtype=dt)
    ref = _exact_product(x, w, dt)
    assert np.array_equal(y, ref)
    assert np.all(np.isfinite(y))


def test_case_b_needs_the_activation_global_scale():
    # "Without g_x the block scales of x, 2^-12, round to 0 in e4m3"
    c, _ = _case("B")
    x = f32np(c["x"])
    _, xs = O.quantize(x, None)
    assert np.all(xs == 0)
    assert np.all(O.quant_dequant(x, None, "f32") == 0)


def test_mutant_drop_gw_fails_case_a_by_the_pages_factor():
    c, spec = _case("A")
    x, w = f32np(c["x"]), f32np(c["w"])
    wc, ws = O.quantize(w, c["g_w"])
    good = O.qqmm(x, wc, ws, c["g_x"], c["g_w"], dtype="f32")
    with O.mutant(O.MUT_DROP_GW):
        bad = O.qqmm(x, wc, ws, c["g_x"], c["g_w"], dtype="f32")
    assert np.array_equal(bad, good * spec["factor"])
    assert not np.array_equal(bad, _exact_product(x, w, "f32"))


def test_mutant_drop_gx_zeroes_case_b():
    c, _ = _case("B")
    x, w = f32np(c["x"]), f32np(c["w"])
    wc, ws = O.quantize(w, c["g_w"])
    with O.mutant(O.MUT_DROP_GX):
        bad = O.qqmm(x, wc, ws, c["g_x"], c["g_w"], dtype="f32")
    assert np.all(bad == 0)
    assert not np.array_equal(bad, _exact_product(x, w, "f32"))


def test_mutant_gw_on_fp16_sum_overflows_case_d():
    c, spec = _case("D")
    x, w = f32np(c["x"]), f32np(c["w"])
    wc, ws = O.quantize(w, c["g_w"])
    ref = _exact_product(x, w, "f16")
    assert np.abs(ref).max() * spec["factor"] > 65504.0  # the page's overflow condition
    with O.mutant(O.MUT_GW_ON_SUM):
        bad = O.qqmm(x, wc, ws, c["g_x"], c["g_w"], dtype="f16")
    assert np.isinf(bad).any()
    good = O.qqmm(x, wc, ws, c["g_x"], c["g_w"], dtype="f16")
    assert np.array_equal(good, ref)


# ------------------------------------------------------------- round trip

@pytest.mark.parametrize("c_exp,enc_exp", [(0, 0), (-12, 12), (3, -3), (-5, 0), (4, 2), (-9, 0)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_round_trip_exact_on_scaled_grid(c_exp, enc_exp, dtype):
    """x = c * grid with +-6c in every group, enc = 2688/g = 2^enc_exp with
    c*enc in [2^-9, 2^8]: every step is exact, so x_hat == x and qqmm equals
    the plain fp64 product of the raw operands."""
    c = 2.0 ** c_exp
    g = 2688.0 / 2.0 ** enc_exp
    assert -9 <= c_exp + enc_exp <= 8
    x = W.grid_tensor(3, 64, seed=100 + c_exp).numpy() * c
    w = W.grid_tensor(5, 64, seed=200 + enc_exp).numpy() * c
    assert np.array_equal(O.quant_dequant(x, g, dtype), x)
    wc, ws = O.quantize(w, g)
    assert np.array_equal(O.dequantize(wc, ws, g, "f32"), w)
    # scale byte is c*enc exactly
    assert np.all(np.array([O.e4m3_value(s) for s in ws.ravel()]) == c * 2.0 ** enc_exp)
    y = O.qqmm(x, wc, ws, g, g, dtype=dtype)
    assert np.array_equal(y, _exact_product(x, w, dtype))


def test_nibble_order_low_nibble_is_even_element():
    x = np.zeros((1, 16), np.float32)
    x[0, 0], x[0, 1] = 6.0, -0.5  # codes 7 and 9
    codes, scales = O.quantize(x, None)
    assert codes[0, 0] == (7 | (9 << 4))
    # byte 1 holds elements 2 and 3 (both +0)
    assert codes[0, 1] == 0


def test_zero_scale_block_gives_signed_zeros():
    x = np.zeros((1, 32), np.float32)
    x[0, 16:] = -0.0
    x[0, 5] = 1e-30  # far below the smallest e4m3 scale
    codes, scales = O.quantize(x, None)
    assert np.all(scales == 0)
    assert codes[0, 2] == 0x00 and np.all(codes[0, 8:] == 0x88)
    xh = O.quant_dequant(x, None, "f32")
    assert np.all(xh == 0)
    assert np.all(np.signbit(xh[0, 16:]))


# ------------------------------------------------------------- general data

def _cfg2_like(rows=64, k=512, seed=7):
    return W.normal((rows, k), 0.02, seed, "bf16", outlier_frac=0.001, outlier_mult=50.0)


def test_invariants_on_outlier_weights():
    w = f32np(_cfg2_like(256, 1024))
    g = O.tensor_amax(w)
    assert g == float(np.abs(w).max())
    codes, scales = O.quantize(w, g)
    # (1) the block holding the tensor amax has the largest scale byte 0x7E
    r, col = np.unravel_index(np.argmax(np.abs(w)), w.shape)
    assert scales[r, col // 16] == 0x7E and scales.max() == 0x7E
    # (2) never the NaN byte and never a sign bit
    assert not np.any(scales == 0x7F) and not np.any(scales & 0x80)
    # (3) in blocks with scale >= 2^-6 the block maximum encodes to +-6
    lo = codes & 15
    hi = codes >> 4
    q = np.empty(w.shape, np.uint8)
    q[:, 0::2], q[:, 1::2] = lo, hi
    blocks = np.abs(w).reshape(w.shape[0], -1, 16)
    amax_b = blocks.max(axis=2, keepdims=True)
    sf = np.vectorize(O.e4m3_value)(scales)
    is_max = (blocks == amax_b) & (sf[:, :, None] >= 2.0 ** -6)
    qb = q.reshape(w.shape[0], -1, 16)
    assert np.all((qb[is_max] & 7) == 7)


def _exact_nearest_e4m3_index(v):
    # nearest e4m3 magnitude to an exact rational v (no ties expected)
    vals = [Fraction(O.e4m3_value(b)) for b in range(0x7F)]
    if v >= vals[-1]:
        return 0x7E
    best = min(range(0x7F), key=lambda b: abs(vals[b] - v))
    return best


def test_block_scales_are_nearest_to_exact_real_scale():
    """With exact rational arithmetic, the decode scale of a block is
    amax_b / 6 * 2688 / g.  The oracle computes it in float32 (two roundings,
    relative error < 2^-23), so its e4m3 byte is the nearest to the real value
    unless that value sits within 2^-21 (relative) of a rounding midpoint.
    A bfloat16 intermediate (relative error up to 2^-9) breaks this."""
    w = f32np(_cfg2_like(128, 512, seed=9))
    g = O.tensor_amax(w)
    vals = [Fraction(O.e4m3_value(b)) for b in range(0x7F)]
    mids = [(a + b) / 2 for a, b in zip(vals, vals[1:])]

    def near_mid(v):
        return any(abs(v - m) <= abs(m) * Fraction(1, 2 ** 21) for m in mids)

    def check(scales):
        bad = 0
        blocks = np.abs(w).reshape(w.shape[0], -1, 16).max(axis=2)
        enc = Fraction(2688) / Fraction(float(np.float32(g)))
        for (r, b), amax in np.ndenumerate(blocks):
            v = Fraction(float(amax)) / 6 * enc
            if near_mid(v):
                continue
            if scales[r, b] != _exact_nearest_e4m3_index(v):
                bad += 1
        return bad

    _, scales = O.quantize(w, g)
    assert check(scales) == 0
    with O.mutant(O.MUT_AMAX6_BF16):
        _, bad_scales = O.quantize(w, g)
    assert check(bad_scales) > 0


def _error_bound_ok(x, g, dtype):
    """|x - x_hat| <= max(1, y_max - 6) * sf * dec * (1 + 2^-20) + ulp_T(x_hat)/2
    per element, y_max = amax_b * enc / sf the largest scaled value of its
    block: half a grid step of e2m1 (at most 1, between 4 and 6) inside the
    range, the clipped excess above 6, scaled back by the block scale."""
    xh = O.quant_dequant(x, g, dtype)
    _, scales = O.quantize(x, g)
    enc = 2688.0 / g if g is not None else 1.0
    dec = g / 2688.0 if g is not None else 1.0
    sf = np.vectorize(O.e4m3_value)(scales).repeat(16, axis=1)
    amax_b = np.abs(x).reshape(x.shape[0], -1, 16).max(axis=2).repeat(16, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        ymax = np.where(sf > 0, amax_b * enc / sf, 0.0)
    step = np.maximum(1.0, ymax - 6.0) * sf * dec * (1 + 2.0 ** -20)
    if dtype == "bf16":
        ulp = np.abs(xh) * 2.0 ** -7
    elif dtype == "f16":
        ulp = np.maximum(np.abs(xh) * 2.0 ** -10, 2.0 ** -24)
    else:
        ulp = np.abs(xh) * 2.0 ** -23
    err = np.abs(x.astype(np.float64) - xh)
    zero_block = sf == 0
    ok = (err <= step + ulp / 2) | (zero_block & (np.abs(x) <= 2.0 ** -10 * dec * 6))
    return ok.all(), err, step


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_round_trip_error_bound_general(dtype):
    x = f32np(W.normal((64, 1024), 1.0, 21, dtype))
    g = O.tensor_amax(x)
    ok, _, _ = _error_bound_ok(x, g, dtype)
    assert ok
    ok, _, _ = _error_bound_ok(x, None, dtype)
    assert ok


def test_error_bound_catches_dropped_global_factor():
    x = f32np(W.normal((16, 256), 1.0, 22, "f32")) * 1e-3
    g = O.tensor_amax(x)
    xh_good = O.quant_dequant(x, g, "f32")
    with O.mutant(O.MUT_DROP_GX):
        # the x round trip ignoring g: compare through qqmm with an identity-ish w
        w = np.eye(256, dtype=np.float32)[:32] * 6
        wc, ws = O.quantize(w, None)
        bad = O.qqmm(x, wc, ws, g, 2688.0, dtype="f32")
    good = O.qqmm(x, wc, ws, g, 2688.0, dtype="f32")
    assert np.allclose(good, xh_good[:, :32] * 6, rtol=0, atol=0)
    assert not np.allclose(bad, good, rtol=1e-2)


def test_encode_order_reading_changes_only_near_ties():
    """Reading: x * (enc / sf) (the CUDA rowwise kernel's order).  The
    alternative (x * enc) / sf changes a few codes, all of them for values
    within a few float32 ulps of an e2m1 midpoint; no pin on the pages decides
    between them (recorded as a reading)."""
    w = f32np(W.normal((1024, 1024), 1.0, 6, "bf16"))
    g = O.tensor_amax(w)
    c0, s0 = O.quantize(w, g)
    with O.mutant(O.MUT_ENC_ORDER):
        c1, s1 = O.quantize(w, g)
    assert np.array_equal(s0, s1)
    diff = np.argwhere(c0 != c1)
    assert len(diff) > 0  # the two orders do differ on this data
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    for r, b in diff:
        for el, sh in ((2 * b, 0), (2 * b + 1, 4)):
            if ((c0[r, b] >> sh) & 15) == ((c1[r, b] >> sh) & 15):
                continue
            sf = O.e4m3_value(s0[r, el // 16])
            y = abs(float(w[r, el]) * (2688.0 / g) / sf)
            assert np.min(np.abs(y - mids) / mids) < 2.0 ** -20, (r, el, y)


def test_qqmm_general_matches_library_matmul_of_decoded_operands():
    x = f32np(W.normal((8, 256), 1.0, 31, "bf16"))
    w = f32np(W.normal((40, 256), 0.02, 32, "bf16"))
    gx, gw = O.tensor_amax(x), O.tensor_amax(w)
    wc, ws = O.quantize(w, gw)
    xh = O.quant_dequant(x, gx, "bf16")
    wh = O.dequantize(wc, ws, gw, "f32")
    ref = np.array([[O.round_to(float(v), "bf16") for v in row]
                    for row in (xh.astype(np.float64) @ wh.astype(np.float64).T)], np.float32)
    y = O.qqmm(x, wc, ws, gx, gw, dtype="bf16")
    assert np.array_equal(y, ref)
    # subsets pick the same elements
    ys = O.qqmm(x, wc, ws, gx, gw, dtype="bf16", rows=[7, 0, 3], cols=[39, 1])
    assert np.array_equal(ys, y[[7, 0, 3]][:, [39, 1]])
    # a transposed operand or a wrong nibble order is caught by the same check
    wc_swapped = ((wc & 15) << 4) | (wc >> 4)
    y_bad = O.qqmm(x, wc_swapped, ws, gx, gw, dtype="bf16")
    assert not np.array_equal(y_bad, y)


# ------------------------------------------------------------- gather_qmm / routing

def test_gather_qmm_exact_grid_per_expert_scales():
    E, T, K, N, top_k = 3, 6, 32, 5, 2
    gs = [336.0, 2688.0, 10.5]
    ws = [W.grid_tensor(N, K, seed=300 + e).numpy() for e in range(E)]
    codes = np.stack([O.quantize(ws[e], gs[e])[0] for e in range(E)])
    scales = np.stack([O.quantize(ws[e], gs[e])[1] for e in range(E)])
    x = W.grid_tensor(T, K, seed=310).numpy()
    idx = W.expert_indices(T, E, top_k, seed=311).numpy()
    assert all(len(set(r)) == top_k for r in idx)
    out = O.gather_qmm(x, codes, scales, idx, global_scale=np.array(gs).reshape(E, 1, 1),
                       dtype="f32")
    for t in range(T):
        for j in range(top_k):
            e = idx[t, j]
            ref = x[t].astype(np.float64) @ ws[e].astype(np.float64).T
            assert np.array_equal(out[t, j], ref.astype(np.float32))
    with O.mutant(O.MUT_DROP_GW):
        bad = O.gather_qmm(x, codes, scales, idx, global_scale=np.array(gs), dtype="f32")
    assert not np.array_equal(bad, out)


def test_moe_route_matches_stable_sort():
    idx = W.expert_indices(257, 8, 2, seed=9).numpy()
    offsets, perm = O.moe_route(idx, 8)
    flat = idx.reshape(-1)
    ref_perm = np.argsort(flat, kind="stable")
    assert np.array_equal(perm, ref_perm)
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=8))]))
    with pytest.raises(ValueError):
        O.moe_route(np.array([[0, 9]]), 8)


def test_tensor_amax_matches_numpy():
    x = f32np(W.normal((33, 77), 3.0, 41, "f32"))
    assert O.tensor_amax(x) == float(np.max(np.abs(x)))
    assert O.tensor_amax(np.zeros(0, np.float32)) == 0.0

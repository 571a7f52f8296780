"""Pins of the oracle's mx modes (mxfp4, mxfp8) against the format
definitions, independent library routines, closed forms and the figures the
pages print.

The modes ("mlx 0.30.7.2 -> 0.30.7.6" diff, page 8, fp_quantize and
fp_dequantize): groups of 32, e2m1 codes (mxfp4) or e4m3 codes (mxfp8), and
an E8M0 block scale decoded as 2^(s - 127); no global scale.  The E8M0 scale
rounds amax / maxval up to a power of two (the pull request referenced from
the "[Metal] global scale for qmm" page, "fix(mlx): bump MLX pin to 81ba1c6a
so mxfp8 block scales round up", sections "Why" and "Validation")."""
import math
import os

import numpy as np
import pytest
import torch

import workloads as W
from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mx_worked_example.txt")
MAXVAL = {"mxfp4": 6.0, "mxfp8": 448.0}
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _golden():
    vals = {}
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            key, v = line.split()
            vals[key] = float(v)
    return vals


def _e4m3_magnitudes():
    """All finite non-negative e4m3 values, from the format's definition:
    subnormals m/8 * 2^-6, normals (1 + m/8) * 2^(e - 7), largest 448."""
    vals = [m / 8 * 2.0 ** -6 for m in range(8)]
    vals += [(1 + m / 8) * 2.0 ** (e - 7) for e in range(1, 16) for m in range(8)]
    return sorted(v for v in vals if v <= 448.0)


def _up_by_frexp(v):
    """Smallest power of two >= v as an E8M0 byte, by frexp (v = f 2^e,
    0.5 <= f < 1): 2^(e - 1) when f == 0.5, else 2^e; clamped to 0..254."""
    if v <= 0:
        return 0
    f, e = math.frexp(v)
    p = e - 1 if f == 0.5 else e
    return min(max(p + 127, 0), 254)


# ------------------------------------------------------------------ E8M0

def test_e8m0_value_definition():
    assert O.e8m0_value(127) == 1.0
    assert O.e8m0_value(0) == 2.0 ** -127
    assert O.e8m0_value(254) == 2.0 ** 127
    assert math.isnan(O.e8m0_value(255))
    for b in range(255):
        assert O.e8m0_value(b) == math.ldexp(1.0, b - 127)


def test_e8m0_round_up_against_frexp():
    rng = np.random.default_rng(3)
    vals = list(np.exp(rng.uniform(-90, 88, 20000)).astype(np.float32))
    for e in range(-126, 127):
        p = np.float32(2.0 ** e)
        vals += [p, np.nextafter(p, np.float32(np.inf)), np.nextafter(p, np.float32(0))]
    vals += [np.float32(0.0), np.float32(2.0 ** -130), np.float32(2.0 ** -127),
             np.float32(3.0e38)]
    for v in vals:
        assert O.e8m0_encode_up(float(v)) == _up_by_frexp(float(v)), v


def test_e8m0_round_up_never_below_nearest_power():
    # torch's float8_e8m0fnu conversion rounds the significand to nearest;
    # rounding up is never below it and at most one power of two above it
    v = np.exp(np.random.default_rng(4).uniform(-60, 60, 5000)).astype(np.float32)
    near = torch.from_numpy(v).to(torch.float8_e8m0fnu).view(torch.uint8).numpy()
    up = np.array([O.e8m0_encode_up(float(a)) for a in v])
    assert ((up == near) | (up == near.astype(int) + 1)).all()
    exact = np.array([float(a) == 2.0 ** (int(b) - 127) for a, b in zip(v, near)])
    assert (up[exact] == near[exact]).all()  # powers of two convert to themselves


# ------------------------------------------------------------------ worked figures

def test_worked_example_block_max_saturates_only_under_nearest():
    """A mxfp8 block whose maximum is 4.8046875: rounding log2(amax / 448) to
    nearest gives 2^-7, which scales the maximum to 615 > 448 (saturated);
    rounding up gives 2^-6 and a scaled maximum of 307.5."""
    g = _golden()
    amax = g["block_max"]
    ratio = np.float32(amax) / np.float32(g["e4m3_max"])
    nearest = round(math.log2(ratio))
    assert amax * 2.0 ** -nearest == g["scaled_max_nearest"]
    assert g["scaled_max_nearest"] > g["e4m3_max"]
    x = np.zeros((1, 32), np.float32)
    x[0, 5] = amax
    x[0, 6] = -1.0
    codes, scales = O.mx_quantize(x, "mxfp8")
    assert scales[0, 0] == 127 - 6
    assert amax * 2.0 ** 6 <= g["e4m3_max"]
    assert O.e4m3_value(codes[0, 5]) == 320.0  # 307.5 is nearer 320 than 288
    with O.mutant(O.MUT_E8M0_NEAREST):
        codes_n, scales_n = O.mx_quantize(x, "mxfp8")
    assert scales_n[0, 0] == 127 + nearest == 120
    assert codes_n[0, 5] == 0x7E  # saturated at 448


@pytest.mark.parametrize("mode", ["mxfp4", "mxfp8"])
def test_block_scale_is_the_smallest_power_that_avoids_saturation(mode):
    """Every block: max|x| <= maxval * scale (the Validation section's bound
    for mxfp8), and max|x| > maxval * scale / 2 unless the scale is the
    smallest E8M0 value; hence no element's scaled magnitude exceeds maxval."""
    x = W.normal((64, 256), 1.0, 11, "bf16", outlier_frac=0.01, outlier_mult=40.0).float().numpy()
    x[3, 32:64] = 0.0
    codes, scales = O.mx_quantize(x, mode)
    mv = MAXVAL[mode]
    amax = np.abs(x).reshape(64, 8, 32).max(axis=2).astype(np.float64)
    sc = np.ldexp(1.0, scales.astype(np.int64) - 127)
    assert (amax <= mv * sc).all()
    tight = scales > 0
    assert (amax[tight] > mv * sc[tight] / 2).all()
    assert scales[3, 1] == 0  # an all-zero block takes the smallest scale
    with O.mutant(O.MUT_E8M0_NEAREST):
        _, scales_n = O.mx_quantize(x, mode)
    sc_n = np.ldexp(1.0, scales_n.astype(np.int64) - 127)
    assert (amax > mv * sc_n).any()  # the rejected reading saturates some blocks


# ------------------------------------------------------------------ element codes

def test_mxfp8_codes_equal_torch_e4m3fn_on_every_bf16_value():
    """Groups whose maximum is 448 get scale 2^0 (byte 127); every other
    element's code is then torch's float8_e4m3fn conversion of it (round to
    nearest even; no value exceeds 448).  All 65,536 bf16 bit patterns with
    |v| <= 448."""
    v = torch.arange(0, 65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).float()
    v = v[torch.isfinite(v) & (v.abs() <= 448)]
    pad = (-v.numel()) % 31
    v = torch.cat([v, torch.zeros(pad)]).reshape(-1, 31)
    x = torch.cat([torch.full((v.shape[0], 1), 448.0), v], dim=1).numpy()
    codes, scales = O.mx_quantize(x.reshape(1, -1), "mxfp8")
    assert (scales == 127).all()
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy().reshape(1, -1)
    assert np.array_equal(codes, ref)


def test_mxfp4_codes_nearest_grid_value_ties_to_even():
    """Groups whose maximum is 6 get scale 2^0; every other element's code is
    the nearest e2m1 grid value, ties to the even code, by brute force over
    the grid, sign kept (also for zero)."""
    rng = np.random.default_rng(5)
    mids = [(a + b) / 2 for a, b in zip(E2M1, E2M1[1:])]
    vals = np.concatenate([rng.uniform(-6, 6, 31 * 300), mids, [-m for m in mids], E2M1,
                           [-0.0, -0.2, 0.25, -0.25]]).astype(np.float32)
    vals = np.concatenate([vals, np.zeros((-vals.size) % 31, np.float32)]).reshape(-1, 31)
    x = np.concatenate([np.full((vals.shape[0], 1), 6.0, np.float32), vals], axis=1).reshape(1, -1)
    codes, scales = O.mx_quantize(x, "mxfp4")
    assert (scales == 127).all()
    nib = np.stack([codes & 15, codes >> 4], axis=-1).reshape(-1)
    for v, q in zip(x.reshape(-1), nib):
        a = abs(float(v))
        d = [abs(a - g) for g in E2M1]
        best = min(range(8), key=lambda c: (d[c], c % 2))
        sign = 8 if math.copysign(1.0, float(v)) < 0 else 0
        assert q == best | sign, (v, q)


# ------------------------------------------------------------------ round trips

def _grid_blocks(rows, k, mode, seed, exps):
    """Values on the element grid with +maxval and -maxval in every group of
    32, each group times 2^e with e from `exps` (cycled over the groups)."""
    rng = np.random.default_rng(seed)
    mags = np.array(E2M1 if mode == "mxfp4" else _e4m3_magnitudes())
    mv = MAXVAL[mode]
    x = rng.choice(mags, size=(rows, k)) * rng.choice([-1.0, 1.0], size=(rows, k))
    g = x.reshape(rows, k // 32, 32)
    for r in range(rows):
        for b in range(k // 32):
            i, j = rng.choice(32, 2, replace=False)
            g[r, b, i], g[r, b, j] = mv, -mv
            g[r, b] *= 2.0 ** exps[(r * (k // 32) + b) % len(exps)]
    return g.reshape(rows, k).astype(np.float32)


@pytest.mark.parametrize("mode", ["mxfp4", "mxfp8"])
def test_round_trip_exact_on_grid_blocks(mode):
    exps = [-20, -3, 0, 5, 17]
    x = _grid_blocks(6, 160, mode, 6, exps)
    codes, scales = O.mx_quantize(x, mode)
    want = np.array([127 + exps[i % len(exps)] for i in range(6 * 5)]).reshape(6, 5)
    assert np.array_equal(scales, want)
    np.testing.assert_array_equal(O.mx_dequantize(codes, scales, mode, "f32"), x)
    np.testing.assert_array_equal(O.mx_quant_dequant(x, mode, "f32"), x)
    np.testing.assert_array_equal(O.mx_quant_dequant(x, mode, "bf16"), x)  # <= 4 significant bits


@pytest.mark.parametrize("mode", ["mxfp4", "mxfp8"])
def test_dequantize_in_f16_is_one_rounding_of_the_exact_value(mode):
    x = W.normal((8, 96), 1.0, 12, "f32").numpy() * np.float32(3e-4)
    codes, scales = O.mx_quantize(x, mode)
    exact = O.mx_dequantize(codes, scales, mode, "f32")
    got = O.mx_dequantize(codes, scales, mode, "f16")
    ref = torch.from_numpy(exact).to(torch.float16).float().numpy()
    np.testing.assert_array_equal(got, ref)


def test_code_layout_and_zero_block():
    """mxfp4: element 2j in the low nibble of byte j; an all-zero (signed)
    group gets scale byte 0 and signed-zero codes that decode to zero."""
    x = np.zeros((1, 64), np.float32)
    x[0, :32] = -0.0
    x[0, 32] = 6.0
    x[0, 33] = -3.0
    codes, scales = O.mx_quantize(x, "mxfp4")
    assert scales[0, 0] == 0 and scales[0, 1] == 127
    assert (codes[0, :16] == 0x88).all()
    assert codes[0, 16] == (0x7 | (0xD << 4))
    c8, s8 = O.mx_quantize(x, "mxfp8")
    assert c8.shape == (1, 64) and (c8[0, :32] == 0x80).all() and s8[0, 0] == 0
    assert (O.mx_dequantize(codes, scales, "mxfp4", "f32")[0, :32] == 0).all()


# ------------------------------------------------------------------ qqmm

@pytest.mark.parametrize("mode", ["mxfp4", "mxfp8"])
def test_qqmm_exact_on_grid_operands(mode):
    """Grid operands round-trip exactly, so the mx qqmm is the float64
    product of the raw operands rounded once to the output type."""
    x = _grid_blocks(8, 128, mode, 7, [-9, 0, 4])
    w = _grid_blocks(24, 128, mode, 8, [-2, 3, 1, 0])
    wc, ws = O.mx_quantize(w, mode)
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    for dt in ("f32", "bf16"):
        ref = np.array([[O.round_to(float(v), dt) for v in row] for row in exact], np.float32)
        np.testing.assert_array_equal(O.mx_qqmm(x, wc, ws, mode, dtype=dt), ref)


@pytest.mark.parametrize("mode", ["mxfp4", "mxfp8"])
def test_qqmm_general_is_the_product_of_the_round_trips(mode):
    """On general data: the product of the two float32 round trips (within
    float64 summation), columns and rows subsets consistent with the whole,
    and the mx quantization error of the product small."""
    x = W.normal((16, 256), 1.0, 13, "bf16").float().numpy()
    w = W.normal((40, 256), 0.02, 14, "bf16").float().numpy()
    wc, ws = O.mx_quantize(w, mode)
    y = O.mx_qqmm(x, wc, ws, mode, dtype="f32")
    xh = O.mx_quant_dequant(x, mode, "f32")
    wh = O.mx_dequantize(wc, ws, mode, "f32")
    np.testing.assert_allclose(y, (xh.astype(np.float64) @ wh.astype(np.float64).T), rtol=1e-6,
                               atol=1e-6)
    sub = O.mx_qqmm(x, wc, ws, mode, dtype="f32", rows=[3, 9], cols=[0, 7, 39])
    np.testing.assert_array_equal(sub, y[[3, 9]][:, [0, 7, 39]])
    full = x.astype(np.float64) @ w.astype(np.float64).T
    rel = np.linalg.norm(y - full) / np.linalg.norm(full)
    assert rel < (0.25 if mode == "mxfp4" else 0.06)  # sanity: two 4- or 8-bit round trips


@pytest.mark.parametrize("mode", ["mxfp4", "mxfp8"])
def test_round_trip_error_within_half_a_grid_step(mode):
    """|x - x_hat| <= half the element grid's step at |x| / scale, times the
    scale: e2m1 steps 0.5 below 2, 1 in [2, 4), 2 in [4, 6]; e4m3 steps
    2^(floor(log2 y) - 3) for y >= 2^-6 and 2^-9 below."""
    x = W.normal((32, 512), 1.0, 15, "bf16", outlier_frac=0.01, outlier_mult=30.0).float().numpy()
    codes, scales = O.mx_quantize(x, mode)
    xh = O.mx_dequantize(codes, scales, mode, "f32").astype(np.float64)
    sc = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=1)
    y = np.abs(x) / sc
    if mode == "mxfp4":
        step = np.where(y < 2, 0.5, np.where(y < 4, 1.0, 2.0))
    else:
        step = np.where(y >= 2.0 ** -6, np.ldexp(1.0, np.floor(np.log2(np.maximum(y, 1e-30))).astype(int) - 3),
                        2.0 ** -9)
    assert (np.abs(x - xh) <= step / 2 * sc).all()
    assert (y <= MAXVAL[mode]).all()


# ------------------------------------------------------------------ gather_qmm

def _decode_independently(codes, scales, mode):
    """w_hat from the format definitions, not through the oracle: e2m1 by its
    value table (sign in bit 3, element 2j in the low nibble of byte j), e4m3
    through torch's float8_e4m3fn, times 2^(s - 127) by ldexp."""
    codes = np.asarray(codes, np.uint8)
    if mode == "mxfp4":
        nib = np.stack([codes & 15, codes >> 4], axis=-1).reshape(*codes.shape[:-1], -1)
        mag = np.array(E2M1, np.float64)[nib & 7]
        vals = np.where(nib & 8, -mag, mag)
    else:
        vals = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    s = np.repeat(np.asarray(scales, np.int64), 32, axis=-1)
    return np.ldexp(vals, s - 127)


def _gather_exact(x, ws, idx, dtype):
    y = np.stack([[x[t].astype(np.float64) @ ws[e].astype(np.float64).T for e in row]
                  for t, row in enumerate(idx)])
    return np.array([[[O.round_to(float(v), dtype) for v in r] for r in p] for p in y], np.float32)


@pytest.mark.parametrize("mode", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_gather_qmm_exact_on_grid_experts(mode, dtype):
    """Three experts of grid blocks (each group of 32 exactly representable,
    a different power of two per expert and group), x on the e2m1 grid: every
    product is exact in float64, so each (t, j) row is the product with the
    raw weights of expert idx[t, j] rounded once.  A wrong expert, layout or
    block scale changes the bits."""
    e_count, n, k = 3, 40, 96
    ws = [_grid_blocks(n, k, mode, 30 + e, [3 * e - 4, e, -e]) for e in range(e_count)]
    codes, scales = zip(*(O.mx_quantize(w, mode) for w in ws))
    codes, scales = np.stack(codes), np.stack(scales)
    x = W.grid_tensor(7, k, seed=33).numpy()
    idx = np.random.default_rng(34).integers(0, e_count, (7, 2)).astype(np.int32)
    got = O.mx_gather_qmm(x, codes, scales, idx, mode, dtype=dtype)
    np.testing.assert_array_equal(got, _gather_exact(x, ws, idx, dtype))
    swapped = O.mx_gather_qmm(x, codes[::-1].copy(), scales[::-1].copy(), idx, mode, dtype=dtype)
    assert not np.array_equal(swapped, got)


@pytest.mark.parametrize("mode", ["mxfp4", "mxfp8"])
def test_gather_qmm_general_against_an_independent_decode(mode):
    """General data: the float64 product with weights decoded from the format
    definitions (sum order only), subsets consistent with the whole, and a
    pair whose expert is out of range gives a zero row."""
    e_count, n, k = 4, 24, 128
    w = W.normal((e_count * n, k), 0.02, 40, "bf16").float().numpy()
    codes, scales = O.mx_quantize(w, mode)
    codes = codes.reshape(e_count, n, -1)
    scales = scales.reshape(e_count, n, -1)
    x = W.normal((5, k), 1.0, 41, "bf16").float().numpy()
    idx = np.array([[0, 3], [2, 2], [1, 0], [3, 1], [2, 0]], np.int32)
    got = O.mx_gather_qmm(x, codes, scales, idx, mode, dtype="f32")
    wh = _decode_independently(codes, scales, mode)
    want = np.stack([[x[t].astype(np.float64) @ wh[e].T for e in row] for t, row in enumerate(idx)])
    np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-9)
    sub = O.mx_gather_qmm(x, codes, scales, idx, mode, dtype="f32", pairs=[(4, 1), (1, 0)],
                          cols=[23, 0, 5])
    np.testing.assert_array_equal(sub, got[[4, 1], [1, 0]][:, [23, 0, 5]])
    bad = idx.copy()
    bad[2, 1] = e_count
    y = O.mx_gather_qmm(x, codes, scales, bad, mode, dtype="f32")
    assert (y[2, 1] == 0).all()
    np.testing.assert_array_equal(np.delete(y.reshape(10, n), 5, 0), np.delete(got.reshape(10, n), 5, 0))

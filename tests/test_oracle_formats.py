"""Pins of the oracle's number formats against the format definitions and
independent library routines (CPU only).

e2m1 and e4m3 are the OCP formats the pages name through their constants
F4E2M1_MAX = 6 and F8E4M3_MAX = 448 ("mlx 0.30.7.2 -> 0.30.7.6" diff, page 7,
fp_quantize.cu); the configs list the e2m1 grid {0, +-0.5, +-1, +-1.5, +-2,
+-3, +-4, +-6}.
"""
import math
import struct

import numpy as np
import pytest
import torch

import oracle as O

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def f32(v):
    return struct.unpack("<f", struct.pack("<f", v))[0]


def next_up(v):
    return float(np.nextafter(np.float32(v), np.float32(np.inf)))


def next_down(v):
    return float(np.nextafter(np.float32(v), np.float32(-np.inf)))


# ------------------------------------------------------------------ e2m1

def test_e2m1_decode_is_the_grid():
    vals = [O.e2m1_value(c) for c in range(16)]
    assert vals[:8] == GRID
    assert vals[8:] == [-v for v in GRID]
    assert math.copysign(1.0, vals[8]) == -1.0  # code 0x8 is -0
    assert max(vals) == 6.0  # F4E2M1_MAX


def test_e2m1_encode_decode_identity():
    for c in range(16):
        v = O.e2m1_value(c)
        assert O.e2m1_encode(v) == c, (c, v)


def test_e2m1_midpoints_go_to_even_code_and_neighbours_split():
    for c in range(7):
        lo, hi = GRID[c], GRID[c + 1]
        mid = (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        for s in (1.0, -1.0):
            sign = 8 if s < 0 else 0
            assert O.e2m1_encode(s * mid) == even | sign, (mid, s)
            assert O.e2m1_encode(s * next_down(mid)) == c | sign
            assert O.e2m1_encode(s * next_up(mid)) == (c + 1) | sign


def test_e2m1_saturates_and_keeps_sign_of_zero():
    for v in (6.0, next_up(6.0), 7.0, 1e30, math.inf):
        assert O.e2m1_encode(v) == 7
        assert O.e2m1_encode(-v) == 15
    assert O.e2m1_encode(0.0) == 0
    assert O.e2m1_encode(-0.0) == 8
    assert O.e2m1_encode(-0.1) == 8
    assert O.e2m1_encode(0.25) == 0 and O.e2m1_encode(-0.25) == 8
    assert O.e2m1_encode(5.0) == 6  # tie between 4 and 6 goes to the even code


def _generic_round_saturate(v, p, emin, emax, vmax):
    r = O.round_ieee(v, p, emin, emax)
    if abs(r) > vmax:
        r = math.copysign(vmax, v)
    return r


def test_e2m1_encoder_agrees_with_generic_ieee_rounding():
    # the exhaustive nearest-value search against an IEEE-style rounding of a
    # 1-bit-fraction format (emin 0, emax 2) with saturation at 6
    rng = np.random.default_rng(0)
    vals = list(rng.uniform(-8, 8, 20000).astype(np.float32)) + \
        list((rng.standard_normal(5000) * 2).astype(np.float32))
    for v in vals:
        v = float(v)
        r = _generic_round_saturate(v, 1, 0, 2, 6.0)
        assert O.e2m1_value(O.e2m1_encode(v)) == r, v


# ------------------------------------------------------------------ e4m3

def test_e4m3_decode_definition_spot_values():
    spots = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x30: 0.5,
             0x38: 1.0, 0x50: 8.0, 0x78: 256.0, 0x7E: 448.0, 0x40: 2.0, 0x3C: 1.5}
    for b, v in spots.items():
        assert O.e4m3_value(b) == v, hex(b)
        assert O.e4m3_value(b | 0x80) == -v
    assert math.isnan(O.e4m3_value(0x7F)) and math.isnan(O.e4m3_value(0xFF))


def test_e4m3_all_bytes_monotone_and_distinct():
    vals = [O.e4m3_value(b) for b in range(0x7F)]
    assert all(b > a for a, b in zip(vals, vals[1:]))
    assert vals[-1] == 448.0  # F8E4M3_MAX
    neg = [O.e4m3_value(b | 0x80) for b in range(0x7F)]
    assert neg == [-v for v in vals]


def test_e4m3_encode_decode_identity():
    for b in range(0x7F):
        assert O.e4m3_encode(O.e4m3_value(b)) == b, hex(b)


def test_e4m3_midpoints_ties_to_even_byte():
    for b in range(0x7E):
        lo, hi = O.e4m3_value(b), O.e4m3_value(b + 1)
        mid = (lo + hi) / 2  # exact in float32 for every pair
        assert f32(mid) == mid
        even = b if b % 2 == 0 else b + 1
        assert O.e4m3_encode(mid) == even, hex(b)
        assert O.e4m3_encode(next_down(mid)) == b
        assert O.e4m3_encode(next_up(mid)) == b + 1


def test_e4m3_saturation_and_underflow():
    for v in (448.0, 450.0, 464.0, 480.0, 1e6, math.inf):
        assert O.e4m3_encode(v) == 0x7E
    assert O.e4m3_encode(2.0 ** -10) == 0x00  # tie between 0 and 2^-9: even byte 0
    assert O.e4m3_encode(next_up(2.0 ** -10)) == 0x01
    assert O.e4m3_encode(2.0 ** -12) == 0x00
    assert O.e4m3_encode(0.0) == 0x00
    # the encoder never produces the NaN byte
    for v in np.linspace(0, 2000, 4001):
        assert O.e4m3_encode(float(v)) != 0x7F


def test_e4m3_encoder_agrees_with_generic_ieee_rounding():
    rng = np.random.default_rng(1)
    vals = np.concatenate([np.exp(rng.uniform(math.log(1e-4), math.log(600), 20000)),
                           rng.uniform(0, 0.02, 2000)]).astype(np.float32)
    for v in vals:
        v = float(v)
        r = _generic_round_saturate(v, 3, -6, 8, 448.0)
        assert O.e4m3_value(O.e4m3_encode(v)) == r, v


# ------------------------------------------------------------------ T rounding

def _all_kinds_of_f32(n, seed):
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 2 ** 32, n, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    extra = np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e-8, 6e-8, 3.0e38, -3.4e38,
                      2.0 ** -133, 2.0 ** -126, 0.30000001], np.float32)
    return np.concatenate([v, extra, (rng.standard_normal(20000) * 100).astype(np.float32)])


@pytest.mark.parametrize("dtype,tdt", [("bf16", torch.bfloat16), ("f16", torch.float16)])
def test_round_to_matches_torch_conversion(dtype, tdt):
    v = _all_kinds_of_f32(60000, 2)
    ref = torch.from_numpy(v).to(tdt).to(torch.float32).numpy()
    got = np.array([O.round_to(float(a), dtype) for a in v], np.float32)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), v[~same][:10]
    # signs of zero too
    assert np.array_equal(np.signbit(got[got == 0]), np.signbit(ref[ref == 0]))

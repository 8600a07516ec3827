"""Pins for oracle.mxfp4 (E2M1 codes, UE8M0 scales, the block-32 quantizer).

Nothing here re-types the oracle's formulas: the E2M1 values come from the
OCP MX bit-field definition, the quantizer is checked by brute force over
every bfloat16 pattern and over all 16 candidate codes, and a few groups are
worked by hand.
"""
import math

import numpy as np
import pytest

from oracle import mxfp4


def ocp_e2m1_value(c):
    # OCP MX v1.0 E2M1: sign bit 3, exponent bits 2..1 with bias 1, mantissa bit 0;
    # exponent field 0 is subnormal (0.m x 2^0).
    s, ex, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
    mag = m * 0.5 if ex == 0 else 2.0 ** (ex - 1) * (1 + m / 2)
    return -mag if s else mag


def test_e2m1_table_matches_bit_fields():
    for c in range(16):
        assert mxfp4.e2m1_decode(c) == ocp_e2m1_value(c), c
    assert sorted({abs(ocp_e2m1_value(c)) for c in range(16)}) == list(mxfp4.E2M1_MAGNITUDES)


def test_ue8m0_values():
    for b in range(255):
        assert mxfp4.ue8m0_decode(b) == math.ldexp(1.0, b - 127)
    assert np.isnan(mxfp4.ue8m0_decode(255))


def brute_code(v, e):
    """Best of the 16 codes for value v under scale 2^e: min distance, then even
    mantissa, then a sign that matches v (decides +0 / -0)."""
    best = None
    for c in range(16):
        d = abs(v - ocp_e2m1_value(c) * 2.0 ** e)
        key = (d, c & 1, int(((c >> 3) & 1) != int(math.copysign(1.0, v) < 0)))
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def check_scale_invariants(amax, sbyte):
    e = int(sbyte) - 127
    assert -127 <= e <= 127
    if amax == 0:
        assert e == -127
        return
    assert amax <= 6.0 * 2.0 ** e
    assert e == -127 or amax > 6.0 * 2.0 ** (e - 1)


def all_finite_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    keep = np.isfinite(f)
    return f[keep].astype(np.float64)


def test_every_bf16_as_lone_value():
    vals = all_finite_bf16()
    grp = np.zeros((vals.size, 32))
    grp[:, 0] = vals
    codes, scales = mxfp4.quantize(grp)
    assert np.all(codes[:, 1:] == 0)                     # +0 stays code 0
    # scale invariants for all
    e = scales[:, 0].astype(np.int64) - 127
    a = np.abs(vals)
    nz = a > 0
    assert np.all(scales[~nz, 0] == 0)
    assert np.all(a[nz] <= np.ldexp(6.0, e[nz]))
    assert np.all((e[nz] == -127) | (a[nz] > np.ldexp(6.0, e[nz] - 1)))
    # code = brute force over the 16 candidates (vectorised form of brute_code)
    cand = np.array([ocp_e2m1_value(c) for c in range(16)])
    approx = cand[None, :] * np.ldexp(1.0, e)[:, None]
    d = np.abs(vals[:, None] - approx)
    odd = (np.arange(16) & 1)[None, :]
    sign_mismatch = ((np.arange(16) >> 3)[None, :] != np.signbit(vals)[:, None]).astype(np.int64)
    dmin = d.min(axis=1, keepdims=True)
    key = np.where(d == dmin, odd * 2 + sign_mismatch, 99)
    expect = key.argmin(axis=1)
    assert np.array_equal(codes[:, 0], expect)
    # spot-check the vectorised brute force against the scalar one
    rng = np.random.default_rng(0)
    for i in rng.integers(0, vals.size, 300):
        assert brute_code(vals[i], int(e[i])) == expect[i]


def test_random_groups_nearest_and_invariants():
    rng = np.random.default_rng(1)
    v = rng.standard_normal((400, 32)) * np.exp(rng.uniform(-30, 30, (400, 1)))
    v[::7, 3] = -0.0
    codes, scales = mxfp4.quantize(v)
    for g in range(400):
        check_scale_invariants(np.abs(v[g]).max(), scales[g, 0])
        e = int(scales[g, 0]) - 127
        for i in range(0, 32, 5):
            assert codes[g, i] == brute_code(v[g, i], e)


def test_hand_worked_groups():
    # amax 3 -> e = -1 (6*2^-1 = 3 >= 3 > 6*2^-2).  Scaled values 6, 1.5, 0.5, -2.5,
    # 0.25, -0.75, 5 give: 6.0 -> 7; 1.5 -> 3; 0.5 -> 1; -2.5 ties 2|3 -> 2.0, negative
    # -> 0xC; 0.25 ties 0|0.5 -> 0; -0.75 ties 0.5|1 -> 1.0, negative -> 0xA;
    # 5 ties 4|6 -> 4.0 -> 6.
    v = np.zeros(32)
    v[:7] = [3.0, 0.75, 0.25, -1.25, 0.125, -0.375, 2.5]
    c, s = mxfp4.quantize(v)
    assert s[0] == 126
    assert list(c[:7]) == [7, 3, 1, 0xC, 0, 0xA, 6]
    # amax 7 -> e = 1 (12 >= 7 > 6); 7/2 = 3.5 ties 3|4 -> 4 (code 6); 1.75/2 = 0.875 -> 1.0 (code 2)
    v = np.zeros(32)
    v[[0, 9, 31]] = [7.0, -1.75, 0.5]
    c, s = mxfp4.quantize(v)
    assert s[0] == 128
    assert (c[0], c[9], c[31]) == (6, 0xA, 0)          # 0.5/2 = 0.25 tie 0|0.5 -> 0
    # all zeros, and a negative zero
    v = np.zeros(32)
    v[4] = -0.0
    c, s = mxfp4.quantize(v)
    assert s[0] == 0 and c[4] == 8 and c.sum() == 8
    # tiny amax clamps to e = -127: 1.5 * 2^-130 / 2^-127 = 0.1875 -> 0, sign kept
    v = np.zeros(32)
    v[0] = -1.5 * 2.0 ** -130
    c, s = mxfp4.quantize(v)
    assert s[0] == 0 and c[0] == 8
    # m > 1.5 moves the scale up by one: amax 1.75 -> e = -1 (3 >= 1.75 > 1.5)
    v = np.zeros(32)
    v[0] = 1.75
    c, s = mxfp4.quantize(v)
    assert s[0] == 126 and c[0] == 6                  # 1.75 * 2 = 3.5 ties 3|4 -> 4.0


def test_representable_round_trip():
    rng = np.random.default_rng(2)
    for _ in range(200):
        e = int(rng.integers(-120, 120))
        mags = rng.choice(mxfp4.E2M1_MAGNITUDES, 32)
        mags[rng.integers(0, 32)] = 6.0                   # amax = 6 * 2^e exactly
        sign = rng.integers(0, 2, 32)
        v = np.where(sign == 1, -mags, mags) * 2.0 ** e
        c, s = mxfp4.quantize(v)
        assert s[0] == e + 127
        assert np.array_equal(mxfp4.e2m1_decode(c) * 2.0 ** e, v)


def test_dequantize_is_idempotent():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((300, 64)) * np.exp(rng.uniform(-5, 5, (300, 1)))
    d1 = mxfp4.dequantize(*mxfp4.quantize_packed(v))
    d2 = mxfp4.dequantize(*mxfp4.quantize_packed(d1))
    assert np.array_equal(d1, d2)
    # and the dequantized error stays within half a grid step of the block scale
    s = mxfp4.quantize(v)[1].astype(np.int64) - 127
    step = np.repeat(np.ldexp(1.0, s), 32, axis=1)      # coarsest E2M1 spacing is 2 * 2^e
    assert np.all(np.abs(d1 - v) <= step)


def test_pack_nibble_order():
    assert list(mxfp4.pack(np.array([1, 2, 0xF, 0]))) == [0x21, 0x0F]
    rng = np.random.default_rng(4)
    c = rng.integers(0, 16, (5, 64)).astype(np.uint8)
    assert np.array_equal(mxfp4.unpack(mxfp4.pack(c)), c)


def test_scale_exponent_wide_range_fp64():
    rng = np.random.default_rng(5)
    a = np.exp(rng.uniform(-100, 100, 20000))
    e = mxfp4.scale_exponent(a)
    inside = (e > -127) & (e < 127)
    assert np.all(a[inside] <= np.ldexp(6.0, e[inside]))
    assert np.all(a[inside] > np.ldexp(6.0, e[inside] - 1))
    exact = np.ldexp(6.0, np.arange(-126, 127))          # boundaries land on the lower e
    assert np.array_equal(mxfp4.scale_exponent(exact), np.arange(-126, 127))

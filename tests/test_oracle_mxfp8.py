"""Pins for oracle.mxfp8 (E4M3 codes with UE8M0 block scales, the fp8xfp4 MMA
type's activation format) and for the fp8xfp4 forward.

Nothing here re-types the oracle's rounding: E4M3 values come from the OCP MX
bit-field definition (and a few textbook values of it), the quantizer is
checked by brute force over every bfloat16 pattern against all 254 finite
codes, ties and subnormals are built from the definition, and the forward is
compared with the dense brute force.
"""
import math

import numpy as np
import pytest

import synth
from oracle import bf16, mxfp4, mxfp8
from oracle.dense import dense_forward
from oracle.forward import forward
from tests.oracle_inputs import all_expert_weights


def ocp_e4m3_value(c):
    # OCP MX v1.0 FP8 E4M3: sign bit 7, exponent bits 6..3 with bias 7, mantissa
    # bits 2..0; exponent field 0 is subnormal (0.m x 2^-6); S.1111.111 is NaN.
    s, ex, m = (c >> 7) & 1, (c >> 3) & 15, c & 7
    if ex == 15 and m == 7:
        return math.nan
    mag = (m / 8) * 2.0 ** -6 if ex == 0 else (1 + m / 8) * 2.0 ** (ex - 7)
    return -mag if s else mag


FINITE = [c for c in range(256) if not math.isnan(ocp_e4m3_value(c))]


def test_e4m3_table_matches_bit_fields():
    for c in range(256):
        want = ocp_e4m3_value(c)
        got = float(mxfp8.e4m3_decode(c))
        assert (math.isnan(want) and math.isnan(got)) or got == want, c
    assert len(FINITE) == 254


def test_e4m3_textbook_values():
    # values the OCP E4M3 definition gives for these codes
    known = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x30: 0.5, 0x38: 1.0,
             0x3C: 1.5, 0x40: 2.0, 0x7E: 448.0, 0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, v in known.items():
        got = float(mxfp8.e4m3_decode(c))
        assert got == v and math.copysign(1, got) == math.copysign(1, v), hex(c)
    assert np.isnan(mxfp8.e4m3_decode(0x7F)) and np.isnan(mxfp8.e4m3_decode(0xFF))
    mags = mxfp8.E4M3_MAGNITUDES
    assert np.all(np.diff(mags) > 0) and mags[-1] == mxfp8.E4M3_MAX


def brute_code(v, e):
    """Best finite code for v under scale 2^e: min distance, then even
    mantissa, then a sign that matches v (decides +0 / -0)."""
    best = None
    for c in FINITE:
        d = abs(v - ocp_e4m3_value(c) * 2.0 ** e)
        key = (d, c & 1, int(((c >> 7) & 1) != int(math.copysign(1.0, v) < 0)))
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def check_scale_invariants(amax, sbyte):
    e = int(sbyte) - 127
    assert -127 <= e <= 127
    if amax == 0:
        assert e == -127
        return
    assert amax <= 448.0 * 2.0 ** e
    assert e == -127 or amax > 448.0 * 2.0 ** (e - 1)


def all_finite_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    return f[np.isfinite(f)].astype(np.float64)


def test_every_bf16_as_lone_value():
    vals = all_finite_bf16()
    groups = np.zeros((vals.size, 32))
    groups[:, 5] = vals
    codes, scales = mxfp8.quantize(groups)
    assert np.all(codes[:, [i for i in range(32) if i != 5]] == 0)
    # brute force over the 254 finite codes, vectorised over the inputs
    e = scales[:, 0].astype(np.int64) - 127
    table = np.array([ocp_e4m3_value(c) for c in FINITE])
    fin = np.array(FINITE)
    r = np.ldexp(vals, -e)
    d = np.abs(r[:, None] - table[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    # among the nearest: even mantissa first, then the sign of the input
    sign_ok = ((fin[None, :] >> 7) & 1) == np.signbit(vals)[:, None]
    score = cand * (4 + 2 * ((fin[None, :] & 1) == 0) + sign_ok)
    want = fin[score.argmax(axis=1)]
    assert np.array_equal(codes[:, 5], want)
    for i in range(0, vals.size, 997):
        assert codes[i, 5] == brute_code(vals[i], int(e[i]))
        check_scale_invariants(abs(vals[i]), scales[i, 0])


def test_random_groups_nearest_and_invariants():
    rng = np.random.default_rng(8)
    v = rng.standard_normal((300, 32)) * np.exp2(rng.integers(-40, 40, (300, 1)))
    codes, scales = mxfp8.quantize(v)
    for g in range(0, 300, 7):
        e = int(scales[g, 0]) - 127
        check_scale_invariants(np.abs(v[g]).max(), scales[g, 0])
        for i in range(32):
            assert codes[g, i] == brute_code(v[g, i], e)


def test_ties_go_to_the_even_code():
    mags = mxfp8.E4M3_MAGNITUDES
    mids = (mags[:-1] + mags[1:]) / 2          # exact in fp64
    grp = np.zeros((mids.size, 32))
    grp[:, 0] = 448.0                          # fixes e = 0
    grp[:, 1] = mids
    grp[:, 2] = -mids
    codes, scales = mxfp8.quantize(grp)
    assert np.all(scales == 127)
    lo = np.arange(mids.size)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(codes[:, 1], want)
    assert np.array_equal(codes[:, 2], want | 0x80)
    # a hair away from the midpoint decides by distance
    up, down = np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf)
    grp[:, 1], grp[:, 2] = up, down
    codes, _ = mxfp8.quantize(grp)
    assert np.array_equal(codes[:, 1], lo + 1) and np.array_equal(codes[:, 2], lo)


def test_subnormals_and_zero():
    grp = np.zeros((6, 32))
    grp[:, 0] = 448.0
    grp[0, 1] = 2.0 ** -9                      # smallest subnormal
    grp[1, 1] = 2.0 ** -10                     # half of it: tie -> 0 (even)
    grp[2, 1] = 3 * 2.0 ** -10                 # 1.5 x smallest: tie -> 2 x smallest (even)
    grp[3, 1] = 15 * 2.0 ** -10                # between 7 and 8 x 2^-9: tie -> 8 (0x08, smallest normal)
    grp[4, 1] = -0.0
    grp[5, 1] = -2.0 ** -12                    # rounds to zero, keeps the sign
    codes, _ = mxfp8.quantize(grp)
    assert list(codes[:, 1]) == [0x01, 0x00, 0x02, 0x08, 0x80, 0x80]
    codes, scales = mxfp8.quantize(np.zeros((1, 32)))
    assert np.all(codes == 0) and scales[0, 0] == 0


def test_representable_round_trip():
    rng = np.random.default_rng(9)
    for _ in range(50):
        e = int(rng.integers(-100, 100))
        c = rng.choice(FINITE, 32)
        c[int(rng.integers(32))] = 0x7E          # amax = 448 * 2^e fixes the scale
        v = np.array([ocp_e4m3_value(int(x)) for x in c]) * 2.0 ** e
        codes, scales = mxfp8.quantize(v[None])
        assert scales[0, 0] == e + 127
        assert np.array_equal(mxfp8.dequantize(codes, scales)[0], v)
        nz = v != 0
        assert np.array_equal(codes[0][nz], c[nz])


def test_scale_exponent_wide_range():
    for k in range(-140, 140):
        a = 448.0 * 2.0 ** k
        e = int(mxfp8.scale_exponent(a))
        assert e == max(-127, min(127, k))
        if -127 < k <= 127:
            assert int(mxfp8.scale_exponent(np.nextafter(a, np.inf))) == min(127, k + 1)


TINY = synth.CONFIGS[0]


def test_fp8_forward_equals_dense_brute_force():
    x = synth.make_tokens(TINY)
    ids, w = synth.make_routing(TINY)
    ids = ids.copy()
    ids[0, 1] = -1
    ids[2, 1] = ids[2, 0]                      # duplicate expert in one token
    W = all_expert_weights(TINY)
    ref = dense_forward(x, ids, w, *W, mma_type="fp8xfp4")
    got = forward(x, ids, w, W, TINY.experts, TINY.inter, mma_type="fp8xfp4")
    assert np.array_equal(got["out_f64"], ref["out_f64"])
    assert got["xq"].shape == (TINY.tokens, TINY.hidden)       # one E4M3 byte per element
    assert got["hq"].shape[1] == TINY.inter
    # the two MMA types differ only in how x and h are rounded: with the same
    # MXFP4 weights, E4M3's 4 significant bits land closer than E2M1's 2 to the
    # result with unrounded activations
    got4 = forward(x, ids, w, W, TINY.experts, TINY.inter)
    W1 = mxfp4.dequantize(W[0], W[1])
    W2 = mxfp4.dequantize(W[2], W[3])
    xv = bf16.decode(x)
    exact = np.zeros_like(got["out_f64"])
    for t in range(TINY.tokens):
        for j in range(TINY.topk):
            e = int(ids[t, j])
            if e >= 0:
                a = W1[e] @ xv[t]
                g, u = a[:TINY.inter], a[TINY.inter:]
                exact[t] += w[t, j] * (W2[e] @ (g / (1 + np.exp(-g)) * u))
    err8 = np.linalg.norm(got["out_f64"] - exact)
    err4 = np.linalg.norm(got4["out_f64"] - exact)
    assert 0 < err8 < err4 / 2


def test_fp8_zero_in_zero_out():
    x = np.zeros((TINY.tokens, TINY.hidden), dtype=np.uint16)
    ids, w = synth.make_routing(TINY)
    got = forward(x, ids, w, all_expert_weights(TINY), TINY.experts, TINY.inter, mma_type="fp8xfp4")
    assert np.all(got["xq"] == 0) and np.all(got["xsf"] == 0)
    assert np.all(got["out"] == 0) and not np.signbit(bf16.decode(got["out"])).any()

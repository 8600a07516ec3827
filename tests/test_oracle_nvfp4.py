"""Pins for oracle.nvfp4 (E2M1 codes, E4M3 scales per 16 elements, an fp32
tensor scale) and for the nvf4xnvf4 forward.

Nothing here re-types the oracle's vectorised code.  The pins are:
  - exact round trips of blocks built from representable values;
  - the NVFP4 dequantization against the MXFP4 one where the two formats
    coincide (power-of-two scales shared by both halves of a 32-block);
  - invariance under a common power-of-two factor on values and tensor scale;
  - saturation, zero and sign cases from the encoding rule;
  - the error bound that the nearest-code rule implies;
  - each block's scale and codes re-derived one element at a time in exact
    rational arithmetic (Python's Fraction), fp32 rounding included;
  - a hand-worked block (the values written out below);
  - the forward against the dense brute force on the tiny layer.
"""
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import bf16, mxfp4, mxfp8, nvfp4
from oracle.dense import dense_forward
from oracle.forward import forward
from tests.oracle_inputs import all_expert_weights_nv, nv_act_scales

E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4),
        Fraction(6)]


def e4m3_value(c):
    # OCP MX v1.0 FP8 E4M3 with the sign bit clear: exponent bits 6..3 (bias
    # 7), mantissa bits 2..0, exponent field 0 subnormal (m/8 * 2^-6)
    ex, m = (c >> 3) & 15, c & 7
    return Fraction(m, 8) * Fraction(1, 64) if ex == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (ex - 7)


E4M3 = [e4m3_value(c) for c in range(0x7F)]          # 0x7F is NaN


def f32_round(x: Fraction) -> Fraction:
    """x rounded to the nearest fp32 value, ties to the even significand (|x| < 2^128)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    q = Fraction(2) ** (max(e, -126) - 23)             # fp32 quantum at a (subnormals below 2^-126)
    n = a / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * q


def nearest(table, x, even_key):
    """Index of the table entry nearest to x; a tie goes to the entry whose even_key(index) is true."""
    best = min(range(len(table)), key=lambda i: (abs(table[i] - x), not even_key(i)))
    return best


def exact_block(v, g):
    """(scale byte, codes) of one 16-value block by the rule in oracle.nvfp4,
    every fp32 step rounded from the exact rational result."""
    vf = [Fraction(float(x)) for x in v]
    G = Fraction(float(np.float32(g)))
    amax = max(abs(x) for x in vf)
    d = f32_round(6 * G)
    sf = min(f32_round(amax / d), Fraction(448))
    s = nearest(E4M3, sf, lambda i: i % 2 == 0)
    if s == 0:
        inv = Fraction(0)
    else:
        inv = f32_round(1 / f32_round(E4M3[s] * G))
    codes = []
    for x, xv in zip(vf, v):
        q = f32_round(x * inv)
        q = max(min(q, Fraction(6)), Fraction(-6))
        m = nearest(E2M1, abs(q), lambda i: i % 2 == 0)
        neg = q < 0 or (q == 0 and np.signbit(xv))
        codes.append(m | (8 if neg else 0))
    return s, codes


def rand_blocks(rng, n, spread=20):
    v = rng.standard_normal((n, 16)) * np.exp2(rng.integers(-spread, spread, (n, 1)))
    return v.astype(np.float32).astype(np.float64)


def test_value_tables():
    assert [float(x) for x in mxfp4.E2M1_MAGNITUDES] == [float(x) for x in E2M1]
    assert np.array_equal(mxfp8.E4M3_MAGNITUDES, np.array([float(x) for x in E4M3]))
    assert float(E4M3[0x7E]) == 448.0 and float(E4M3[1]) == 2.0 ** -9


@pytest.mark.parametrize("g", [1.0, 2.0 ** -7, 3.7e-4, 0.0123, 151.25])
def test_blocks_match_exact_rational_rule(g):
    rng = np.random.default_rng(11)
    v = rand_blocks(rng, 60)
    v[0] = 0.0
    v[1, :8] = -0.0
    v[2] *= 1e6                                   # saturates the scale at 448 for small g
    v[3, 3] = -v[3, 3]
    v = v.astype(np.float32).astype(np.float64)
    codes, scales = nvfp4.quantize(v, g)
    for b in range(v.shape[0]):
        s, c = exact_block(v[b], g)
        assert scales[b, 0] == s, (b, scales[b, 0], s)
        assert list(codes[b]) == c, b


def test_representable_blocks_round_trip():
    rng = np.random.default_rng(12)
    for _ in range(200):
        g = 2.0 ** int(rng.integers(-30, 10))
        s = int(rng.integers(1, 0x7F))           # any finite nonzero E4M3 scale
        c = rng.integers(0, 16, 16).astype(np.uint8)
        c[int(rng.integers(16))] = 0x7 | (8 * int(rng.integers(2)))   # |6| fixes the block scale
        v = mxfp4.e2m1_decode(c) * float(E4M3[s]) * g
        codes, scales = nvfp4.quantize(v[None], g)
        assert scales[0, 0] == s
        nz = v != 0
        assert np.array_equal(codes[0][nz], c[nz])
        assert np.array_equal(nvfp4.dequantize(mxfp4.pack(codes), scales, g)[0], v)


def test_dequantize_agrees_with_mxfp4_where_the_formats_coincide():
    rng = np.random.default_rng(13)
    packed = rng.integers(0, 256, (40, 64)).astype(np.uint8)          # 128 elements a row
    e = rng.integers(-6, 9, (40, 4))                                   # one power of two per 32-block
    nv_scales = np.repeat(((e + 7) << 3).astype(np.uint8), 2, axis=1)  # E4M3 code of 2^e, both halves
    mx_scales = (e + 127).astype(np.uint8)
    assert np.array_equal(nvfp4.dequantize(packed, nv_scales, 1.0), mxfp4.dequantize(packed, mx_scales))


def test_power_of_two_factor_on_values_and_tensor_scale_changes_nothing():
    rng = np.random.default_rng(14)
    v = rand_blocks(rng, 300, spread=6)
    for g, k in ((0.011, 5), (0.011, -9), (2.5, 3), (1.7e-3, -20)):
        a = nvfp4.quantize(v, g)
        b = nvfp4.quantize(np.ldexp(v, k), np.float32(np.ldexp(np.float32(g), k)))
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_saturation_zero_and_sign():
    g = np.float32(0.01)
    blk = np.zeros((4, 16))
    blk[0, 0] = 6 * 448 * float(g) * 4          # four times the largest value: saturates
    blk[0, 1] = -blk[0, 0] / 2
    blk[1, 3] = -0.0                             # zero block with a negative zero
    blk[2] = -1e-30                              # scale rounds to 0: codes 0 with the sign
    blk[3, 0] = 1.0
    blk[3, 1] = -1e-9                            # tiny negative in a live block: -0 code
    blk = blk.astype(np.float32).astype(np.float64)
    codes, scales = nvfp4.quantize(blk, g)
    assert scales[0, 0] == 0x7E and codes[0, 0] == 0x7 and codes[0, 1] == 0xF
    assert scales[1, 0] == 0 and codes[1, 3] == 0x8 and np.all(codes[1, [0, 1, 2]] == 0)
    assert scales[2, 0] == 0 and np.all(codes[2] == 0x8)
    assert codes[3, 1] == 0x8 and codes[3, 0] == 0x7
    deq = nvfp4.dequantize(mxfp4.pack(codes), scales, g)
    assert deq[0, 0] == 6 * 448 * float(g) and deq[0, 1] == -deq[0, 0]


def test_error_bound_of_the_nearest_code_rule():
    # Blocks whose scale lands in E4M3's normal range without saturating: the
    # scale is within 1/16 of amax / (6g), so |q| <= 6 * 17/16 < 6.5 and each
    # element is off by at most half a gap of the E2M1 grid (1 between 4 and
    # 6), or by the clamp above 6 (< 0.5): |v - v_hat| <= e4m3(s) * g.
    rng = np.random.default_rng(15)
    g = np.float32(0.004)
    v = rand_blocks(rng, 2000, spread=3)
    codes, scales = nvfp4.quantize(v, g)
    sv = mxfp8.e4m3_decode(scales)
    ok = (sv >= 2.0 ** -6) & (sv < 448)
    assert ok.mean() > 0.9
    err = np.abs(nvfp4.dequantize(mxfp4.pack(codes), scales, g) - v)
    bound = sv[:, 0] * float(g) * (1 + 1e-6)
    assert np.all(err[ok[:, 0]] <= bound[ok[:, 0], None])
    # and never worse than one sixth of the block maximum, times 17/16
    amax = np.abs(v).max(axis=1)
    assert np.all(err[ok[:, 0]].max(axis=1) <= amax[ok[:, 0]] / 6 * 17 / 16 * (1 + 1e-6))


def test_hand_worked_block():
    # g = 1/4.  Block maximum 7.5 (element 0): sf = 7.5 / 1.5 = 5 -> E4M3 5.0
    # (exponent field 9, mantissa 2: code 0x4A).  inv = 1 / (5 * 0.25) = 0.8.
    # q = v * 0.8:  7.5 -> 6 (code 7);  1.25 -> 1.0 (code 2);  -2.5 -> -2.0
    # (code 0xC); 0.3125 -> 0.25: a tie between 0 and 0.5 goes to the even
    # code 0;  3.125 -> 2.5: a tie between 2 and 3 goes to 2 (code 4, even);
    # 4.375 -> 3.5: a tie between 3 and 4 goes to 4 (code 6, even); -0.625 ->
    # -0.5 (code 9).  fp32(0.8) is a little above 0.8, but every product
    # rounds back to the value above in fp32.
    g = 0.25
    blk = np.zeros((2, 16))
    blk[0, :7] = [7.5, 1.25, -2.5, 0.3125, 3.125, 4.375, -0.625]
    codes, scales = nvfp4.quantize(blk, g)
    assert scales[0, 0] == 0x4A
    assert list(codes[0, :7]) == [0x7, 0x2, 0xC, 0x0, 0x4, 0x6, 0x9]
    # second block: maximum f32(0.01755), sf = 0.0117 (below 2^-6, E4M3's
    # smallest normal): subnormal steps of 2^-9 = 0.001953125, and
    # 0.0117 / 0.001953125 = 5.99 -> 6 steps (code 0x06, 0.01171875)
    blk[1, 0] = float(np.float32(0.01755))
    codes, scales = nvfp4.quantize(blk, g)
    assert scales[1, 0] == 0x06


def test_tensor_scale_maps_the_maximum_to_the_largest_code():
    for amax in (1.0, 5.37, 0.113, 1e-20, 3e20):
        g = nvfp4.tensor_scale(amax)
        blk = np.zeros((1, 16))
        blk[0, 0] = np.float32(amax)
        codes, scales = nvfp4.quantize(blk, g)
        assert codes[0, 0] == 0x7
        assert scales[0, 0] == 0x7E              # 448: fp32 roundings move sf by ulps, E4M3 steps are 32


TINY = synth.CONFIGS[0]


def test_nv_forward_equals_dense_brute_force():
    x = synth.make_tokens(TINY)
    ids, w = synth.make_routing(TINY)
    ids = ids.copy()
    ids[0, 1] = -1
    ids[2, 1] = ids[2, 0]                      # duplicate expert in one token
    W, gw1, gw2 = all_expert_weights_nv(TINY)
    gx, gh = nv_act_scales(TINY, x)
    ts = (gx, gh, gw1, gw2)
    ref = dense_forward(x, ids, w, *W, mma_type="nvf4xnvf4", tensor_scales=ts)
    got = forward(x, ids, w, W, TINY.experts, TINY.inter, mma_type="nvf4xnvf4", tensor_scales=ts)
    # the dequantized values carry the fp32 tensor scales, so the two fp64
    # summation orders differ in the last bits only
    assert np.allclose(got["out_f64"], ref["out_f64"], rtol=1e-12, atol=1e-15)
    assert np.array_equal(got["out"], ref["out"])
    assert got["xsf"].shape == (TINY.tokens, TINY.hidden // 16)
    assert got["hq"].shape[1] == TINY.inter // 2 and got["hsf"].shape[1] == TINY.inter // 16
    # every requantized block is live (nonzero scale) and none saturated
    assert np.all(got["hsf"] > 0) and np.all(got["hsf"] < 0x7E)


def test_nv_forward_zero_in_zero_out():
    x = np.zeros((TINY.tokens, TINY.hidden), dtype=np.uint16)
    ids, w = synth.make_routing(TINY)
    W, gw1, gw2 = all_expert_weights_nv(TINY)
    got = forward(x, ids, w, W, TINY.experts, TINY.inter, mma_type="nvf4xnvf4",
                  tensor_scales=(0.01, 0.01, gw1, gw2))
    assert np.all(got["out"] == 0) and np.all(got["xsf"] == 0) and np.all(got["hsf"] == 0)


def test_nv_weights_are_close_to_the_fp32_weights():
    W, gw1, gw2 = all_expert_weights_nv(TINY)
    w1, w2 = synth.expert_weights_f32(TINY, 3)
    d1 = nvfp4.dequantize(W[0][3], W[1][3], gw1[3])
    d2 = nvfp4.dequantize(W[2][3], W[3][3], gw2[3])
    assert np.linalg.norm(d1 - w1) / np.linalg.norm(w1) < 0.12
    assert np.linalg.norm(d2 - w2) / np.linalg.norm(w2) < 0.12
    # and closer than MXFP4 gets with its power-of-two scale per 32
    m1 = mxfp4.dequantize(*mxfp4.quantize_packed(w1))
    assert np.linalg.norm(d1 - w1) < np.linalg.norm(m1 - w1)

"""Why NVFP4 does not run on the gfx950 block-scaled MFMA, pinned by enumeration.

The pages name an NVFP4 variant of the layer and nothing more ([P3] prhub
digest of sglang PR "bump sgl-deep-gemm to 0.1.7, MegaMoE uses the mma_type
API for MXFP4", "Motivation").  NVFP4 in its public definition stores E2M1
elements with one E4M3 scale per 16 elements (and an fp32 scale per tensor).
The block-scaled MFMA of gfx950 takes elements in E2M1, E2M3, E3M2, E4M3 or
E5M2 and one power-of-two (UE8M0) scale per 32 elements, so feeding it NVFP4
exactly would mean writing each value v * s (v an E2M1 value, s an E4M3 scale)
as one of those elements times a power of two.  The enumeration below shows
that v * s needs up to 6 significant bits, while every element format of that
MFMA holds at most 4, so no folding of the E4M3 scale into the elements is
exact; every v * s is exact in bfloat16 and in fp16, whose dense MFMAs are the
ones left.  The NVFP4 kernels (csrc/gemm_nv.hip) run on the fp16 one, with
the products e2m1 * e4m3 formed in registers (the 16-bit MFMA rate is
measured by moe_ceiling_mfma_bf16)."""
from fractions import Fraction

import numpy as np

from oracle import bf16
from oracle.mxfp4 import E2M1_MAGNITUDES
from oracle.mxfp8 import E4M3_MAGNITUDES

# significant bits (implicit leading one included) of each element format of
# the f8f6f4 MFMA: E2M1, E2M3, E3M2, E4M3, E5M2
F8F6F4_SIGNIFICAND_BITS = {"e2m1": 2, "e2m3": 4, "e3m2": 3, "e4m3": 4, "e5m2": 3}


def significant_bits(x: Fraction) -> int:
    """Bits from the leading to the trailing one of a positive dyadic rational."""
    assert x > 0 and x.denominator & (x.denominator - 1) == 0
    n = x.numerator
    while n % 2 == 0:
        n //= 2
    return n.bit_length()


def _products():
    vs = [Fraction(float(v)) for v in E2M1_MAGNITUDES if v > 0]
    ss = [Fraction(float(s)) for s in E4M3_MAGNITUDES if s > 0]
    return [(v, s, v * s) for v in vs for s in ss]


def test_the_value_sets_are_the_formats():
    # E2M1: 0.5 .. 6 in 7 positive values; E4M3 (no NaN): 126 positive values, 2^-9 .. 448
    assert sorted(float(v) for v in E2M1_MAGNITUDES if v > 0) == [0.5, 1, 1.5, 2, 3, 4, 6]
    pos = sorted(float(s) for s in E4M3_MAGNITUDES if s > 0)
    assert len(pos) == 126 and pos[0] == 2.0 ** -9 and pos[-1] == 448.0


def test_folded_nvfp4_values_need_more_bits_than_any_f8f6f4_element():
    prods = _products()
    bits = np.array([significant_bits(p) for _, _, p in prods])
    widest = max(F8F6F4_SIGNIFICAND_BITS.values())
    assert bits.max() == 6
    # e.g. 1.5 * 1.875 = 2.8125 = 0b10.1101
    assert significant_bits(Fraction(3, 2) * Fraction(15, 8)) == 6
    too_wide = {(v, s) for (v, s, _), b in zip(prods, bits) if b > widest}
    # Closed form: the odd part of v is 1 or 3 and that of s one of 1..15, so
    # v * s overflows 4 bits exactly when v is 1.5, 3 or 6 (odd part 3) and the
    # odd part of s is 7 or more (3 * 7 = 21 = 0b10101).  Scales with that odd
    # part: 5 of the 8 mantissas (1, 3, 5, 6, 7) in exponent fields 1..14, 4 in
    # field 15 (mantissa 7 there is NaN), and the subnormal 7/8 * 2^-6: 75.
    def odd(x):
        n = Fraction(x).numerator
        while n % 2 == 0:
            n //= 2
        return n
    assert too_wide == {(v, s) for v, s, _ in prods if odd(v) == 3 and odd(s) >= 7}
    assert len(too_wide) == 3 * (14 * 5 + 4 + 1) == 225


def test_every_nvfp4_value_is_exact_in_16_bit_formats():
    vals = np.array([float(p) for _, _, p in _products()])
    assert np.array_equal(bf16.decode(bf16.encode(vals)), vals)
    assert np.array_equal(vals.astype(np.float16).astype(np.float64), vals)
    assert vals.max() == 6 * 448 and vals.min() == 0.5 * 2.0 ** -9

"""MXFP8 (E4M3): FP8 E4M3 element codes with one UE8M0 scale per block of 32.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[P3] "Key source snippets", the fp8xfp4 branch of _run_mega_routed: the
activations of the fp8xfp4 MMA type are quantized to FP8 by pre_dispatch with
quant_group_size=32, and the weights stay MXFP4.  The pages name FP8 and the
per-32 grouping but not the element format; the reading taken here is the
[OCP-MX] MXFP8 E4M3 element with the UE8M0 scale of MXFP4:

  E4M3 code c (8 bits): sign = bit 7, exponent = bits 6..3 (bias 7),
      mantissa = bits 2..0.  Exponent field 0 is subnormal: m/8 * 2^-6.
      Otherwise (1 + m/8) * 2^(exp - 7).  The largest finite magnitude is
      0x7E = 448; 0x7F and 0xFF are NaN; there is no infinity.
  One code per byte (no packing).

Scale rule (the MXFP4 reading with E4M3's largest magnitude): the scale of a
block with absolute maximum a is 2^e for the smallest integer e with
a <= 448 * 2^e, clamped to [-127, 127] (a == 0 gives e = -127).  Nothing
saturates under this rule, so NaN codes are never produced.

Rounding: each element v becomes the E4M3 value nearest to v / 2^e; a tie goes
to the code whose mantissa is even (code bit 0 clear).  The sign bit is copied
from v, so -0 and small negatives give code 0x80.
"""
from __future__ import annotations

import numpy as np

GROUP = 32
E4M3_MAX = 448.0
SCALE_EXP_MIN = -127
SCALE_EXP_MAX = 127


def e4m3_decode(codes) -> np.ndarray:
    """fp64 value of each 8-bit code, from its bit fields ([OCP-MX] E4M3)."""
    c = np.asarray(codes).astype(np.int64)
    ex = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(ex == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, ex - 7))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return np.where((c >> 7) & 1, -mag, mag)


# Magnitudes of the non-negative finite codes 0x00 .. 0x7E, in code order
# (which is also increasing order).
E4M3_MAGNITUDES = e4m3_decode(np.arange(0x7F))


def scale_exponent(amax) -> np.ndarray:
    """Smallest integer e with amax <= 448*2^e, clamped to [-127, 127].

    A float estimate, then walked to the exact answer by comparisons against
    448*2^e, which are exact in fp64.
    """
    a = np.asarray(amax, dtype=np.float64)
    assert np.all(np.isfinite(a)) and np.all(a >= 0)
    with np.errstate(divide="ignore"):
        est = np.ceil(np.log2(np.where(a > 0, a, 1.0) / E4M3_MAX))
    e = np.clip(est, SCALE_EXP_MIN - 2, SCALE_EXP_MAX + 2).astype(np.int64)
    for _ in range(4):
        too_small = a > np.ldexp(E4M3_MAX, e)
        e = np.where(too_small, e + 1, e)
        can_lower = a <= np.ldexp(E4M3_MAX, e - 1)
        e = np.where(can_lower, e - 1, e)
    e = np.where(a == 0, SCALE_EXP_MIN, e)
    return np.clip(e, SCALE_EXP_MIN, SCALE_EXP_MAX)


def round_to_e4m3(r) -> np.ndarray:
    """Nearest E4M3 code for each (already scaled) value; ties to the even code.

    The two table neighbours of |r| are found by binary search; the closer one
    wins, and on equal distance the one with an even code.  Sign copied from r.
    """
    r = np.asarray(r, dtype=np.float64)
    mag = np.abs(r)
    assert np.all(mag <= E4M3_MAX), "scaled value outside the E4M3 range"
    tab = E4M3_MAGNITUDES
    hi = np.clip(np.searchsorted(tab, mag, side="left"), 0, len(tab) - 1)
    lo = np.clip(hi - 1, 0, len(tab) - 1)
    d_lo = mag - tab[lo]
    d_hi = tab[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    sign = np.signbit(r).astype(np.int64)
    return (idx | (sign << 7)).astype(np.uint8)


def quantize(v, chunk_rows: int = 1 << 14):
    """Quantize along the last axis in blocks of 32.

    v: finite float array [..., K] with K % 32 == 0.
    Returns (codes uint8 [..., K], scale bytes uint8 [..., K/32]).
    """
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    assert K % GROUP == 0
    assert np.all(np.isfinite(v))
    lead = v.shape[:-1]
    flat = v.reshape(-1, K // GROUP, GROUP)
    codes = np.empty(flat.shape, dtype=np.uint8)
    scales = np.empty(flat.shape[:2], dtype=np.uint8)
    for s in range(0, flat.shape[0], chunk_rows):
        blk = flat[s:s + chunk_rows]
        e = scale_exponent(np.abs(blk).max(axis=-1))
        r = np.ldexp(blk, -e[..., None])                      # exact: power-of-two scaling
        codes[s:s + chunk_rows] = round_to_e4m3(r)
        scales[s:s + chunk_rows] = (e + 127).astype(np.uint8)
    return codes.reshape(*lead, K), scales.reshape(*lead, K // GROUP)


def quantize_packed(v):
    """Same as quantize(): E4M3 codes are whole bytes, so packing is the identity."""
    return quantize(v)


def dequantize(codes, scales) -> np.ndarray:
    """fp64 values [..., K] of codes [..., K] with scale bytes [..., K/32]."""
    vals = e4m3_decode(codes)
    K = vals.shape[-1]
    sc = np.ldexp(1.0, np.asarray(scales).astype(np.int64) - 127)
    return (vals.reshape(*vals.shape[:-1], K // GROUP, GROUP) * sc[..., None]).reshape(vals.shape)

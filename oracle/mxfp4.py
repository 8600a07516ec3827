"""MXFP4: E2M1 element codes with one UE8M0 scale per block of 32.

[P3] section "Key source snippets", the mxf4xmxf4 branch of _run_mega_routed:
activations are packed to E2M1 by pre_dispatch with group_size=32.  [P1]
title: both operands of the W4A4 kernel are packed FP4.  The bit-level formats
are those of [OCP-MX]:

  E2M1 code c (4 bits): sign = bit 3, exponent = bits 2..1 (bias 1),
      mantissa = bit 0.  Magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.  No Inf/NaN.
  UE8M0 scale byte b: value 2^(b-127); b = 255 is NaN.
  Packing: two codes per byte, the even element in the low nibble.

Scale rule (not fixed by the pages; the reading taken here): the scale of a
block with absolute maximum a is 2^e for the smallest integer e with
a <= 6 * 2^e, clamped to [-127, 127] (a == 0 gives e = -127).  Nothing
saturates under this rule.

Rounding: each element v becomes the E2M1 value nearest to v / 2^e; a tie goes
to the code with an even mantissa bit.  The sign bit is copied from v, so -0
and small negatives give code 0x8.
"""
from __future__ import annotations

import numpy as np

GROUP = 32
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1_MAX = 6.0
SCALE_EXP_MIN = -127
SCALE_EXP_MAX = 127


def e2m1_decode(codes) -> np.ndarray:
    """fp64 value of each 4-bit code ([OCP-MX] E2M1)."""
    c = np.asarray(codes).astype(np.int64)
    mag = E2M1_MAGNITUDES[c & 7]
    return np.where((c >> 3) & 1, -mag, mag)


def ue8m0_decode(b) -> np.ndarray:
    """fp64 value 2^(b-127) of each scale byte; NaN for 255 ([OCP-MX] E8M0)."""
    b = np.asarray(b).astype(np.int64)
    v = np.ldexp(1.0, b - 127)
    return np.where(b == 255, np.nan, v)


def scale_exponent(amax) -> np.ndarray:
    """Smallest integer e with amax <= 6*2^e, clamped to [-127, 127].

    Starts from a float estimate and then walks it to the exact answer with
    comparisons against 6*2^e, which are exact in fp64.
    """
    a = np.asarray(amax, dtype=np.float64)
    assert np.all(np.isfinite(a)) and np.all(a >= 0)
    with np.errstate(divide="ignore"):
        est = np.ceil(np.log2(np.where(a > 0, a, 1.0) / E2M1_MAX))
    e = np.clip(est, SCALE_EXP_MIN - 2, SCALE_EXP_MAX + 2).astype(np.int64)
    for _ in range(4):  # at most one step is ever needed; walk both ways
        too_small = a > np.ldexp(E2M1_MAX, e)
        e = np.where(too_small, e + 1, e)
        can_lower = a <= np.ldexp(E2M1_MAX, e - 1)
        e = np.where(can_lower, e - 1, e)
    e = np.where(a == 0, SCALE_EXP_MIN, e)
    return np.clip(e, SCALE_EXP_MIN, SCALE_EXP_MAX)


def round_to_e2m1(r) -> np.ndarray:
    """Nearest E2M1 code for each (already scaled) value; ties to the even code.

    The magnitude index is the arg-min of |  |r| - table  | over the 8 table
    entries; on a tie between two adjacent entries the even index (mantissa
    bit 0) wins.  Sign bit copied from r.
    """
    r = np.asarray(r, dtype=np.float64)
    mag = np.abs(r)
    assert np.all(mag <= E2M1_MAX), "scaled value outside the E2M1 range"
    d = np.abs(mag[..., None] - E2M1_MAGNITUDES)            # [..., 8]
    dmin = d.min(axis=-1, keepdims=True)
    cand = d == dmin
    even = cand & (np.arange(8) % 2 == 0)
    idx = np.where(even.any(axis=-1), even.argmax(axis=-1), cand.argmax(axis=-1))
    sign = np.signbit(r).astype(np.int64)
    return (idx | (sign << 3)).astype(np.uint8)


def quantize(v, chunk_rows: int = 1 << 14):
    """Quantize along the last axis in blocks of 32.

    v: finite float array [..., K] with K % 32 == 0.
    Returns (codes uint8 [..., K] one code per element, scale bytes uint8 [..., K/32]).
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
        codes[s:s + chunk_rows] = round_to_e2m1(r)
        scales[s:s + chunk_rows] = (e + 127).astype(np.uint8)
    return codes.reshape(*lead, K), scales.reshape(*lead, K // GROUP)


def pack(codes) -> np.ndarray:
    """[..., K] codes -> [..., K/2] bytes; byte j = code[2j] | code[2j+1] << 4."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack(packed) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] codes (inverse of pack)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def quantize_packed(v):
    """quantize() followed by pack(): (packed codes [..., K/2], scales [..., K/32])."""
    c, s = quantize(v)
    return pack(c), s


def dequantize(packed, scales) -> np.ndarray:
    """fp64 values [..., K] of packed codes [..., K/2] with scale bytes [..., K/32]."""
    vals = e2m1_decode(unpack(packed))
    K = vals.shape[-1]
    sc = ue8m0_decode(scales)
    return (vals.reshape(*vals.shape[:-1], K // GROUP, GROUP) * sc[..., None]).reshape(vals.shape)

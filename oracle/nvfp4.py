"""NVFP4: E2M1 element codes, one E4M3 scale per block of 16, one fp32 scale per tensor.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name an NVFP4 variant of the layer and nothing more ([P3] prhub
digest of sglang PR "bump sgl-deep-gemm to 0.1.7, MegaMoE uses the mma_type
API for MXFP4", "Motivation": the library release adds NVFP4 mega-MoE
support).  The reading taken here is the public NVFP4 format:

    value = e2m1(code) * e4m3(scale byte) * g

  code        the E2M1 code of oracle.mxfp4 (two a byte, even element low);
  scale byte  an [OCP-MX] FP8 E4M3 code (oracle.mxfp8's bit fields) with the
              sign bit clear, one per 16 consecutive elements along the
              contraction axis;
  g           one fp32 tensor scale > 0 per tensor: per layer for the
              activations x and h, per expert matrix for W1 and W2.

Encoding a block (the pages fix no rule; this is the plain one, with every
step one fp32 operation rounded to nearest even, the precision in which the
device takes the same decisions):

    d   = f32(6 * g)
    sf  = f32(amax / d)            amax = the largest |v| of the block
    s   = the E4M3 code nearest to min(sf, 448), ties to the even code
    inv = 0 if s encodes 0, else f32(1 / f32(e4m3(s) * g))
    q   = f32(v * inv) clamped to [-6, 6]
    code = the E2M1 code nearest to q, ties to the even code, sign copied
           from q (so -0 and small negatives give 0x8).

The block scale saturates at 448 and the codes at +-6, so values beyond
6 * 448 * g come out as +-6 * 448 * g.  The tensor scale is the caller's (a
calibration constant, like a weight); tensor_scale() is the usual choice
amax / (6 * 448), which makes the largest block of the tensor land on the
largest scale.  g must lie in [2^-100, 2^100] so that every step above stays
finite.
"""
from __future__ import annotations

import numpy as np

from . import mxfp4, mxfp8

GROUP = 16
E4M3_MAX = 448.0
E2M1_MAX = 6.0
G_MIN = 2.0 ** -100
G_MAX = 2.0 ** 100


def _f32(v):
    return np.asarray(v, dtype=np.float32)


def tensor_scale(amax) -> np.float32:
    """The tensor scale that maps a tensor's absolute maximum to 6 * 448: f32(f32(amax) / 2688)."""
    return np.float32(np.float32(amax) / np.float32(6.0 * E4M3_MAX))


def _check_g(g) -> np.float32:
    g = np.float32(g)
    assert np.isfinite(g) and G_MIN <= float(g) <= G_MAX, g
    return g


def scale_codes(amax, g) -> np.ndarray:
    """E4M3 scale byte of blocks with absolute maxima `amax` (fp32 values) under tensor scale g."""
    g = _check_g(g)
    a = _f32(amax)
    assert np.all(a >= 0) and np.all(a.astype(np.float64) == np.asarray(amax, dtype=np.float64))
    d = np.float32(np.float32(6.0) * g)
    with np.errstate(over="ignore"):
        sf = (a / d).astype(np.float32)
    sf = np.minimum(sf, np.float32(E4M3_MAX))
    return mxfp8.round_to_e4m3(sf.astype(np.float64))


def scale_values(scale_bytes) -> np.ndarray:
    """fp64 value of each E4M3 scale byte (sign bit clear)."""
    s = np.asarray(scale_bytes)
    assert np.all((s & 0x80) == 0)
    return mxfp8.e4m3_decode(s)


def quantize(v, g, chunk_rows: int = 1 << 14):
    """Quantize along the last axis in blocks of 16.

    v: fp32-representable finite values [..., K], K % 16 == 0 (bf16 inputs,
       fp32 weights, or h rounded to fp32).
    Returns (codes uint8 [..., K] one code per element, scale bytes uint8 [..., K/16]).
    """
    g = _check_g(g)
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    assert K % GROUP == 0
    assert np.all(np.isfinite(v))
    v32 = v.astype(np.float32)
    assert np.array_equal(v32.astype(np.float64), v), "values must be fp32-representable"
    lead = v.shape[:-1]
    flat = v32.reshape(-1, K // GROUP, GROUP)
    codes = np.empty(flat.shape, dtype=np.uint8)
    scales = np.empty(flat.shape[:2], dtype=np.uint8)
    for r0 in range(0, flat.shape[0], chunk_rows):
        blk = flat[r0:r0 + chunk_rows]
        s = scale_codes(np.abs(blk).max(axis=-1), g)
        t = (scale_values(s).astype(np.float32) * g).astype(np.float32)
        with np.errstate(divide="ignore"):
            inv = np.where(s == 0, np.float32(0), (np.float32(1) / t).astype(np.float32)).astype(np.float32)
        with np.errstate(over="ignore"):
            q = (blk * inv[..., None]).astype(np.float32)
        q = np.minimum(np.maximum(q, np.float32(-E2M1_MAX)), np.float32(E2M1_MAX))
        codes[r0:r0 + chunk_rows] = mxfp4.round_to_e2m1(q.astype(np.float64))
        scales[r0:r0 + chunk_rows] = s
    return codes.reshape(*lead, K), scales.reshape(*lead, K // GROUP)


def quantize_packed(v, g):
    """quantize() followed by mxfp4.pack(): (packed codes [..., K/2], scale bytes [..., K/16])."""
    c, s = quantize(v, g)
    return mxfp4.pack(c), s


def dequantize(packed, scales, g) -> np.ndarray:
    """fp64 values [..., K] of packed codes [..., K/2] with scale bytes [..., K/16] and tensor scale g."""
    vals = mxfp4.e2m1_decode(mxfp4.unpack(packed))
    K = vals.shape[-1]
    sc = scale_values(scales) * float(np.float32(g))
    return (vals.reshape(*vals.shape[:-1], K // GROUP, GROUP) * sc[..., None]).reshape(vals.shape)

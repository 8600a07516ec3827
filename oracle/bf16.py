"""bfloat16 encode/decode for the oracle.

The layer's input and output are bfloat16 ([P3] "Key source snippets":
pre_dispatch takes the model's hidden_states; the final output is in the
model's dtype).  The output is rounded once, from the fp64 result, to the
nearest bfloat16 with ties to even.
"""
from __future__ import annotations

import numpy as np

_MANT_BITS = 7          # explicit mantissa bits of bfloat16
_EMIN = -126            # smallest normal exponent


def decode(bits) -> np.ndarray:
    """fp64 value of each bf16 bit pattern (uint16)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def encode(v) -> np.ndarray:
    """Nearest bfloat16 (ties to even) of each finite fp64 value, as uint16 bits.

    The quantum of the bf16 grid around v is 2^(max(E, -126) - 7) where
    2^E <= |v| < 2^(E+1); v / quantum is rounded half-to-even (np.rint) and
    scaled back, which is exact in fp64.  Results of magnitude 2^128 or more
    become +-Inf.
    """
    v = np.asarray(v, dtype=np.float64)
    assert np.all(np.isfinite(v))
    _, ex = np.frexp(v)                       # |v| = f * 2^ex, f in [0.5, 1)
    E = np.where(v == 0, _EMIN, ex - 1)
    q = np.maximum(E, _EMIN) - _MANT_BITS
    r = np.ldexp(np.rint(np.ldexp(v, -q)), q)
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, v), r)
    out32 = r.astype(np.float32)              # exact: r is on the bf16 grid
    out32 = np.where(v == 0, np.copysign(np.float32(0), v), out32).astype(np.float32)
    return (out32.view(np.uint32) >> 16).astype(np.uint16)

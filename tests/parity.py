"""Comparison rules between the device path and the oracle.

  codes/scales of x, routing arrays ........ bit-exact
  requantized h codes ...................... on groups whose scale bytes agree,
      >= 99.9 % of elements identical (+0 and -0 are one grid point) and every
      difference at most one step on the signed E2M1 grid; a group whose scale
      bytes differ must have its oracle absmax within 1e-4 (relative) of a scale
      boundary 6 * 2^e
  y (GEMM2 result, stored bf16) ............ relative L2 error <= 4e-3 against
      the oracle's fp64 y, and >= 99.9 % of its bf16 values equal to the
      oracle's y rounded to bf16
  final bf16 output ........................ relative L2 error <= 5e-3
"""
import numpy as np

from oracle import mxfp4

OUT_REL_L2 = 5e-3
REQUANT_IDENTICAL = 0.999
Y_REL_L2 = 4e-3          # y is stored in bfloat16: one rounding, relative error <= 2^-8


def grid_index(codes):
    c = np.asarray(codes).astype(np.int64)
    mag = c & 7
    return np.where(c & 8, -mag, mag)


def compare_requant(g_hq, g_hsf, r_hq, r_hsf, r_h):
    """Returns a dict of statistics; asserts the rules above."""
    gc, rc = mxfp4.unpack(g_hq), mxfp4.unpack(r_hq)
    same = np.asarray(g_hsf) == np.asarray(r_hsf)
    mask = np.repeat(same, 32, axis=-1)
    d = np.abs(grid_index(gc) - grid_index(rc))
    n = int(mask.sum())
    ident = int(((d == 0) & mask).sum())
    stats = dict(elements=n, identical=ident, max_step=int(d[mask].max()) if n else 0,
                 scale_mismatch_groups=int((~same).sum()))
    assert n == 0 or ident / n >= REQUANT_IDENTICAL, stats
    assert stats["max_step"] <= 1, stats
    if stats["scale_mismatch_groups"]:
        h32 = np.asarray(r_h, dtype=np.float64).astype(np.float32).astype(np.float64)
        amax = np.abs(h32.reshape(*h32.shape[:-1], -1, 32)).max(axis=-1)[~same]
        nearest = 6.0 * 2.0 ** np.round(np.log2(np.maximum(amax, 1e-300) / 6.0))
        rel = np.abs(amax / nearest - 1.0)
        assert np.all(rel <= 1e-4), (stats, rel.max())
    return stats


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / den) if den > 0 else float(np.linalg.norm(a - b))


def check_y(g_y, r_y):
    """g_y: device y decoded to float; r_y: oracle fp64 y (same rows)."""
    from oracle import bf16
    err = rel_l2(g_y, r_y) if np.asarray(r_y).size else 0.0
    same = float(np.mean(bf16.encode(np.asarray(g_y, np.float64)) == bf16.encode(r_y))) if np.asarray(r_y).size else 1.0
    assert err <= Y_REL_L2, err
    assert same >= 0.999, same
    return err, same

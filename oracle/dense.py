"""Brute-force dense evaluation of the layer, for tiny inputs.

Every expert is applied to every token (no sort, no gather), and the routing
enters only as a mask in the combine:  out[t] = sum over slots j with a valid
id e = ids[t, j] of w[t, j] * y_e(t).  It shares the MXFP4 and bf16 helpers of
the oracle (pinned on their own) but none of its routing or GEMM code, so it
checks oracle.route and oracle.forward independently.
"""
from __future__ import annotations

import numpy as np

from . import bf16, mxfp4, mxfp8


def dense_forward(x_bf16, topk_ids, topk_weights, w1_codes, w1_scales, w2_codes, w2_scales,
                  mma_type: str = "mxf4xmxf4"):
    """mma_type "fp8xfp4" quantizes x and h to MXFP8 E4M3 instead of MXFP4."""
    act = mxfp8 if mma_type == "fp8xfp4" else mxfp4
    x_bits = np.asarray(x_bf16, dtype=np.uint16)
    ids = np.asarray(topk_ids)
    w = np.asarray(topk_weights, dtype=np.float64)
    T, H = x_bits.shape
    E, twoI, _ = np.asarray(w1_codes).shape
    I = twoI // 2
    k = ids.shape[1]
    xq, xsf = act.quantize_packed(bf16.decode(x_bits))
    x_hat = act.dequantize(xq, xsf)                             # [T, H]
    W1 = mxfp4.dequantize(w1_codes, w1_scales)                  # [E, 2I, H]
    W2 = mxfp4.dequantize(w2_codes, w2_scales)                  # [E, H, I]
    acc = np.einsum("th,enh->etn", x_hat, W1)                   # [E, T, 2I]
    gate, up = acc[..., :I], acc[..., I:]
    with np.errstate(over="ignore"):
        h = gate / (1.0 + np.exp(-gate)) * up                   # [E, T, I]
    hq, hsf = act.quantize_packed(h.astype(np.float32).astype(np.float64))
    y = np.einsum("eti,ehi->eth", act.dequantize(hq, hsf), W2)  # [E, T, H]
    out = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            if 0 <= e < E:
                out[t] = out[t] + w[t, j] * y[e, t]
    return dict(out_f64=out, out=bf16.encode(out), y_all=y, h_all=h)

"""Brute-force dense evaluation of the layer, for tiny inputs.

Every expert is applied to every token (no sort, no gather), and the routing
enters only as a mask in the combine:  out[t] = sum over slots j with a valid
id e = ids[t, j] of w[t, j] * y_e(t).  It shares the format codecs (mxfp4,
mxfp8, nvfp4) and bf16 helpers of the oracle (pinned on their own) but none of
its routing or GEMM code, so it checks oracle.route and oracle.forward
independently.
"""
from __future__ import annotations

import numpy as np

from . import bf16, mxfp4, mxfp8, nvfp4


def dense_forward(x_bf16, topk_ids, topk_weights, w1_codes, w1_scales, w2_codes, w2_scales,
                  mma_type: str = "mxf4xmxf4", tensor_scales=None):
    """mma_type "fp8xfp4" quantizes x and h to MXFP8 E4M3 instead of MXFP4;
    "nvf4xnvf4" makes x, h and the weights NVFP4 with tensor_scales =
    (g_x, g_h, g_w1 [E], g_w2 [E])."""
    x_bits = np.asarray(x_bf16, dtype=np.uint16)
    ids = np.asarray(topk_ids)
    w = np.asarray(topk_weights, dtype=np.float64)
    T, H = x_bits.shape
    E, twoI, _ = np.asarray(w1_codes).shape
    I = twoI // 2
    k = ids.shape[1]
    xv = bf16.decode(x_bits)
    if mma_type == "nvf4xnvf4":
        g_x, g_h, g_w1, g_w2 = tensor_scales
        x_hat = nvfp4.dequantize(*nvfp4.quantize_packed(xv, g_x), g_x)
        W1 = np.stack([nvfp4.dequantize(w1_codes[e], w1_scales[e], g_w1[e]) for e in range(E)])
        W2 = np.stack([nvfp4.dequantize(w2_codes[e], w2_scales[e], g_w2[e]) for e in range(E)])
        requant = lambda v: nvfp4.dequantize(*nvfp4.quantize_packed(v, g_h), g_h)   # noqa: E731
    else:
        act = mxfp8 if mma_type == "fp8xfp4" else mxfp4
        x_hat = act.dequantize(*act.quantize_packed(xv))
        W1 = mxfp4.dequantize(w1_codes, w1_scales)              # [E, 2I, H]
        W2 = mxfp4.dequantize(w2_codes, w2_scales)              # [E, H, I]
        requant = lambda v: act.dequantize(*act.quantize_packed(v))                 # noqa: E731
    acc = np.einsum("th,enh->etn", x_hat, W1)                   # [E, T, 2I]
    gate, up = acc[..., :I], acc[..., I:]
    with np.errstate(over="ignore"):
        h = gate / (1.0 + np.exp(-gate)) * up                   # [E, T, I]
    y = np.einsum("eti,ehi->eth", requant(h.astype(np.float32).astype(np.float64)), W2)  # [E, T, H]
    out = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            if 0 <= e < E:
                out[t] = out[t] + w[t, j] * y[e, t]
    return dict(out_f64=out, out=bf16.encode(out), y_all=y, h_all=h)

"""The W4A4 routed-expert layer, step by step, in fp64.

Steps (the layer that [P1] measures as one fused kernel; the pages print only
pre_dispatch and the buffer, [P3] "Key source snippets", so the stage list is
the plain reading of a routed SwiGLU expert layer with activation="swiglu" and
MXFP4 operands on both sides):

  1. pre_dispatch: quantize every token row of x to MXFP4 (group 32) once.
  2. route: stable counting sort of the routed rows by expert (oracle.route).
  3. GEMM1 per expert e over its rows:  acc = x_hat[t] . W1_hat[e]^T  (fp64);
     gate = acc[:, :I], up = acc[:, I:]  -- W1 rows [0, I) are gate and
     [I, 2I) are up, the split that _interleave_mega_moe_gate_up slices ([P3]
     "Key source snippets");  h = silu(gate) * up = gate / (1 + exp(-gate)) * up.
  4. requantize h to MXFP4 along I (same rule as step 1).  The pages leave the
     precision of h open; the device keeps h in fp32, so the code decision is
     taken on h rounded to fp32 on both sides (h itself is kept in fp64).
  5. GEMM2: y = h_hat . W2_hat[e]^T  (fp64).
  6. combine: out[t] = sum over valid slots j, in slot order, of w[t, j] * y[pos(t, j)],
     in fp64, then rounded once to bfloat16.  A token with no valid slot gives +0.

The top-k weights are applied in the combine only and are used as given.

mma_type (the pages' two MMA types, [P3] "Implementation breakdown" items 1-3,
and the NVFP4 variant its "Motivation" names): "mxf4xmxf4" quantizes x
(step 1) and h (step 4) to MXFP4; "fp8xfp4" quantizes both to MXFP8 E4M3
(oracle.mxfp8); the weights are MXFP4 in both.  "nvf4xnvf4" makes x, h and the
weights NVFP4 (oracle.nvfp4: E4M3 scales per 16 elements and an fp32 tensor
scale), with the tensor scales passed as `tensor_scales` = (g_x, g_h,
g_w1 [E], g_w2 [E]); the weight scale arrays then hold one byte per 16
elements.

Weight operands are passed either as arrays (w1_codes [E, 2I, H/2],
w1_scales [E, 2I, H/32], w2_codes [E, H, I/2], w2_scales [E, H, I/32]) or as a
callable e -> (w1_codes[e], w1_scales[e], w2_codes[e], w2_scales[e]) so that a
caller can supply experts lazily.
"""
from __future__ import annotations

import numpy as np

from . import bf16, mxfp4, mxfp8, nvfp4
from .route import route

MMA_TYPES = ("mxf4xmxf4", "fp8xfp4", "nvf4xnvf4")


def act_format(mma_type: str):
    """The activation format module of an MX MMA type: mxfp4 or mxfp8."""
    assert mma_type in MMA_TYPES[:2], mma_type
    return mxfp8 if mma_type == "fp8xfp4" else mxfp4


class NvTensor:
    """The NVFP4 codec of one tensor (oracle.nvfp4) with its tensor scale g,
    with the quantize_packed / dequantize interface of the MX format modules."""

    def __init__(self, g):
        self.g = np.float32(g)

    def quantize_packed(self, v):
        return nvfp4.quantize_packed(v, self.g)

    def dequantize(self, packed, scales):
        return nvfp4.dequantize(packed, scales, self.g)


def _expert_getter(weights):
    if callable(weights):
        return weights
    w1c, w1s, w2c, w2s = weights
    return lambda e: (w1c[e], w1s[e], w2c[e], w2s[e])


def to_f32(v):
    """Round fp64 values to the nearest fp32 (ties to even) and return them as fp64."""
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def silu_mul(gate, up):
    """SwiGLU: gate / (1 + exp(-gate)) * up, no clamp, no bias, fp64."""
    with np.errstate(over="ignore"):
        return gate / (1.0 + np.exp(-gate)) * up


def expert_gemm2(hq, hsf, w2_codes, w2_scales, act=mxfp4, wfmt=mxfp4):
    """Step 5 for one expert's rows: y = h_hat . W2_hat^T in fp64, h_hat the
    dequantized requantized h (act: the activation format, oracle.mxfp4,
    oracle.mxfp8 or an NvTensor) and W2_hat the dequantized W2 [H, I] (wfmt:
    oracle.mxfp4, or the expert's NvTensor)."""
    return act.dequantize(hq, hsf) @ wfmt.dequantize(w2_codes, w2_scales).T


def combine(y, pos, topk_weights, want=None):
    """Step 6: out[t] = sum over the valid slots j (pos >= 0), in slot order and
    starting from +0, of w[t, j] * y[pos[t * k + j]], in fp64; a token with no
    valid slot gives +0.  Rows of tokens outside `want` (a boolean mask) are
    NaN.  Rounding to bfloat16 is the caller's."""
    w = np.asarray(topk_weights, dtype=np.float64)
    T, k = w.shape
    H = y.shape[1]
    out = np.full((T, H), np.nan)
    for t in range(T):
        if want is not None and not want[t]:
            continue
        acc = np.zeros(H)
        for j in range(k):
            p = pos[t * k + j]
            if p >= 0:
                acc = acc + w[t, j] * y[p]
        out[t] = acc
    return out


def forward(x_bf16, topk_ids, topk_weights, weights, num_experts: int, inter: int,
            tokens=None, keep_acc: bool = False, experts=None, mma_type: str = "mxf4xmxf4",
            tensor_scales=None):
    """Run the layer.

    x_bf16        uint16 [T, H] bfloat16 bit patterns
    topk_ids      int    [T, k]
    topk_weights  float  [T, k]
    weights       arrays or callable (see module doc)
    tokens        optional iterable of token indices: compute y only for the
                  routed rows of these tokens and out only for them (other
                  rows of y / out are NaN).  None = all tokens.
    experts       optional iterable of expert indices: run steps 3-5 only for
                  these experts' rows and skip step 6 (out stays NaN); used to
                  time a bounded slice of the layer.  None = all experts.
    tensor_scales (g_x, g_h, g_w1 [E], g_w2 [E]) for mma_type "nvf4xnvf4"

    Returns a dict with every intermediate:
      xq, xsf          codes of x ([T, H/2] packed E2M1, or [T, H] E4M3) and scale bytes
                       [T, H/32] (NVFP4: [T, H/16])
      counts, offsets, sorted_rows, pos
      acc              fp64 [n_valid, 2I] GEMM1 result (gate | up), only with keep_acc
      h                fp64 [n_valid, I] (NaN where not computed), in sorted order
      hq, hsf          codes [n_valid, I/2] (E2M1) or [n_valid, I] (E4M3), scale bytes [n_valid, I/32]
      y                fp64 [n_valid, H]
      out_f64          fp64 [T, H]
      out              uint16 [T, H] bfloat16 bits
    """
    x_bits = np.asarray(x_bf16, dtype=np.uint16)
    ids = np.asarray(topk_ids)
    w = np.asarray(topk_weights, dtype=np.float64)
    T, H = x_bits.shape
    k = ids.shape[1]
    E, I = int(num_experts), int(inter)
    get = _expert_getter(weights)

    if mma_type == "nvf4xnvf4":
        g_x, g_h, g_w1, g_w2 = tensor_scales
        act_x, act = NvTensor(g_x), NvTensor(g_h)
        w1fmt = lambda e: NvTensor(np.asarray(g_w1, dtype=np.float32)[e])   # noqa: E731
        w2fmt = lambda e: NvTensor(np.asarray(g_w2, dtype=np.float32)[e])   # noqa: E731
        group = nvfp4.GROUP
    else:
        assert tensor_scales is None
        act_x = act = act_format(mma_type)
        w1fmt = w2fmt = lambda e: mxfp4                                     # noqa: E731
        group = mxfp4.GROUP
    xv = bf16.decode(x_bits)
    xq, xsf = act_x.quantize_packed(xv)                        # step 1
    x_hat = act_x.dequantize(xq, xsf)

    counts, offsets, sorted_rows, pos = route(ids, E)          # step 2
    nv = int(offsets[E])

    if tokens is None:
        want = np.ones(T, dtype=bool)
    else:
        want = np.zeros(T, dtype=bool)
        want[np.asarray(list(tokens), dtype=np.int64)] = True

    h = np.full((nv, I), np.nan)
    hq = np.zeros((nv, I if act is mxfp8 else I // 2), dtype=np.uint8)
    hsf = np.zeros((nv, I // group), dtype=np.uint8)
    y = np.full((nv, H), np.nan)
    acc_all = np.full((nv, 2 * I), np.nan) if keep_acc else None

    expert_list = range(E) if experts is None else sorted(set(int(e) for e in experts))
    for e in expert_list:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if lo == hi:
            continue
        p_idx = np.arange(lo, hi)
        rows = sorted_rows[lo:hi]
        tok = rows // k
        sel = want[tok]
        if not sel.any():
            continue
        p_idx, tok = p_idx[sel], tok[sel]
        w1c, w1s, w2c, w2s = get(e)
        W1 = w1fmt(e).dequantize(w1c, w1s)                     # [2I, H]
        acc = x_hat[tok] @ W1.T                                # step 3
        h_e = silu_mul(acc[:, :I], acc[:, I:])
        hq_e, hsf_e = act.quantize_packed(to_f32(h_e))        # step 4
        y_e = expert_gemm2(hq_e, hsf_e, w2c, w2s, act, w2fmt(e))   # step 5
        h[p_idx], hq[p_idx], hsf[p_idx], y[p_idx] = h_e, hq_e, hsf_e, y_e
        if keep_acc:
            acc_all[p_idx] = acc

    if experts is None:                                        # step 6
        out = combine(y, pos, w, want)
    else:
        out = np.full((T, H), np.nan)
    out_bits = np.zeros((T, H), dtype=np.uint16)
    if experts is None:
        out_bits[want] = bf16.encode(out[want])

    return dict(xq=xq, xsf=xsf, counts=counts, offsets=offsets, sorted_rows=sorted_rows,
                pos=pos, acc=acc_all, h=h, hq=hq, hsf=hsf, y=y, out_f64=out, out=out_bits)

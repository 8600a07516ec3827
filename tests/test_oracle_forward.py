"""Pins for oracle.forward: brute-force dense evaluation, exact rational GEMM
entries, closed-form single-expert example, zero-in/zero-out and scaling
invariants."""
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import bf16, mxfp4
from oracle.dense import dense_forward
from oracle.forward import forward
from tests.oracle_inputs import all_expert_weights

TINY = synth.CONFIGS[0]


@pytest.fixture(scope="module")
def tiny():
    x = synth.make_tokens(TINY)
    ids, w = synth.make_routing(TINY)
    W = all_expert_weights(TINY)
    return x, ids, w, W


def test_topk_weights_sum_to_one():
    for cfg in synth.CONFIGS[:3]:
        ids, w = synth.make_routing(cfg)
        assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6)
        assert all(len(set(r)) == cfg.topk for r in ids.tolist())


def test_forward_equals_dense_brute_force(tiny):
    x, ids, w, W = tiny
    ref = dense_forward(x, ids, w, *W)
    got = forward(x, ids, w, W, TINY.experts, TINY.inter)
    assert np.array_equal(got["out_f64"], ref["out_f64"])
    assert np.array_equal(got["out"], ref["out"])


def test_forward_equals_dense_with_masked_and_duplicate_ids(tiny):
    x, ids, w, W = tiny
    ids = ids.copy()
    ids[0, 1] = -1               # masked slot
    ids[1, :] = -1               # token with no valid slot -> +0
    ids[2, 1] = ids[2, 0]        # same expert twice
    ids[3, 0] = TINY.experts     # out of range
    ref = dense_forward(x, ids, w, *W)
    got = forward(x, ids, w, W, TINY.experts, TINY.inter)
    assert np.array_equal(got["out"], ref["out"])
    assert np.all(got["out"][1] == 0)


def _field_value(code):
    s, ex, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = Fraction(m, 2) if ex == 0 else Fraction(2) ** (ex - 1) * (1 + Fraction(m, 2))
    return -mag if s else mag


def _row_exact(packed_row, scale_row):
    """Exact rational values of one packed MXFP4 row, decoded from the bit fields."""
    vals = []
    for j, byte in enumerate(packed_row.tolist()):
        for code in (byte & 15, byte >> 4):            # even element in the low nibble
            vals.append(_field_value(code) * Fraction(2) ** (int(scale_row[len(vals) // 32]) - 127))
    return vals


def test_gemm_entries_are_exact(tiny):
    x, ids, w, W = tiny
    w1c, w1s, w2c, w2s = W
    got = forward(x, ids, w, W, TINY.experts, TINY.inter)
    I = TINY.inter
    rng = np.random.default_rng(0)
    k = TINY.topk
    for p in rng.choice(len(got["sorted_rows"]), 6, replace=False):
        r = int(got["sorted_rows"][p])
        t, e = r // k, int(ids.reshape(-1)[r])
        xr = _row_exact(got["xq"][t], got["xsf"][t])
        for n in rng.choice(I, 3, replace=False):
            g = sum(a * b for a, b in zip(xr, _row_exact(w1c[e, n], w1s[e, n])))
            u = sum(a * b for a, b in zip(xr, _row_exact(w1c[e, I + n], w1s[e, I + n])))
            h = float(g) / (1.0 + np.exp(-float(g))) * float(u)
            assert got["h"][p, n] == h
        hr = _row_exact(got["hq"][p], got["hsf"][p])
        for m in rng.choice(TINY.hidden, 3, replace=False):
            yv = sum(a * b for a, b in zip(hr, _row_exact(w2c[e, m], w2s[e, m])))
            assert got["y"][p, m] == float(yv)


def test_single_expert_closed_form():
    # E=1, k=1, T=1, H=I=32.  x = e_0 (1.0) so gate_i = g_i and up_i = u_i exactly;
    # W2 is the cyclic permutation y_m = h_hat[(m + 1) % 32]; w = 1.
    H = I = 32
    vals = [1.0, -1.5, 2.0, 0.5, -3.0, 4.0, 6.0, -0.75]
    g = np.array([vals[i % 8] * 2.0 ** ((i // 8) - 1) for i in range(I)])
    u = np.array([vals[(3 * i + 1) % 8] * 2.0 ** (1 - (i // 8)) for i in range(I)])
    W1 = np.zeros((2 * I, H))
    W1[:I, 0], W1[I:, 0] = g, u
    W2 = np.zeros((H, I))
    for m in range(H):
        W2[m, (m + 1) % I] = 1.0
    w1c, w1s = mxfp4.quantize_packed(W1)
    w2c, w2s = mxfp4.quantize_packed(W2)
    assert np.array_equal(mxfp4.dequantize(w1c, w1s), W1)      # all entries representable
    x = np.zeros((1, H), np.uint16)
    x[0, 0] = 0x3F80                                           # bf16 1.0
    got = forward(x, np.zeros((1, 1), np.int32), np.ones((1, 1), np.float32),
                  (w1c[None], w1s[None], w2c[None], w2s[None]), 1, I)
    h = np.array([gi / (1.0 + np.exp(-gi)) * ui for gi, ui in zip(g, u)])
    assert np.array_equal(got["h"][0], h)
    h_hat = mxfp4.dequantize(*mxfp4.quantize_packed(h.astype(np.float32)))
    # the combine sums from +0, so a lone -0 term comes out as +0
    want = 0.0 + np.array([h_hat[(m + 1) % I] for m in range(H)])
    assert np.array_equal(got["out_f64"][0], want)
    assert np.array_equal(got["out"][0], bf16.encode(want))


def test_zero_in_zero_out(tiny):
    x, ids, w, W = tiny
    got = forward(np.zeros_like(x), ids, w, W, TINY.experts, TINY.inter)
    assert np.all(got["xq"] == 0) and np.all(got["xsf"] == 0)
    assert np.all(got["out"] == 0)
    zW = tuple(np.zeros_like(a) for a in W)
    got = forward(x, ids, w, zW, TINY.experts, TINY.inter)
    assert np.all(got["out"] == 0)


def test_doubling_weights_doubles_output(tiny):
    x, ids, w, W = tiny
    a = forward(x, ids, w, W, TINY.experts, TINY.inter)
    b = forward(x, ids, 2 * w, W, TINY.experts, TINY.inter)
    assert np.array_equal(b["out_f64"], 2 * a["out_f64"])


def test_token_subset_matches_full(tiny):
    x, ids, w, W = tiny
    full = forward(x, ids, w, W, TINY.experts, TINY.inter)
    sub = forward(x, ids, w, W, TINY.experts, TINY.inter, tokens=[3, 7, 11])
    for t in (3, 7, 11):
        assert np.array_equal(sub["out"][t], full["out"][t])

"""GPU tier, stage by stage, through the C ABI: each stage against the oracle
on the same seeded inputs, with exact cases where the arithmetic is exact."""
import numpy as np
import pytest
import torch

from oracle import bf16, mxfp4
from oracle.forward import combine, expert_gemm2
from oracle.route import route
from synth import f32_to_bf16_bits as _f32_to_bf16_bits
from tests.gpu_support import dev, dev_bf16, host_bits, layer_for, log, planes_from_rows


def synth_bf16(v):
    return _f32_to_bf16_bits(np.asarray(v, dtype=np.float32))

pytestmark = pytest.mark.gpu


def _quantize_dev(src_t):
    from block_scaled_fp4_pre_amd import _lib
    rows, cols = src_t.shape
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device="cuda")
    _lib.moe_w4a4_quantize(src_t, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def test_quantize_every_bf16_pattern_as_lone_value():
    log("[test] quantize: every finite bf16 pattern")
    bits = np.arange(1 << 16, dtype=np.uint32)
    keep = ((bits >> 7) & 0xFF) != 0xFF
    b = bits[keep].astype(np.uint16)
    grp = np.zeros((b.size, 32), np.uint16)
    grp[:, 0] = b
    grp[:, 17] = b[::-1]                  # a second value, so both positions are exercised
    c, s = _quantize_dev(dev_bf16(grp))
    rc, rs = mxfp4.quantize_packed(bf16.decode(grp))
    assert np.array_equal(s, rs)
    assert np.array_equal(c, rc)


def test_quantize_random_bf16_and_fp32():
    log("[test] quantize: random bf16 / fp32 rows, odd row count")
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((129, 4096)) * np.exp(rng.uniform(-20, 20, (129, 1)))).astype(np.float32)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)  # truncation is fine: any bf16 is a valid input
    c, s = _quantize_dev(dev_bf16(xb))
    rc, rs = mxfp4.quantize_packed(bf16.decode(xb))
    assert np.array_equal(s, rs) and np.array_equal(c, rc)
    w = (rng.standard_normal((1000, 256)) * 0.02).astype(np.float32)
    w[::5] *= np.float32(1e-30)
    w[3, :] = 0.0
    w[4, 7] = -0.0
    c, s = _quantize_dev(dev(w))
    rc, rs = mxfp4.quantize_packed(w.astype(np.float64))
    assert np.array_equal(s, rs) and np.array_equal(c, rc)


@pytest.mark.parametrize("T,k,E,masked", [
    (1, 1, 1, False), (3, 2, 8, True), (129, 6, 256, True), (1000, 6, 256, False),
    (171, 6, 256, True), (16384, 6, 256, False), (700, 16, 512, True), (2048, 4, 3, True)])
def test_route_matches_oracle(T, k, E, masked):
    log(f"[test] route T={T} k={k} E={E} masked={masked}")
    rng = np.random.default_rng(T * 31 + E)
    lo = -2 if masked else 0
    hi = E + 2 if masked else E
    ids = rng.integers(lo, hi, (T, k)).astype(np.int32)
    layer = layer_for(256, 128, E, k, T)
    layer.run_stages(2, T, topk_ids=dev(ids))
    torch.cuda.synchronize()
    counts, offsets, srt, pos = route(ids, E)
    ws = layer.ws
    assert np.array_equal(ws("counts", (E,), torch.int32).cpu().numpy(), counts)
    assert np.array_equal(ws("offsets", (E + 1,), torch.int32).cpu().numpy(), offsets)
    assert np.array_equal(ws("sorted_rows", (T * k,), torch.int32)[:srt.size].cpu().numpy(), srt)
    assert np.array_equal(ws("pos", (T * k,), torch.int32).cpu().numpy(), pos)
    if (T * k + E - 1) // E > 16:
        # many rows per expert: the route also lists equal-size (expert, first row)
        # tiles, in expert order, covering every expert's rows exactly once
        nt = int(ws("num_tiles", (1,), torch.int32).cpu().numpy()[0])
        tiles = [tuple(t) for t in ws("tiles", (nt, 2), torch.int32).cpu().numpy().tolist()]
        steps = {b[1] - a[1] for a, b in zip(tiles, tiles[1:]) if a[0] == b[0]}
        assert len(steps) <= 1
        rows_per_tile = steps.pop() if steps else max(int(counts.max()), 1)
        want = [(e, i * rows_per_tile) for e in range(E) for i in range(-(-int(counts[e]) // rows_per_tile))]
        assert tiles == want


def _grid_group(rng, rows, K):
    """Values on the E2M1 grid with one +-6 per group of 32: every scale byte is 127."""
    v = rng.choice(np.concatenate([mxfp4.E2M1_MAGNITUDES, -mxfp4.E2M1_MAGNITUDES]), (rows, K))
    v[:, ::32] = np.where(rng.random((rows, K // 32)) < 0.5, 6.0, -6.0)
    return v


def _canonical_from_values(W1, W2):
    w1c, w1s = mxfp4.quantize_packed(W1)
    w2c, w2s = mxfp4.quantize_packed(W2)
    return w1c, w1s, w2c, w2s


@pytest.mark.parametrize("T,E,k", [(16, 4, 2), (77, 3, 1), (40, 1, 1)])
def test_gemm1_accumulators_exact(T, E, k):
    """With every scale byte 127 each product is a multiple of 0.25 and every
    partial sum stays below 2^18: fp32 accumulation is exact, so the device's
    gate/up accumulators must equal the oracle's fp64 ones bit for bit."""
    log(f"[test] gemm1 exact T={T} E={E} k={k}")
    H, I = 512, 256
    rng = np.random.default_rng(11 + T)
    x = _grid_group(rng, T, H)
    xb = bf16.encode(x)
    W1 = np.stack([_grid_group(rng, 2 * I, H) for _ in range(E)])
    W2 = np.stack([_grid_group(rng, H, I) for _ in range(E)])
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    w = np.full((T, k), 1.0 / k, np.float32)
    W = _canonical_from_values(W1, W2)
    assert np.all(W[1] == 127) and np.all(W[3] == 127)
    layer = layer_for(H, I, E, k, T)
    layer.load_canonical(*(dev(a) for a in W))
    acc = torch.full((T * k, 2 * I), float("nan"), device="cuda")
    layer.run_stages(1 | 2 | 4, T, x=dev_bf16(xb), topk_ids=dev(ids), gemm1_acc=acc)
    torch.cuda.synchronize()
    from oracle.forward import forward
    ref = forward(xb, ids, w, W, E, I, keep_acc=True)
    got = acc.cpu().numpy()[:ref["acc"].shape[0]]
    assert np.array_equal(got.astype(np.float64), ref["acc"])


def test_gemm2_exact_on_injected_rows():
    """GEMM2 alone on requantized rows and a routing written by the test."""
    log("[test] gemm2 exact on injected h")
    H, I, E, k, T = 512, 256, 5, 2, 37
    rng = np.random.default_rng(5)
    W1 = np.zeros((E, 2 * I, H))
    W2 = np.stack([_grid_group(rng, H, I) for _ in range(E)])
    W = _canonical_from_values(W1, W2)
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    counts, offsets, srt, pos = route(ids, E)
    hvals = _grid_group(rng, srt.size, I)
    hq, hsf = mxfp4.quantize_packed(hvals)
    layer = layer_for(H, I, E, k, T)
    layer.load_canonical(*(dev(a) for a in W))
    ws = layer.ws
    ws("counts", (E,), torch.int32).copy_(torch.from_numpy(counts))
    ws("offsets", (E + 1,), torch.int32).copy_(torch.from_numpy(offsets))
    ws("hq", (I // 128, T * k, 64), torch.uint8)[:, :srt.size].copy_(torch.from_numpy(planes_from_rows(hq, I // 128)))
    ws("hsf", (I // 128, T * k, 4), torch.uint8)[:, :srt.size].copy_(torch.from_numpy(planes_from_rows(hsf, I // 128)))
    layer.run_stages(8, T)
    torch.cuda.synchronize()
    # the fp32 accumulators are exact here, so the stored bf16 y is the exact
    # product rounded once to bf16 (nearest even)
    y = host_bits(ws("y", (T * k, H), torch.bfloat16)[:srt.size])
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        assert np.array_equal(y[lo:hi], bf16.encode(expert_gemm2(hq[lo:hi], hsf[lo:hi], W[2][e], W[3][e])))


def test_combine_exact_cases():
    """y is injected as bf16; with k = 1 and w = 1 the output is y bit for bit."""
    log("[test] combine exact cases")
    H, I, E = 512, 256, 6
    rng = np.random.default_rng(9)
    for k, T in ((1, 50), (4, 33)):
        ids = rng.integers(-1, E, (T, k)).astype(np.int32)
        counts, offsets, srt, pos = route(ids, E)
        y_bits = synth_bf16(rng.standard_normal((max(srt.size, 1), H)) * 3)
        y = bf16.decode(y_bits)
        w = rng.random((T, k)).astype(np.float32) if k > 1 else np.ones((T, k), np.float32)
        layer = layer_for(H, I, E, k, T)
        ws = layer.ws
        ws("pos", (T * k,), torch.int32).copy_(torch.from_numpy(pos))
        ws("y", (T * k, H), torch.int16)[:srt.size].copy_(torch.from_numpy(y_bits[:srt.size].view(np.int16)))
        out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        outs = []
        for scale in (1.0, 2.0):
            layer.run_stages(16, T, topk_weights=dev(w * np.float32(scale)), out=out)
            torch.cuda.synchronize()
            outs.append(host_bits(out).copy())
        ref = combine(y, pos, w)
        if k == 1:
            assert np.array_equal(outs[0], bf16.encode(ref))   # out = bf16(y) exactly
        else:
            diff = np.abs(bf16.decode(outs[0]) - bf16.decode(bf16.encode(ref)))
            ulp = np.abs(bf16.decode(bf16.encode(ref))) * 2.0 ** -7 + 1e-38
            assert np.all(diff <= ulp)
        assert np.array_equal(bf16.decode(outs[1]), 2 * bf16.decode(outs[0]))   # doubling w
        empty = np.all(ids < 0, axis=1)
        assert np.all(outs[0][empty] == 0)

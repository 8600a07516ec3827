"""GPU tier of the NVFP4 MMA type (nvf4xnvf4) through the C ABI.

  - quantization bit-exact against oracle.nvfp4 (every finite bf16 pattern,
    random rows, saturating and vanishing scales, fp32 weights);
  - GEMM1's accumulators and GEMM2's y bit-exact on inputs whose fp32 sums
    are exact (this pins the lane layout of the fp16 operands, the FP4 ->
    fp16 conversion times the block scale, and the placement of every scale
    byte);
  - every stage against the oracle on small layers: one and two token tiles,
    experts with more rows than a pass holds (the weights streamed once per
    pass), empty experts, masked and duplicate ids; and on the LDS-staged
    form (gemm_lds_nv.hip) with one and several 128-row tiles per expert,
    Zipf routing, and the XCD-paired block order of the DSV4 shape;
  - the DSV4 shape at 64, 512, 4096 and 16384 (Zipf) tokens with weights
    quantized on the device:
    the device's NVFP4 weights against the oracle's, and every routed row of
    sampled tokens against the oracle.
Weights of the small layers are quantized by the oracle and loaded as
canonical NVFP4; the tensor scales come from tests/oracle_inputs.py."""
import numpy as np
import pytest
import torch

import synth
from oracle import bf16, mxfp4, mxfp8, nvfp4
from oracle.forward import expert_gemm2, forward, NvTensor
from oracle.route import route
from tests import parity
from tests.gpu_support import dev, dev_bf16, host_bits, log, planes_from_rows, rows_from_planes
from tests.oracle_inputs import (NV_WEIGHT_SCALES, all_expert_weights_nv, lazy_expert_weights_nv, nv_act_scales)

pytestmark = pytest.mark.gpu

NV = 2
Q, RT, G1, G2, CB = 1, 2, 4, 8, 16


def _lib():
    from block_scaled_fp4_pre_amd import _lib as lib
    return lib


def nv_layer(H, I, E, k, T):
    from block_scaled_fp4_pre_amd.layer import MoeW4A4Layer
    return MoeW4A4Layer(H, I, E, k, T, mma_type=NV)


def _quantize_nv_dev(src_t, g):
    rows, cols = src_t.shape
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device="cuda")
    _lib().moe_w4a4_quantize_nvfp4(src_t, g, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def nv_workspace_host(layer, T):
    H, I, E, k, M = layer.H, layer.I, layer.E, layer.k, layer.max_tokens
    ws = layer.ws
    counts = ws("counts", (E,), torch.int32).cpu().numpy()
    nv = int(counts.sum())
    return dict(
        xq=ws("xq", (M, H // 2), torch.uint8)[:T].cpu().numpy(),
        xsf=ws("xsf", (M, H // 16), torch.uint8)[:T].cpu().numpy(),
        counts=counts,
        offsets=ws("offsets", (E + 1,), torch.int32).cpu().numpy(),
        sorted_rows=ws("sorted_rows", (M * k,), torch.int32)[:nv].cpu().numpy(),
        pos=ws("pos", (M * k,), torch.int32)[:T * k].cpu().numpy(),
        hq=rows_from_planes(ws("hq", (I // 128, M * k, 64), torch.uint8), nv),
        hsf=rows_from_planes(ws("hsf", (I // 64, M * k, 4), torch.uint8), nv),
        y=ws("y", (M * k, H), torch.bfloat16)[:nv].float().cpu().numpy().astype(np.float64),
    )


def test_nv_quantize_every_bf16_pattern_as_lone_value():
    log("[test] nvfp4 quantize: every finite bf16 pattern")
    bits = np.arange(1 << 16, dtype=np.uint32)
    b = bits[((bits >> 7) & 0xFF) != 0xFF].astype(np.uint16)
    grp = np.zeros((b.size, 32), np.uint16)
    grp[:, 0] = b
    grp[:, 17] = b[::-1]
    for g in (1.0, 3.7e-4, 151.25, 2.0 ** -100):
        c, s = _quantize_nv_dev(dev_bf16(grp), g)
        rc, rs = nvfp4.quantize_packed(bf16.decode(grp), g)
        assert np.array_equal(s, rs), g
        assert np.array_equal(c, rc), g


def test_nv_quantize_random_rows_and_fp32_weights():
    log("[test] nvfp4 quantize: random bf16 rows and fp32 weights")
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((129, 4096)) * np.exp(rng.uniform(-8, 8, (129, 1)))).astype(np.float32)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    xv = bf16.decode(xb)
    for g in (nvfp4.tensor_scale(np.abs(xv).max()), np.float32(1e-3), np.float32(7.77)):
        c, s = _quantize_nv_dev(dev_bf16(xb), float(g))
        rc, rs = nvfp4.quantize_packed(xv, g)
        assert np.array_equal(s, rs) and np.array_equal(c, rc), g
    w = (rng.standard_normal((1000, 256)) * 0.02).astype(np.float32)
    w[::5] *= np.float32(1e-6)
    w[3, :] = 0.0
    w[4, 7] = -0.0
    g = nvfp4.tensor_scale(np.abs(w).max())
    c, s = _quantize_nv_dev(dev(w), float(g))
    rc, rs = nvfp4.quantize_packed(w.astype(np.float64), g)
    assert np.array_equal(s, rs) and np.array_equal(c, rc)


def _grid_blocks(rng, rows, K, scale_codes=(0x30, 0x38, 0x40)):
    """NVFP4 values e2m1 * e4m3 (g = 1) with one +-6 per block of 16, so that
    the block's scale is the drawn one: 0.5, 1 or 2."""
    c = rng.integers(0, 16, (rows, K)).astype(np.uint8)
    c[:, ::16] = 7 | (8 * rng.integers(0, 2, (rows, K // 16))).astype(np.uint8)
    s = rng.choice(np.array(scale_codes, np.uint8), (rows, K // 16))
    return mxfp4.e2m1_decode(c) * np.repeat(mxfp8.e4m3_decode(s), 16, axis=1)


# powers of two: the tensor scales keep every product and sum exact
EXACT_SCALES = dict(gx=0.5, gh=2.0 ** -4, gw1=2.0 ** -3, gw2=2.0 ** -2)


def _exact_weights(rng, E, H, I):
    W1 = [_grid_blocks(rng, 2 * I, H) * EXACT_SCALES["gw1"] for _ in range(E)]
    W2 = [_grid_blocks(rng, H, I) * EXACT_SCALES["gw2"] for _ in range(E)]
    q1 = [nvfp4.quantize_packed(w, EXACT_SCALES["gw1"]) for w in W1]
    q2 = [nvfp4.quantize_packed(w, EXACT_SCALES["gw2"]) for w in W2]
    W = (np.stack([q[0] for q in q1]), np.stack([q[1] for q in q1]),
         np.stack([q[0] for q in q2]), np.stack([q[1] for q in q2]))
    gw1 = np.full(E, EXACT_SCALES["gw1"], np.float32)
    gw2 = np.full(E, EXACT_SCALES["gw2"], np.float32)
    return W, gw1, gw2


@pytest.mark.parametrize("T,E,k", [(16, 4, 2), (77, 3, 1), (40, 1, 1)])
def test_nv_gemm1_accumulators_exact(T, E, k):
    """Every product (e2m1 * e4m3 * g)^2 is a multiple of 2^-9 below 2^3 and
    K = 512: fp32 sums are exact in any order, so the device's gate/up (sums
    times g_x * g_w1) must equal the oracle's fp64 ones bit for bit."""
    log(f"[test] nvfp4 gemm1 exact T={T} E={E} k={k}")
    H, I = 512, 256
    rng = np.random.default_rng(31 + T)
    xb = bf16.encode(_grid_blocks(rng, T, H) * EXACT_SCALES["gx"])
    W, gw1, gw2 = _exact_weights(rng, E, H, I)
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    w = np.full((T, k), 1.0 / k, np.float32)
    ts = (EXACT_SCALES["gx"], EXACT_SCALES["gh"], gw1, gw2)
    layer = nv_layer(H, I, E, k, T)
    layer.load_canonical(*(dev(a) for a in W), tensor_scales=ts)
    acc = torch.full((T * k, 2 * I), float("nan"), device="cuda")
    layer.run_stages(Q | RT | G1, T, x=dev_bf16(xb), topk_ids=dev(ids), gemm1_acc=acc)
    torch.cuda.synchronize()
    ref = forward(xb, ids, w, W, E, I, keep_acc=True, mma_type="nvf4xnvf4", tensor_scales=ts)
    got = nv_workspace_host(layer, T)
    assert np.array_equal(got["xq"], ref["xq"]) and np.array_equal(got["xsf"], ref["xsf"])
    assert np.array_equal(acc.cpu().numpy()[:ref["acc"].shape[0]].astype(np.float64), ref["acc"])


def test_nv_gemm2_exact_on_injected_rows():
    """GEMM2 alone on NVFP4 rows of h and a routing written by the test: the
    sums are exact, so y is the exact product rounded once to bf16."""
    log("[test] nvfp4 gemm2 exact on injected h")
    H, I, E, k, T = 512, 256, 5, 2, 37
    rng = np.random.default_rng(41)
    W, gw1, gw2 = _exact_weights(rng, E, H, I)
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    counts, offsets, srt, pos = route(ids, E)
    gh = EXACT_SCALES["gh"]
    hq, hsf = nvfp4.quantize_packed(_grid_blocks(rng, srt.size, I) * gh, gh)
    layer = nv_layer(H, I, E, k, T)
    layer.load_canonical(*(dev(a) for a in W), tensor_scales=(EXACT_SCALES["gx"], gh, gw1, gw2))
    ws = layer.ws
    ws("counts", (E,), torch.int32).copy_(torch.from_numpy(counts))
    ws("offsets", (E + 1,), torch.int32).copy_(torch.from_numpy(offsets))
    ws("hq", (I // 128, T * k, 64), torch.uint8)[:, :srt.size].copy_(torch.from_numpy(planes_from_rows(hq, I // 128)))
    ws("hsf", (I // 64, T * k, 4), torch.uint8)[:, :srt.size].copy_(torch.from_numpy(planes_from_rows(hsf, I // 64)))
    layer.run_stages(G2, T)
    torch.cuda.synchronize()
    y = host_bits(ws("y", (T * k, H), torch.bfloat16)[:srt.size])
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        ref = expert_gemm2(hq[lo:hi], hsf[lo:hi], W[2][e], W[3][e], NvTensor(gh), NvTensor(gw2[e]))
        assert np.array_equal(y[lo:hi], bf16.encode(ref)), e


SHAPES = [
    synth.CONFIGS[0],                                                        # one 16-row tile
    synth.LayerConfig(120, "nv_h512_i256_e8_k2_t24_zipf", 24, 512, 256, 8, 2, "zipf", 120, 1.5),
    synth.LayerConfig(121, "nv_h1024_i512_e16_k2_t100", 100, 1024, 512, 16, 2, "uniform", 121),
    synth.LayerConfig(122, "nv_h512_i256_e4_k1_t60_zipf", 60, 512, 256, 4, 1, "zipf", 122, 1.5),
    synth.LayerConfig(123, "nv_h1024_i512_e16_k1_t160_empty_zipf", 160, 1024, 512, 16, 1, "zipf", 123, 2.0),
    synth.LayerConfig(124, "nv_h512_i256_e8_k2_t600", 600, 512, 256, 8, 2, "uniform", 124),   # tiled, 2 tiles
    synth.LayerConfig(125, "nv_h1024_i512_e16_k2_t1000", 1000, 1024, 512, 16, 2, "uniform", 125),  # tiled, 1 tile
    synth.LayerConfig(126, "nv_h1024_i512_e8_k2_t1500_zipf", 1500, 1024, 512, 8, 2, "zipf", 126, 1.1),
    synth.LayerConfig(127, "nv_h768_i384_e8_k2_t400", 400, 768, 384, 8, 2, "uniform", 127),   # odd blocks: streaming
    synth.LayerConfig(128, "nv_h4096_i2048_e8_k2_t512", 512, 4096, 2048, 8, 2, "uniform", 128),  # XCD-paired order
]


def run_nv(layer, x, ids, w, ts):
    T = x.shape[0]
    out = layer.forward(dev_bf16(x), dev(ids), dev(w))
    torch.cuda.synchronize()
    return dict(out=host_bits(out), **nv_workspace_host(layer, T))


def check_nv_stages(got, ref, gh, rows=None):
    """Every intermediate against the oracle (rows: sorted-row positions to
    compare, default all)."""
    for name in ("xq", "xsf", "counts", "offsets", "sorted_rows", "pos"):
        assert np.array_equal(got[name], ref[name]), name
    sel = slice(None) if rows is None else rows
    g_hq, g_hsf, r_hq, r_hsf = got["hq"][sel], got["hsf"][sel], ref["hq"][sel], ref["hsf"][sel]
    st = parity.nv_compare_requant(g_hq, g_hsf, r_hq, r_hsf, ref["h"][sel], gh)
    assert np.all(r_hsf < 0x7E), "calibration: a block of h saturated"
    exact = parity.same_h_rows(g_hq, g_hsf, r_hq, r_hsf)
    err_y, same_y = parity.check_y(got["y"][sel], ref["y"][sel], exact_rows=exact)
    return st, err_y, same_y


@pytest.mark.parametrize("cfg", SHAPES, ids=lambda c: c.name)
def test_nv_layer_all_tokens(cfg):
    log(f"[test] nvfp4 layer {cfg.name}")
    x = synth.make_tokens(cfg)
    ids, w = synth.make_routing(cfg)
    if cfg.index == 0:
        ids = ids.copy()
        ids[0, 1] = -1                 # a masked slot
        ids[2, 1] = ids[2, 0]          # a duplicate expert
    W, gw1, gw2 = all_expert_weights_nv(cfg)
    gx, gh = nv_act_scales(cfg, x)
    ts = (gx, gh, gw1, gw2)
    layer = nv_layer(cfg.hidden, cfg.inter, cfg.experts, cfg.topk, cfg.tokens)
    layer.load_canonical(*(dev(a) for a in W), tensor_scales=ts)
    got = run_nv(layer, x, ids, w, ts)
    counts = got["counts"]
    log(f"    rows per expert {counts.tolist()}")
    rows_hint = -(-int(counts.sum()) // cfg.experts)
    if cfg.name.endswith("zipf") and rows_hint <= 16:
        assert counts.max() > 16                                  # more than one pass over the weights
    if cfg.name.endswith("zipf") and rows_hint > 16:
        assert counts.max() > 2 * 128                             # a hot expert with several 128-row tiles
    ref = forward(x, ids, w, W, cfg.experts, cfg.inter, mma_type="nvf4xnvf4", tensor_scales=ts)
    st, err_y, same_y = check_nv_stages(got, ref, gh)
    err = parity.rel_l2(bf16.decode(got["out"]), ref["out_f64"])
    log(f"    requant {st}  y rel-L2 {err_y:.2e} bf16-equal {same_y:.5f}  out rel-L2 {err:.2e}")
    assert err <= parity.OUT_REL_L2
    again = run_nv(layer, x, ids, w, ts)
    assert np.array_equal(again["out"], got["out"])               # deterministic


@pytest.fixture(scope="module")
def dsv4_nv_layer():
    """The DSV4-shaped layer with the synthetic weights quantized to NVFP4 on
    the device (fixed tensor scales), and its canonical buffers."""
    cfg = synth.CONFIGS[2]
    layer = nv_layer(cfg.hidden, cfg.inter, cfg.experts, cfg.topk, cfg.tokens)
    g1, g2 = NV_WEIGHT_SCALES
    log("[fixture] quantizing the DSV4 weights to NVFP4 on the device")
    x = synth.make_tokens(cfg)
    gx, gh = nv_act_scales(cfg, x)
    bufs = layer.load_fp32(lambda e: synth.expert_weights_f32(cfg, e), keep_canonical=True,
                           tensor_scales=(gx, gh, np.full(cfg.experts, g1, np.float32),
                                          np.full(cfg.experts, g2, np.float32)))
    torch.cuda.synchronize()
    yield layer, bufs, (gx, gh)
    del layer, bufs
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cfg_index", [1, 2, 3, 4])
def test_nv_dsv4_sampled_tokens(dsv4_nv_layer, cfg_index):
    cfg = synth.CONFIGS[cfg_index]
    big, bufs, (gx, gh) = dsv4_nv_layer
    log(f"[test] nvfp4 DSV4 {cfg.name}: every routed row of sampled tokens")
    layer = big.with_capacity(cfg.tokens)
    x = synth.make_tokens(cfg)
    ids, w = synth.make_routing(cfg)
    got = run_nv(layer, x, ids, w, None)
    rng = np.random.default_rng(cfg_index)
    toks = sorted(rng.choice(cfg.tokens, 2, replace=False).tolist())
    getter = lazy_expert_weights_nv(cfg, NV_WEIGHT_SCALES)
    E = cfg.experts
    ts = (gx, gh, np.full(E, NV_WEIGHT_SCALES[0], np.float32), np.full(E, NV_WEIGHT_SCALES[1], np.float32))
    ref = forward(x, ids, w, getter, E, cfg.inter, tokens=toks, mma_type="nvf4xnvf4", tensor_scales=ts)
    # the device's NVFP4 weights of the sampled tokens' experts equal the oracle's
    experts = sorted({int(e) for t in toks for e in ids[t]})
    for e in experts:
        for mine, theirs in zip((b[e].cpu().numpy() for b in bufs), getter(e)):
            assert np.array_equal(mine, theirs), e
    rows = np.sort(np.array([p for t in toks for p in ref["pos"][t * cfg.topk:(t + 1) * cfg.topk] if p >= 0]))
    for name in ("xq", "xsf", "counts", "offsets", "sorted_rows", "pos"):
        assert np.array_equal(got[name], ref[name]), name
    st, err_y, same_y = check_nv_stages(got, ref, gh, rows=rows)
    err = parity.rel_l2(bf16.decode(got["out"][toks]), ref["out_f64"][toks])
    log(f"    rows {rows.size} requant {st}  y rel-L2 {err_y:.2e} bf16-equal {same_y:.5f}  out rel-L2 {err:.2e}")
    assert err <= parity.OUT_REL_L2

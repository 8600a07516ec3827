"""GPU tier for the single-launch forward (moe_w4a4_forward_mega), compared
with the oracle on every token and every intermediate it leaves in the
workspace (quantized tokens, route, requantized h, y, output):

  mega_h512_i512_e8_k2_t16         K slices of one step (H = I = 512)
  mega_h1024_i512_e16_k2_t64_zipf  experts with more than 16 rows (several
                                   passes per work item) and experts with none
  mega_h2048_i1024_e64_k6_t42      252 routed rows
  mega_h512_i4096_e8_k2_t24        8-step GEMM2 slices (one W2 unit per item)
  mega_h4096_i512_e16_k4_t16       8-step GEMM1 slices, 1-step GEMM2 slices
  DSV4-Flash shape, T = 1, 8, 42   the 8- and 4-step slices of hidden 4096 and
                                   inter 2048 (6, 48 and 252 routed rows)

plus routing edge cases (masked, out-of-range and duplicate ids, a token with
no valid slot, one token, 256 routed rows), determinism, back-to-back calls
with different token counts on one workspace interleaved with the multi-launch
forward, a HIP graph replayed on new inputs, and the error word of the
kernel's bounded waits staying 0.  The fp8xfp4 type (E4M3 tokens and h, 8-row
GEMM1 passes) on the same shapes, the DSV4 sizes and two edge cases, held to
its oracle and the MFMA model's element rules on every row.  The kernel's
token encoder of both types on every finite bf16 pattern."""
import dataclasses
import functools
import zlib

import numpy as np
import pytest
import torch

import synth
from oracle.forward import forward
from tests.gpu_support import dev, dev_bf16, host_bits, layer_for, log, run_config, run_inputs, synth_layer
from tests.oracle_inputs import all_expert_weights, all_experts_parallel
from tests.test_gpu_layer import check_all_stages

pytestmark = pytest.mark.gpu
FP8 = 1   # MOE_MMA_FP8_X_MXF4

SHAPES = [
    synth.LayerConfig(140, "mega_h512_i512_e8_k2_t16", 16, 512, 512, 8, 2, "uniform", 140),
    synth.LayerConfig(141, "mega_h1024_i512_e16_k2_t64_zipf", 64, 1024, 512, 16, 2, "zipf", 141, 2.0),
    synth.LayerConfig(142, "mega_h2048_i1024_e64_k6_t42", 42, 2048, 1024, 64, 6, "uniform", 142),
    synth.LayerConfig(143, "mega_h512_i4096_e8_k2_t24", 24, 512, 4096, 8, 2, "uniform", 143),
    synth.LayerConfig(144, "mega_h4096_i512_e16_k4_t16", 16, 4096, 512, 16, 4, "uniform", 144),
]
DSV4_TOKENS = [1, 8, 42]


@functools.lru_cache(maxsize=1)
def dsv4_weights():
    """e -> the oracle's MXFP4 weights of DSV4 expert e (both MMA types)."""
    return all_experts_parallel(synth.CONFIGS[1])


@functools.lru_cache(maxsize=4)
def stacked_weights(cfg):
    W = all_expert_weights(cfg)
    return W, (lambda e: (W[0][e], W[1][e], W[2][e], W[3][e]))


def err_word(layer):
    """The kernel's error word (a wait that ran out of polls sets it); the
    rest of the state region must be back at zero after every call."""
    from block_scaled_fp4_pre_amd import _lib
    st = layer.ws("mega", (_lib.MOE_MEGA_STATE_BYTES // 8,), torch.int64).cpu().numpy()
    err = int(st[_lib.MOE_MEGA_ERR_WORD])
    st[_lib.MOE_MEGA_ERR_WORD] = 0
    assert not st.any(), np.nonzero(st)[0][:8]
    return err


@pytest.fixture(scope="module")
def layers():
    out = {}
    for cfg in SHAPES:
        layer = layer_for(cfg.hidden, cfg.inter, cfg.experts, cfg.topk, cfg.tokens)
        layer.load_fp32(lambda e, c=cfg: synth.expert_weights_f32(c, e), threads=4)
        out[cfg.name] = layer
    return out


@pytest.mark.parametrize("cfg", SHAPES, ids=lambda c: c.name)
def test_mega_all_tokens(cfg, layers):
    log(f"[test] mega {cfg.name}")
    layer = layers[cfg.name]
    got = run_config(layer, cfg, mega=True)
    counts = got["counts"]
    log(f"    rows per expert: max {counts.max()}, empty {(counts == 0).sum()}")
    if "zipf" in cfg.name:
        assert counts.max() > 16 and (counts == 0).any()
    ref = forward(got["x"], got["ids"], got["w"], all_expert_weights(cfg), cfg.experts, cfg.inter)
    check_all_stages(got, ref, cfg.topk)
    assert err_word(layer) == 0


@pytest.mark.parametrize("T", DSV4_TOKENS)
def test_mega_dsv4_every_row(T):
    cfg = dataclasses.replace(synth.CONFIGS[1], name=f"dsv4flash_t{T}", tokens=T)
    log(f"[test] mega DSV4-Flash T={T}")
    layer = synth_layer(1, T)
    got = run_config(layer, cfg, mega=True)
    log(f"    {int((got['counts'] > 0).sum())} active experts; oracle")
    ref = forward(got["x"], got["ids"], got["w"], dsv4_weights(), cfg.experts, cfg.inter)
    check_all_stages(got, ref, cfg.topk)
    assert err_word(layer) == 0


@pytest.mark.parametrize("cfg", SHAPES, ids=lambda c: c.name)
def test_mega_fp8_all_tokens(cfg, layers):
    log(f"[test] mega fp8xfp4 {cfg.name}")
    layer = layers[cfg.name].with_capacity(cfg.tokens, mma_type=FP8)
    got = run_config(layer, cfg, mega=True)
    counts = got["counts"]
    log(f"    rows per expert: max {counts.max()}, empty {(counts == 0).sum()}")
    if "zipf" in cfg.name:
        assert counts.max() > 16 and (counts == 0).any()    # several 8-row GEMM1 passes
    W, getter = stacked_weights(cfg)
    ref = forward(got["x"], got["ids"], got["w"], W, cfg.experts, cfg.inter, mma_type="fp8xfp4")
    check_all_stages(got, ref, cfg.topk, weights=getter)
    assert err_word(layer) == 0


@pytest.mark.parametrize("T", DSV4_TOKENS)
def test_mega_fp8_dsv4_every_row(T):
    cfg = dataclasses.replace(synth.CONFIGS[1], name=f"dsv4flash_t{T}", tokens=T)
    log(f"[test] mega fp8xfp4 DSV4-Flash T={T}")
    layer = synth_layer(1, T, FP8)
    got = run_config(layer, cfg, mega=True)
    log(f"    {int((got['counts'] > 0).sum())} active experts; oracle")
    W = dsv4_weights()
    ref = forward(got["x"], got["ids"], got["w"], W, cfg.experts, cfg.inter, mma_type="fp8xfp4")
    check_all_stages(got, ref, cfg.topk, weights=W)
    assert err_word(layer) == 0


@pytest.mark.parametrize("mma", [0, FP8], ids=["mxf4xmxf4", "fp8xfp4"])
def test_mega_quantizes_every_bf16_pattern(mma):
    """The kernel's token encoder (the one its GEMM1 items use for their
    tiles; block 0 writes its x-hat to the workspace) on every finite bf16
    pattern as a lone value of its 32-group, at positions 0 and 17: codes and
    scales bit-exact against the oracle's quantizer, in two calls of 255
    tokens of hidden 4096."""
    from oracle import bf16, mxfp4, mxfp8
    log(f"[test] mega quantize: every finite bf16 pattern, mma_type {mma}")
    H, I, E = 4096, 512, 8
    bits = np.arange(1 << 16, dtype=np.uint32)
    vals = bits[((bits >> 7) & 0xFF) != 0xFF].astype(np.uint16)      # 65280 finite patterns
    grp = np.zeros((vals.size, 32), np.uint16)
    grp[:, 0] = vals
    grp[:, 17] = vals[::-1]
    T = 255
    x_all = grp.reshape(-1, T, H)                                     # 2 calls of 255 tokens x 128 groups
    assert x_all.shape[0] == 2
    rng = np.random.default_rng(5)
    layer = layer_for(H, I, E, 1, T, mma_type=mma)
    layer.load_fp32(lambda e: ((rng.standard_normal((2 * I, H)) * 0.02).astype(np.float32),
                               (rng.standard_normal((H, I)) * 0.02).astype(np.float32)), threads=1)
    ids = (np.arange(T, dtype=np.int32) % E).reshape(T, 1)
    w = np.ones((T, 1), np.float32)
    for x in x_all:
        layer.forward_mega(dev_bf16(x), dev(ids), dev(w))
        torch.cuda.synchronize()
        xq = layer.ws("xq", (T, H if mma else H // 2), torch.uint8).cpu().numpy()
        xsf = layer.ws("xsf", (T, H // 32), torch.uint8).cpu().numpy()
        rc, rs = (mxfp8.quantize if mma else mxfp4.quantize_packed)(bf16.decode(x))
        assert np.array_equal(xsf, rs)
        assert np.array_equal(xq, rc)
    assert err_word(layer) == 0


@pytest.mark.parametrize("case", ["T1", "masked_dups", "no_valid_slot", "rows256", "fp8_masked_dups",
                                  "fp8_rows256"])
def test_mega_edge_cases(case, layers):
    log(f"[test] mega edge case {case}")
    fp8 = case.startswith("fp8_")
    case = case[4:] if fp8 else case
    cfg = SHAPES[0]
    E, k = cfg.experts, cfg.topk
    rng = np.random.default_rng(zlib.crc32(case.encode()))
    T = {"T1": 1, "rows256": 128}.get(case, 16)
    x = synth.f32_to_bf16_bits(rng.standard_normal((T, cfg.hidden)).astype(np.float32))
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    if case == "masked_dups":
        ids[::3, 1] = -1
        ids[1::3, 1] = ids[1::3, 0]
        ids[7, 0] = E + 3
    if case == "no_valid_slot":
        ids[4, :] = -1
        ids[9, :] = E
    layer = layers[cfg.name].with_capacity(max(T, cfg.tokens), mma_type=FP8 if fp8 else 0)
    got = run_inputs(layer, x, ids, w, mega=True)
    W, getter = stacked_weights(cfg)
    ref = forward(x, ids, w, W, E, cfg.inter, mma_type="fp8xfp4" if fp8 else "mxf4xmxf4")
    check_all_stages(got, ref, k, weights=getter if fp8 else None)
    if case == "no_valid_slot":
        assert np.all(got["out"][4] == 0) and np.all(got["out"][9] == 0)
    assert err_word(layer) == 0


def test_mega_deterministic_and_reusable(layers):
    """Two identical calls give identical bits; calls with other token counts
    and multi-launch forwards in between leave the next call unaffected."""
    log("[test] mega determinism and workspace reuse")
    cfg = SHAPES[2]
    layer = layers[cfg.name]
    x = synth.make_tokens(cfg)
    ids, w = synth.make_routing(cfg)
    xd, idd, wd = dev_bf16(x), dev(ids), dev(w)
    first = host_bits(layer.forward_mega(xd, idd, wd))
    for T in (1, 5, 42, 17):
        layer.forward_mega(xd[:T], idd[:T], wd[:T])
        layer.forward(xd[:T], idd[:T], wd[:T])
    again = host_bits(layer.forward_mega(xd, idd, wd))
    torch.cuda.synchronize()
    assert np.array_equal(first, again)
    multi = host_bits(layer.forward(xd, idd, wd))
    log(f"    multi-launch vs single-launch outputs bit-identical on {float(np.mean(multi == first)):.4f}")
    assert err_word(layer) == 0


def test_forward_takes_the_single_launch_path_for_few_rows(layers):
    """moe_w4a4_forward runs the single-launch kernel up to MOE_MEGA_AUTO_ROWS
    routed rows (its output then equals moe_w4a4_forward_mega's bit for bit),
    and so does the allocation-free forward on the library's static scratch."""
    from block_scaled_fp4_pre_amd import _lib
    log("[test] automatic single-launch path")
    cfg = SHAPES[2]
    layer = layers[cfg.name]
    T = _lib.MOE_MEGA_AUTO_ROWS // cfg.topk
    x = synth.make_tokens(cfg)[:T]
    ids, w = synth.make_routing(cfg)
    xd, idd, wd = dev_bf16(x), dev(ids[:T]), dev(w[:T])
    mega = host_bits(layer.forward_mega(xd, idd, wd))
    auto = host_bits(layer.forward(xd, idd, wd))
    out = torch.empty((T, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    for _ in range(2):                          # the scratch's state region is left zero for the next call
        _lib.moe_w4a4_forward_noalloc(layer.cfg, layer.prepared, T, xd, idd, wd, out)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(out), mega)
    assert np.array_equal(auto, mega)
    assert err_word(layer) == 0


def test_fp8_forward_takes_the_single_launch_path_for_few_rows(layers):
    """The same for the fp8xfp4 type, up to MOE_MEGA_AUTO_ROWS_FP8 routed rows."""
    from block_scaled_fp4_pre_amd import _lib
    log("[test] automatic single-launch path, fp8xfp4")
    cfg = SHAPES[2]
    layer = layers[cfg.name].with_capacity(cfg.tokens, mma_type=FP8)
    T = _lib.MOE_MEGA_AUTO_ROWS_FP8 // cfg.topk
    x = synth.make_tokens(cfg)[:T]
    ids, w = synth.make_routing(cfg)
    xd, idd, wd = dev_bf16(x), dev(ids[:T]), dev(w[:T])
    mega = host_bits(layer.forward_mega(xd, idd, wd))
    auto = host_bits(layer.forward(xd, idd, wd))
    out = torch.empty((T, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    _lib.moe_w4a4_forward_noalloc(layer.cfg, layer.prepared, T, xd, idd, wd, out)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out), mega)
    assert np.array_equal(auto, mega)
    assert err_word(layer) == 0


def test_mega_wait_that_gives_up_sets_the_error_word_and_drains(layers):
    """Failure handling, forced from the host: the per-expert h counts are
    set beforehand to a value they can never count to, so every GEMM2 item's
    bounded wait gives up.  The launch still ends (the first wait to give up
    sets the abort word, after which no wait waits), the error word reads 1
    and the rest of the state region is back at zero; with the error word
    cleared, the next call gives the clean call's bits again."""
    from block_scaled_fp4_pre_amd import _lib
    log("[test] mega: a wait that gives up")
    cfg = SHAPES[0]
    layer = layers[cfg.name].with_capacity(cfg.tokens)
    x = synth.make_tokens(cfg)
    ids, w = synth.make_routing(cfg)
    xd, idd, wd = dev_bf16(x), dev(ids), dev(w)
    clean = host_bits(layer.forward_mega(xd, idd, wd))
    torch.cuda.synchronize()
    assert err_word(layer) == 0
    st = layer.ws("mega", (_lib.MOE_MEGA_STATE_BYTES // 8,), torch.int64)
    st[_lib.MOE_MEGA_HCOUNT_WORD:_lib.MOE_MEGA_HCOUNT_WORD + cfg.experts] = 1 << 40
    torch.cuda.synchronize()
    layer.forward_mega(xd, idd, wd)
    torch.cuda.synchronize()
    assert err_word(layer) == 1                 # and every other word zero again
    st[_lib.MOE_MEGA_ERR_WORD] = 0
    again = host_bits(layer.forward_mega(xd, idd, wd))
    torch.cuda.synchronize()
    assert err_word(layer) == 0
    assert np.array_equal(again, clean)


def test_mega_graph_replays_equal_eager(layers):
    log("[test] mega graph capture and replay")
    cfg = SHAPES[1]
    layer = layers[cfg.name]
    sets = []
    for i in range(2):
        c = dataclasses.replace(cfg, index=cfg.index + 500 * i)
        ids, w = synth.make_routing(c)
        sets.append((dev_bf16(synth.make_tokens(c)), dev(ids), dev(w)))
    eager = [host_bits(layer.forward_mega(*s)) for s in sets]
    torch.cuda.synchronize()
    assert not np.array_equal(eager[0], eager[1])
    x_s, ids_s, w_s = (t.clone() for t in sets[0])
    out_s = torch.empty((cfg.tokens, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.forward_mega(x_s, ids_s, w_s, out=out_s)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward_mega(x_s, ids_s, w_s, out=out_s)
    torch.cuda.synchronize()
    for i, which in enumerate((1, 0, 1)):
        for dst, src in zip((x_s, ids_s, w_s), sets[which]):
            dst.copy_(src)
        g.replay()
        torch.cuda.synchronize()
        got = host_bits(out_s)
        log(f"    replay {i} on input set {which}: bit-identical {np.array_equal(got, eager[which])}")
        assert np.array_equal(got, eager[which])
        assert np.array_equal(host_bits(layer.forward_mega(*sets[1 - which])), eager[1 - which])
        torch.cuda.synchronize()
    assert err_word(layer) == 0

"""GPU tier, whole forward through moe_w4a4_forward, against the oracle:
the tiny configuration, odd shapes and routing edge cases, determinism."""
import zlib

import numpy as np
import pytest
import torch

import synth
from oracle.forward import forward
from tests.gpu_support import dev, dev_bf16, host_bits, layer_for, log, run_config, run_inputs
from tests.oracle_inputs import all_expert_weights
from tests.parity import OUT_REL_L2, check_y, compare_requant, fp8_model_checks, rel_l2, same_h_rows

pytestmark = pytest.mark.gpu
TINY = synth.CONFIGS[0]


def check_all_stages(got, ref, k, weights=None):
    """weights: for the fp8xfp4 MMA type (E4M3 codes for x and h), e -> the
    oracle's (W1 codes, W1 scales, W2 codes, W2 scales) of expert e, which the
    MFMA model's element rules need (on every row; with got["acc"], GEMM1's
    captured accumulators, checked bit for bit too)."""
    from oracle import bf16
    fp8 = weights is not None
    assert np.array_equal(got["xq"], ref["xq"]) and np.array_equal(got["xsf"], ref["xsf"])
    for key in ("counts", "offsets", "sorted_rows", "pos"):
        assert np.array_equal(got[key], ref[key]), key
    stats = compare_requant(got["hq"], got["hsf"], ref["hq"], ref["hsf"], ref["h"], fp8=fp8)
    exact = same_h_rows(got["hq"], got["hsf"], ref["hq"], ref["hsf"])
    if fp8:
        stats.update(fp8_model_checks(got, ref, k, weights))
    y_err, y_same = check_y(got["y"], ref["y"], exact, bf16_rule=not fp8)
    o_err = rel_l2(bf16.decode(got["out"]), ref["out_f64"])
    same = float(np.mean(got["out"] == ref["out"])) if got["out"].size else 1.0
    log(f"    requant {stats}  rows with identical h {int(exact.sum())}/{exact.size}  "
        f"y rel-L2 {y_err:.2e} (bf16-equal {y_same:.4f})  out rel-L2 {o_err:.2e}  "
        f"out bit-identical {same:.4f}")
    assert o_err <= OUT_REL_L2
    return o_err


@pytest.fixture(scope="module")
def tiny_layer():
    layer = layer_for(TINY.hidden, TINY.inter, TINY.experts, TINY.topk, 1024)
    layer.load_fp32(lambda e: synth.expert_weights_f32(TINY, e))
    return layer


@pytest.fixture(scope="module")
def tiny_weights():
    return all_expert_weights(TINY)


def test_tiny_config_end_to_end(tiny_layer, tiny_weights):
    log("[test] tiny config end to end")
    got = run_config(tiny_layer, TINY)
    ref = forward(got["x"], got["ids"], got["w"], tiny_weights, TINY.experts, TINY.inter)
    check_all_stages(got, ref, TINY.topk)


def _run_custom(layer, x, ids, w, acc=False):
    return run_inputs(layer, x, ids, w, acc=acc)


@pytest.mark.parametrize("case", ["T1", "T3", "T129", "T1000", "one_expert", "masked_dups", "zero_x"])
def test_tiny_dims_edge_cases(tiny_layer, tiny_weights, case):
    log(f"[test] edge case {case}")
    rng = np.random.default_rng(zlib.crc32(case.encode()))
    T = {"T1": 1, "T3": 3, "T129": 129, "T1000": 1000}.get(case, 200)
    E, k = TINY.experts, TINY.topk
    x = synth.f32_to_bf16_bits(rng.standard_normal((T, TINY.hidden)).astype(np.float32))
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    if case == "one_expert":
        ids[:, 0] = 5                       # 200 rows on one expert: many token tiles
        ids[:, 1] = rng.integers(0, 2, T)   # experts 2,3,4,6,7 get nothing
    if case == "masked_dups":
        ids[::3, 1] = -1
        ids[1::3, 1] = ids[1::3, 0]
        ids[5, :] = -1
        ids[7, 0] = E + 3
    if case == "zero_x":
        x[:] = 0
    got = _run_custom(tiny_layer, x, ids, w)
    ref = forward(x, ids, w, tiny_weights, E, TINY.inter)
    check_all_stages(got, ref, k)
    if case == "zero_x":
        assert np.all(got["out"] == 0) and np.all(got["xsf"] == 0)


def test_single_expert_single_slot():
    log("[test] E=1, k=1 dense MXFP4 MLP")
    H, I, T = 256, 128, 70
    rng = np.random.default_rng(3)
    W1 = (rng.standard_normal((1, 2 * I, H)) * 0.05).astype(np.float32)
    W2 = (rng.standard_normal((1, H, I)) * 0.05).astype(np.float32)
    layer = layer_for(H, I, 1, 1, T)
    layer.load_fp32(lambda e: (W1[e], W2[e]))
    x = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    ids = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1), np.float32)
    got = _run_custom(layer, x, ids, w)
    from oracle import mxfp4
    Wq = (*mxfp4.quantize_packed(W1[0].astype(np.float64)), *mxfp4.quantize_packed(W2[0].astype(np.float64)))
    ref = forward(x, ids, w, tuple(a[None] for a in Wq), 1, I)
    check_all_stages(got, ref, 1)


def test_forward_is_deterministic(tiny_layer):
    log("[test] determinism")
    cfg = TINY
    x = synth.make_tokens(cfg, 16)
    ids, w = synth.make_routing(cfg, 16)
    xs, idt, wt = dev_bf16(np.tile(x, (40, 1))), dev(np.tile(ids, (40, 1))), dev(np.tile(w, (40, 1)))
    a = host_bits(tiny_layer.forward(xs, idt, wt))
    b = host_bits(tiny_layer.forward(xs, idt, wt))
    assert np.array_equal(a, b)


def test_zero_tokens_is_a_no_op(tiny_layer):
    out = torch.full((4, TINY.hidden), 7.0, dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((0, TINY.hidden), dtype=torch.bfloat16, device="cuda")
    from block_scaled_fp4_pre_amd import _lib
    _lib.moe_w4a4_forward(tiny_layer.cfg, tiny_layer.prepared, 0, x, torch.zeros((0, 2), dtype=torch.int32,
                          device="cuda"), torch.zeros((0, 2), device="cuda"), out, tiny_layer.workspace)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


EXTREMES = [  # (E, k, T, H, I, mma_type)
    (5, 2, 37, 256, 128, 0), (7, 3, 1000, 256, 128, 0), (512, 8, 300, 256, 128, 0), (512, 16, 2000, 256, 128, 0),
    (6, 2, 40, 768, 384, 0), (6, 2, 600, 768, 384, 0), (6, 2, 40, 768, 384, 1), (6, 2, 600, 768, 384, 1),
    (4, 1, 40, 16384, 256, 0), (4, 1, 40, 8192, 256, 1), (4, 1, 40, 256, 8192, 1),
]


@pytest.mark.parametrize("E,k,T,H,I,mma", EXTREMES,
                         ids=[f"E{e}_k{k}_T{t}_H{h}_I{i}_{'fp8' if m else 'fp4'}" for e, k, t, h, i, m in EXTREMES])
def test_expert_count_extremes(E, k, T, H, I, mma):
    """Odd expert counts and the largest E and k the ABI takes, on every token:
    the streaming path (E5, E512_k8), the LDS-staged path (E7), and 32000
    routed rows, past the one-block pre-dispatch limit, so quantization and
    routing run as separate kernels (E512_k16).  Then H = 768, I = 384 (6 and
    3 K steps: the 2- and 1-slot weight rings and the 8- and 4-chunk token
    swizzles of the streaming GEMMs), streaming and LDS-staged, for both MMA
    types.  Last, K too long for a streaming GEMM's token tile to fit a CU's
    LDS at 10 rows per expert (H = 16384 with MXFP4 tokens; H = 8192 and
    I = 8192 with E4M3): those run on the LDS-staged path."""
    from oracle import mxfp4
    log(f"[test] E={E} k={k} T={T} H={H} I={I} mma_type={mma}")
    rng = np.random.default_rng(1000 * E + k + 7 * H + T)
    W1 = (rng.standard_normal((E, 2 * I, H)) * 0.05).astype(np.float32)
    W2 = (rng.standard_normal((E, H, I)) * 0.05).astype(np.float32)
    layer = layer_for(H, I, E, k, T, mma_type=mma)
    layer.load_fp32(lambda e: (W1[e], W2[e]), threads=4)
    x = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    got = _run_custom(layer, x, ids, w, acc=bool(mma))
    c1, s1 = mxfp4.quantize_packed(W1)
    c2, s2 = mxfp4.quantize_packed(W2)
    ref = forward(x, ids, w, (c1, s1, c2, s2), E, I, mma_type="fp8xfp4" if mma else "mxf4xmxf4",
                  keep_acc=bool(mma))
    weights = (lambda e: (c1[e], s1[e], c2[e], s2[e])) if mma else None
    check_all_stages(got, ref, k, weights=weights)

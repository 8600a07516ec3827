"""GPU tier at the full DeepSeek-V4-Flash shapes (hidden 4096, inter 2048, 256
experts, top-6), each on a workspace sized for its own token count, as the
benchmark launches them, for both MMA types:

  T = 64, 512   one whole oracle forward: every routed row's requantized h and
                y, and every token's output
  T = 4096      every row of the hottest, the coldest and the median expert
  T = 16384     and of the last expert in sorted order (positions up to R);
  (Zipf)        the output on the routed rows of sampled tokens

Quantized tokens and the routing are checked in full everywhere.  With the
fp8xfp4 type the MFMA model's element rules (tests/parity.py,
fp8_model_checks) run on the checked rows too, with GEMM1's accumulators
captured and compared bit for bit; on the hottest Zipf expert (12,666 rows)
the model covers its first and last 256 rows."""
import numpy as np
import pytest

import synth
from oracle import bf16, mxfp4, mxfp8
from oracle.forward import forward
from oracle.route import route
from tests.gpu_support import log, run_config, synth_layer
from tests.oracle_inputs import all_experts_parallel
from tests.parity import OUT_REL_L2, check_y, compare_requant, fp8_model_checks, rel_l2, same_h_rows
from tests.test_gpu_layer import check_all_stages

pytestmark = pytest.mark.gpu
DSV4 = [c for c in synth.CONFIGS if c.weight_set == 1]
MMA = {0: "mxf4xmxf4", 1: "fp8xfp4"}
MODEL_ROWS_PER_EXPERT = 512


def _layer(cfg, mma):
    return synth_layer(1, cfg.tokens, mma)


def _check_inputs_stages(got, cfg, fp8):
    q = mxfp8.quantize if fp8 else mxfp4.quantize_packed
    rq, rs = q(bf16.decode(got["x"]))
    assert np.array_equal(got["xq"], rq) and np.array_equal(got["xsf"], rs)
    counts, offsets, srt, pos = route(got["ids"], cfg.experts)
    for a, b in ((got["counts"], counts), (got["offsets"], offsets), (got["sorted_rows"], srt), (got["pos"], pos)):
        assert np.array_equal(a, b)
    return counts, offsets, pos


@pytest.mark.parametrize("mma", [0, 1], ids=lambda m: MMA[m])
@pytest.mark.parametrize("cfg", DSV4[:2], ids=lambda c: c.name)
def test_full_size_every_row(cfg, mma):
    fp8 = mma == 1
    layer = _layer(cfg, mma)
    log(f"[test] full size {cfg.name} {MMA[mma]}: forward")
    got = run_config(layer, cfg, acc=fp8)
    counts, _, _ = _check_inputs_stages(got, cfg, fp8)
    log(f"    xq/route exact; {int((counts > 0).sum())} active experts; oracle weights")
    W = all_experts_parallel(synth.CONFIGS[1])
    log("    oracle forward")
    ref = forward(got["x"], got["ids"], got["w"], W, cfg.experts, cfg.inter, mma_type=MMA[mma])
    log("    comparing")
    check_all_stages(got, ref, cfg.topk, weights=W if fp8 else None)


def _chosen_experts(counts):
    live = np.nonzero(counts)[0]
    order = live[np.argsort(counts[live], kind="stable")]
    return sorted({int(order[-1]), int(order[0]), int(order[len(order) // 2]), int(live[-1])})


@pytest.mark.parametrize("mma", [0, 1], ids=lambda m: MMA[m])
@pytest.mark.parametrize("cfg", DSV4[2:], ids=lambda c: c.name)
def test_full_size_chosen_experts(cfg, mma):
    fp8 = mma == 1
    layer = _layer(cfg, mma)
    x = synth.make_tokens(cfg)
    ids, _ = synth.make_routing(cfg)
    counts, offsets, _, _ = route(ids, cfg.experts)
    exps = _chosen_experts(counts)
    rows = np.concatenate([np.arange(offsets[e], offsets[e + 1]) for e in exps])
    model_rows = np.concatenate([np.unique(np.concatenate([
        np.arange(offsets[e], min(offsets[e] + MODEL_ROWS_PER_EXPERT // 2, offsets[e + 1])),
        np.arange(max(offsets[e + 1] - MODEL_ROWS_PER_EXPERT // 2, offsets[e]), offsets[e + 1])])) for e in exps])
    log(f"[test] full size {cfg.name} {MMA[mma]}: experts {exps} with {[int(counts[e]) for e in exps]} rows "
        f"(positions {rows.min()}..{rows.max()} of {int(counts.sum())})")
    got = run_config(layer, cfg, acc=fp8, acc_rows=model_rows if fp8 else None)
    _check_inputs_stages(got, cfg, fp8)
    W = all_experts_parallel(synth.CONFIGS[1])
    log("    oracle on the chosen experts")
    ref = forward(got["x"], got["ids"], got["w"], W, cfg.experts, cfg.inter, experts=exps, mma_type=MMA[mma])
    stats = compare_requant(got["hq"][rows], got["hsf"][rows], ref["hq"][rows], ref["hsf"][rows], ref["h"][rows],
                            fp8=fp8)
    exact = same_h_rows(got["hq"][rows], got["hsf"][rows], ref["hq"][rows], ref["hsf"][rows])
    y_err, y_same = check_y(got["y"][rows], ref["y"][rows], exact, bf16_rule=not fp8)
    if fp8:
        stats.update(fp8_model_checks(got, ref, cfg.topk, W, rows=model_rows))
    log(f"    requant {stats} y rel-L2 {y_err:.2e} (bf16-equal {y_same:.4f})")
    # the output of sampled tokens, which the oracle computes one by one
    rng = np.random.default_rng(cfg.index + 10 * mma)
    toks = sorted(rng.choice(cfg.tokens, 2, replace=False).tolist())
    ref_t = forward(got["x"], got["ids"], got["w"], W, cfg.experts, cfg.inter, tokens=toks, mma_type=MMA[mma])
    o_err = rel_l2(bf16.decode(got["out"][toks]), ref_t["out_f64"][toks])
    log(f"    out rel-L2 on tokens {toks}: {o_err:.2e}")
    assert o_err <= OUT_REL_L2

"""GPU tier at the full DeepSeek-V4-Flash shapes (hidden 4096, inter 2048, 256
experts, top-6) for T = 64, 512, 4096 and 16384 (Zipf routing), in the launch
configuration the benchmark times.  Quantized tokens and the routing are
checked in full; GEMM1/requant, GEMM2 and the output on the routed rows of a
few sampled tokens, which the oracle computes one by one."""
import numpy as np
import pytest
import torch

import synth
from oracle import bf16
from oracle.forward import forward
from oracle.route import route
from tests.gpu_support import log, run_config, synth_layer
from tests.oracle_inputs import lazy_expert_weights
from tests.parity import OUT_REL_L2, check_y, compare_requant, rel_l2, same_h_rows

pytestmark = pytest.mark.gpu
DSV4 = [c for c in synth.CONFIGS if c.weight_set == 1]
_oracle_weights = lazy_expert_weights(synth.CONFIGS[1])


@pytest.mark.parametrize("cfg", DSV4, ids=lambda c: c.name)
def test_full_size_sampled(cfg):
    layer = synth_layer(1, 16384)
    log(f"[test] full size {cfg.name}: forward")
    got = run_config(layer, cfg)
    x, ids, w = got["x"], got["ids"], got["w"]
    # pre-dispatch quantization and routing: complete
    from oracle import mxfp4
    rq, rs = mxfp4.quantize_packed(bf16.decode(x))
    assert np.array_equal(got["xq"], rq) and np.array_equal(got["xsf"], rs)
    counts, offsets, srt, pos = route(ids, cfg.experts)
    for a, b in ((got["counts"], counts), (got["offsets"], offsets), (got["sorted_rows"], srt), (got["pos"], pos)):
        assert np.array_equal(a, b)
    log(f"    xq/route exact; rows per expert max {counts.max()} min {counts.min()}")
    # sampled tokens through the oracle
    rng = np.random.default_rng(cfg.index)
    toks = sorted(rng.choice(cfg.tokens, 2, replace=False).tolist())
    log(f"    oracle on tokens {toks}")
    ref = forward(x, ids, w, _oracle_weights, cfg.experts, cfg.inter, tokens=toks)
    rows = np.array([pos[t * cfg.topk + j] for t in toks for j in range(cfg.topk) if pos[t * cfg.topk + j] >= 0])
    stats = compare_requant(got["hq"][rows], got["hsf"][rows], ref["hq"][rows], ref["hsf"][rows], ref["h"][rows])
    y_err, y_same = check_y(got["y"][rows], ref["y"][rows],
                            same_h_rows(got["hq"][rows], got["hsf"][rows], ref["hq"][rows], ref["hsf"][rows]))
    o_err = rel_l2(bf16.decode(got["out"][toks]), ref["out_f64"][toks])
    log(f"    requant {stats} y rel-L2 {y_err:.2e} (bf16-equal {y_same:.4f}) out rel-L2 {o_err:.2e}")
    assert o_err <= OUT_REL_L2

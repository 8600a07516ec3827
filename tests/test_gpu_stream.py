"""GPU tier for the streaming path (few routed rows per expert: weights streamed
through the register ring, the expert's token tile in LDS), compared with the
oracle on every token and every intermediate, at shapes the oracle finishes in
seconds:

  h1024_i512_e16  GEMM1 with 2 units per wave (4 unit groups per expert) and
                  GEMM2 with 4 workgroups per expert; two 16-row token tiles
  h512_i256_e8    16-row token tiles (about 6 rows per expert; the hot
                  expert's 19 take two passes)
  e4_k1_zipf      a hot expert with more rows than one pass holds (24): the
                  weights are streamed once per pass
  h1024_i512_e4_k1_zipf  the same with the 4-slot weight ring of the DSV4
                  shape's K loops (H and I multiples of 512)
  e16_k1_empty_zipf  two-tile launches (10 rows per expert on average) in
                  which 5 of the 16 experts get no rows: their workgroups
                  issue the first ring loads before reading the row count,
                  then wait for them and exit; the hot expert takes 5 passes"""
import numpy as np
import pytest

import synth
from oracle.forward import forward
from tests.gpu_support import layer_for, log, run_config
from tests.oracle_inputs import all_expert_weights
from tests.test_gpu_layer import check_all_stages

pytestmark = pytest.mark.gpu

SHAPES = [
    synth.LayerConfig(110, "stream_h1024_i512_e16_k2_t100", 100, 1024, 512, 16, 2, "uniform", 110),
    synth.LayerConfig(111, "stream_h512_i256_e8_k2_t24", 24, 512, 256, 8, 2, "zipf", 111, 1.1),
    synth.LayerConfig(112, "stream_h512_i256_e4_k1_t60_zipf", 60, 512, 256, 4, 1, "zipf", 112, 1.5),
    synth.LayerConfig(113, "stream_h1024_i512_e4_k1_t60_zipf", 60, 1024, 512, 4, 1, "zipf", 113, 1.5),
    synth.LayerConfig(114, "stream_h1024_i512_e16_k1_t160_empty_zipf", 160, 1024, 512, 16, 1, "zipf", 114, 2.0),
]


@pytest.mark.parametrize("cfg", SHAPES, ids=lambda c: c.name)
def test_stream_path_all_tokens(cfg):
    log(f"[test] stream {cfg.name}")
    layer = layer_for(cfg.hidden, cfg.inter, cfg.experts, cfg.topk, cfg.tokens)
    layer.load_fp32(lambda e: synth.expert_weights_f32(cfg, e), threads=4)
    got = run_config(layer, cfg)
    counts = got["counts"]
    log(f"    rows per expert {counts.tolist()}")
    assert -(-int(counts.sum()) // cfg.experts) <= 16          # the streaming path's range
    if cfg.name.endswith("zipf"):
        assert counts.max() > 24                                # a second pass over the weights
    if "empty" in cfg.name:
        assert -(-int(counts.sum()) // cfg.experts) > 8 and (counts == 0).any()   # two-tile form, empty experts
    ref = forward(got["x"], got["ids"], got["w"], all_expert_weights(cfg), cfg.experts, cfg.inter)
    check_all_stages(got, ref, cfg.topk)


"""GPU tier for the prefill path (many routed rows per expert: the tiled GEMMs
with both operands staged in LDS), compared with the oracle on every token and
every intermediate, at shapes the oracle finishes in seconds:

  h512_i512   4 K steps per GEMM; the generic work order (weight blocks per
              expert not a multiple of the 8 XCDs)
  h2048_i1024 16 / 8 K steps; the per-XCD paired work order
  h256_i128   2 / 1 K steps: fewer K steps than ring stages
  e16         about 125 rows per expert: each expert's mean fits one tile, so
              weights load non-temporal and GEMM1 takes two weight blocks per
              workgroup; some experts spill into a second tile
  t600_e8     about 150 rows per expert: several tiles per expert, default
              load policy
  h1024_i512_e16_k2_t1000  about 125 rows per expert (the single-tile form)
              with one expert spilling into a second tile
  h512_i1024_e32_k4_t800_zipf0.7  Zipf(0.7) over 32 experts at about 100
              rows per expert: the single-tile form with several tiles on
              the hot experts

Zipf routing gives hot experts with several full 128-row tiles and a ragged
last tile, and cold experts with a single short tile."""
import numpy as np
import pytest
import torch

import synth
from oracle.forward import forward
from tests.gpu_support import layer_for, log, run_config
from tests.oracle_inputs import all_expert_weights
from tests.test_gpu_layer import check_all_stages

pytestmark = pytest.mark.gpu

SHAPES = [
    synth.LayerConfig(100, "prefill_h512_i512_e4_k2_t600", 600, 512, 512, 4, 2, "zipf", 100, 1.1),
    synth.LayerConfig(101, "prefill_h2048_i1024_e8_k2_t1500", 1500, 2048, 1024, 8, 2, "zipf", 101, 1.1),
    synth.LayerConfig(102, "prefill_h256_i128_e8_k2_t2000", 2000, 256, 128, 8, 2, "uniform", 102),
    synth.LayerConfig(103, "prefill_h512_i512_e16_k2_t1000", 1000, 512, 512, 16, 2, "uniform", 103),
    synth.LayerConfig(104, "prefill_h512_i512_e8_k2_t600", 600, 512, 512, 8, 2, "uniform", 104),
    synth.LayerConfig(105, "prefill_h1024_i512_e16_k2_t1000", 1000, 1024, 512, 16, 2, "uniform", 105),
    synth.LayerConfig(106, "prefill_h512_i1024_e32_k4_t800_zipf0.7", 800, 512, 1024, 32, 4, "zipf", 106, 0.7),
]


@pytest.mark.parametrize("cfg", SHAPES, ids=lambda c: c.name)
def test_prefill_path_all_tokens(cfg):
    log(f"[test] prefill {cfg.name}")
    layer = layer_for(cfg.hidden, cfg.inter, cfg.experts, cfg.topk, cfg.tokens)
    layer.load_fp32(lambda e: synth.expert_weights_f32(cfg, e), threads=4)
    torch.cuda.synchronize()
    got = run_config(layer, cfg)
    counts = got["counts"]
    log(f"    rows per expert {counts.tolist()}")
    assert counts.max() > 128 and (counts % 128).max() > 0      # several tiles and a ragged one
    ref = forward(got["x"], got["ids"], got["w"], all_expert_weights(cfg), cfg.experts, cfg.inter)
    check_all_stages(got, ref, cfg.topk)
    # the tiled GEMM1's token scales: those of sorted row q's token, bit for bit
    nv = int(counts.sum())
    assert np.array_equal(got["xsf_planes"], got["xsf"][got["sorted_rows"][:nv] // cfg.topk])
    # a second forward on the same workspace gives the same bits
    again = run_config(layer, cfg)
    assert np.array_equal(again["out"], got["out"]) and np.array_equal(again["hq"], got["hq"])

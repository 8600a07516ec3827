"""GPU tier for the fp8xfp4 MMA type (MXFP8 E4M3 activations, MXFP4 weights):
the same kernels with the token operand in FP8, compared with the oracle run
with mma_type="fp8xfp4".

  quantize        every bfloat16 pattern as a lone value in a group, through
                  the pre-dispatch quantization stage: codes and scales exact
  tiny / stream   the streaming path on every token (16- and 32-row passes,
                  2 units per wave in GEMM1; a two-tile launch in which 5 of
                  16 experts get no rows and the hot expert takes 5 passes)
  prefill         the LDS-staged path on every token: the per-XCD work order
                  with several tiles per expert, and the single-tile form
                  (non-temporal weights, two weight blocks per GEMM1 workgroup),
                  also with one expert spilling into a second tile, and with
                  Zipf(0.7) routing over 32 experts
Every row of these also goes through the MFMA model's element rules, with
GEMM1's accumulators captured and held to the model's bound (tests/parity.py,
fp8_model_checks).  The DeepSeek-V4-Flash shapes at full size are in
tests/test_gpu_fullsize.py."""
import numpy as np
import pytest
import torch

import synth
from block_scaled_fp4_pre_amd import _lib
from oracle import bf16, mxfp8
from oracle.forward import forward
from oracle.route import route
from tests.gpu_support import dev_bf16, layer_for, log, run_config
from tests.oracle_inputs import all_expert_weights
from tests.test_gpu_layer import check_all_stages

pytestmark = pytest.mark.gpu
FP8 = _lib.MOE_MMA_FP8_X_MXF4


def test_fp8_quantize_every_bf16_pattern():
    log("[test] fp8 quantize: every bf16 pattern")
    H = 256
    bits = np.arange(1 << 16, dtype=np.uint32)
    finite = np.isfinite((bits << 16).view(np.float32))
    vals = bits[finite].astype(np.uint16)
    T = -(-vals.size // (H // 32))
    x = np.zeros((T * (H // 32), 32), dtype=np.uint16)
    x[:vals.size, 9] = vals                    # one value per 32-group, the rest +0
    x = x.reshape(T, H)
    layer = layer_for(H, 128, 4, 1, T, mma_type=FP8)
    layer.run_stages(_lib.MOE_STAGE_QUANT, T, x=dev_bf16(x))
    torch.cuda.synchronize()
    xq = layer.ws("xq", (T, H), torch.uint8).cpu().numpy()
    xsf = layer.ws("xsf", (T, H // 32), torch.uint8).cpu().numpy()
    rq, rs = mxfp8.quantize(bf16.decode(x))
    assert np.array_equal(xsf, rs)
    assert np.array_equal(xq, rq)


SHAPES = [
    synth.CONFIGS[0],
    synth.LayerConfig(120, "fp8_stream_h1024_i512_e16_k2_t100", 100, 1024, 512, 16, 2, "uniform", 120),
    synth.LayerConfig(114, "fp8_stream_h1024_i512_e16_k1_t160_empty_zipf", 160, 1024, 512, 16, 1, "zipf", 114, 2.0),
    synth.LayerConfig(121, "fp8_prefill_h2048_i1024_e8_k2_t1500_zipf", 1500, 2048, 1024, 8, 2, "zipf", 121, 1.1),
    synth.LayerConfig(122, "fp8_prefill_h512_i512_e16_k2_t1000", 1000, 512, 512, 16, 2, "uniform", 122),
    synth.LayerConfig(123, "fp8_prefill_h1024_i512_e16_k2_t1000", 1000, 1024, 512, 16, 2, "uniform", 123),
    synth.LayerConfig(124, "fp8_prefill_h512_i1024_e32_k4_t800_zipf0.7", 800, 512, 1024, 32, 4, "zipf", 124, 0.7),
]


@pytest.mark.parametrize("cfg", SHAPES, ids=lambda c: c.name)
def test_fp8_all_tokens(cfg):
    log(f"[test] fp8 {cfg.name}")
    layer = layer_for(cfg.hidden, cfg.inter, cfg.experts, cfg.topk, cfg.tokens, mma_type=FP8)
    layer.load_fp32(lambda e: synth.expert_weights_f32(cfg, e), threads=4)
    got = run_config(layer, cfg, acc=True)
    log(f"    rows per expert {got['counts'].tolist()[:16]}")
    W = all_expert_weights(cfg)
    ref = forward(got["x"], got["ids"], got["w"], W, cfg.experts, cfg.inter, mma_type="fp8xfp4")
    check_all_stages(got, ref, cfg.topk, weights=lambda e: (W[0][e], W[1][e], W[2][e], W[3][e]))
    if cfg.tokens * cfg.topk > 16 * cfg.experts:     # the LDS-staged path: its GEMM1 scale planes
        nv = int(got["counts"].sum())
        assert np.array_equal(got["xsf_planes"], got["xsf"][got["sorted_rows"][:nv] // cfg.topk])
    again = run_config(layer, cfg)
    assert np.array_equal(again["out"], got["out"]) and np.array_equal(again["hq"], got["hq"])

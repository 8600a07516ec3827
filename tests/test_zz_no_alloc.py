"""moe_w4a4_forward_noalloc (the forward on the library's static scratch, for
callers that cannot allocate) against moe_w4a4_forward on a caller-owned
workspace, through the C ABI: two calls in a row, the second with fewer
tokens, on both GEMM paths (many rows per expert: LDS-staged tiles; few:
weight streaming), for all three MMA types.  The forward is deterministic, so the
outputs must be bit-identical.  A size past the scratch is refused on the
host with MOE_ESCRATCH."""
import numpy as np
import pytest
import torch

import synth
from block_scaled_fp4_pre_amd import _lib
from tests.gpu_support import dev, dev_bf16, host_bits, layer_for, log

pytestmark = pytest.mark.gpu

CFG = synth.LayerConfig(130, "noalloc_h1024_i512_e8_k2", 2000, 1024, 512, 8, 2, "uniform", 130)


def _inputs(T, seed):
    cfg = synth.LayerConfig(CFG.index + seed, CFG.name, T, CFG.hidden, CFG.inter, CFG.experts, CFG.topk,
                            CFG.routing, CFG.weight_set)
    x = synth.make_tokens(cfg)
    ids, w = synth.make_routing(cfg)
    return dev_bf16(x), dev(ids), dev(w)


# NVFP4 tensor scales (x, h, W1, W2): calibration constants above the
# synthetic data's absolute maxima
NV_SCALES = (2.0 ** -8, 8.0 / 2688, 6.1e-5, 5.3e-5)


@pytest.mark.parametrize("mma", [_lib.MOE_MMA_MXF4_X_MXF4, _lib.MOE_MMA_FP8_X_MXF4, _lib.MOE_MMA_NVF4_X_NVF4],
                         ids=["mxf4xmxf4", "fp8xfp4", "nvf4xnvf4"])
def test_noalloc_forward_matches_the_workspace_forward(mma):
    log(f"[test] no-alloc forward, mma_type {mma}")
    layer = layer_for(CFG.hidden, CFG.inter, CFG.experts, CFG.topk, CFG.tokens, mma_type=mma)
    ts = None
    if mma == _lib.MOE_MMA_NVF4_X_NVF4:
        gx, gh, g1, g2 = NV_SCALES
        ts = (gx, gh, np.full(CFG.experts, g1, np.float32), np.full(CFG.experts, g2, np.float32))
    layer.load_fp32(lambda e: synth.expert_weights_f32(CFG, e), threads=4, tensor_scales=ts)
    torch.cuda.synchronize()
    for T, seed in ((2000, 1), (50, 2)):        # 250 then 13 rows per expert: tiled, then streaming
        x, ids, w = _inputs(T, seed)
        log(f"    T={T}")
        ref = layer.forward(x, ids, w)
        got = torch.full_like(ref, float("nan"))
        _lib.moe_w4a4_forward_noalloc(layer.cfg, layer.prepared, T, x, ids, w, got)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(got), host_bits(ref)), T


def test_noalloc_refuses_more_than_its_scratch():
    log("[test] no-alloc forward past its scratch")
    H, I, E, k = 4096, 2048, 16, 6
    cfg = _lib.make_cfg(H, I, E, k, 4096)
    T = 4096
    lay = _lib.moe_w4a4_workspace_layout(_lib.make_cfg(H, I, E, k, T))
    assert lay["total"] > _lib.MOE_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros((T, k), dtype=torch.int32, device="cuda")
    w = torch.zeros((T, k), dtype=torch.float32, device="cuda")
    out = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    prep = torch.zeros(256, dtype=torch.uint8, device="cuda")      # never read: refused before any launch
    with pytest.raises(_lib.MoeError) as ei:
        _lib.moe_w4a4_forward_noalloc(cfg, prep, T, x, ids, w, out)
    assert ei.value.status == _lib.MOE_ESCRATCH
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0

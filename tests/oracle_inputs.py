"""Test-side assembly of oracle inputs: synthetic fp32 weights quantized by the
oracle's own MXFP4 or NVFP4 quantizer (never by the device path), and the
NVFP4 tensor scales the tests use."""
import functools

import numpy as np

import synth
from oracle import mxfp4, nvfp4


def quantize_expert(cfg, e):
    w1, w2 = synth.expert_weights_f32(cfg, e)
    w1c, w1s = mxfp4.quantize_packed(w1)
    w2c, w2s = mxfp4.quantize_packed(w2)
    return w1c, w1s, w2c, w2s


def all_expert_weights(cfg):
    parts = [quantize_expert(cfg, e) for e in range(cfg.experts)]
    return tuple(np.stack([p[i] for p in parts]) for i in range(4))


def lazy_expert_weights(cfg):
    return functools.lru_cache(maxsize=None)(lambda e: quantize_expert(cfg, e))


def _quantize_expert_job(args):
    cfg, e = args
    return quantize_expert(cfg, e)


@functools.lru_cache(maxsize=1)
def all_experts_parallel(cfg, workers=8):
    """Every expert's oracle-quantized weights for cfg's weight set, computed
    once per process by a pool of fresh interpreters (spawned, so they never
    inherit the test process's device state); a getter e -> weights."""
    import concurrent.futures
    import multiprocessing
    ctx = multiprocessing.get_context("spawn")
    with concurrent.futures.ProcessPoolExecutor(max_workers=workers, mp_context=ctx) as ex:
        parts = list(ex.map(_quantize_expert_job, [(cfg, e) for e in range(cfg.experts)], chunksize=4))
    return lambda e: parts[e]


def quantize_expert_nv(cfg, e, scales=None):
    """Expert e's NVFP4 weights, each matrix with the tensor scale of its own
    absolute maximum, or with scales = (g_w1, g_w2) when given:
    ((w1c, w1s, w2c, w2s), g_w1, g_w2)."""
    w1, w2 = synth.expert_weights_f32(cfg, e)
    if scales is None:
        g1, g2 = nvfp4.tensor_scale(np.abs(w1).max()), nvfp4.tensor_scale(np.abs(w2).max())
    else:
        g1, g2 = np.float32(scales[0]), np.float32(scales[1])
    w1c, w1s = nvfp4.quantize_packed(w1, g1)
    w2c, w2s = nvfp4.quantize_packed(w2, g2)
    return (w1c, w1s, w2c, w2s), g1, g2


def all_expert_weights_nv(cfg):
    """(stacked (w1c, w1s, w2c, w2s), g_w1 fp32 [E], g_w2 fp32 [E])."""
    parts = [quantize_expert_nv(cfg, e) for e in range(cfg.experts)]
    W = tuple(np.stack([p[0][i] for p in parts]) for i in range(4))
    return W, np.array([p[1] for p in parts], np.float32), np.array([p[2] for p in parts], np.float32)


def lazy_expert_weights_nv(cfg, scales):
    """e -> expert e's NVFP4 weights (w1c, w1s, w2c, w2s) under the fixed tensor
    scales (g_w1, g_w2), quantized on first use."""
    return functools.lru_cache(maxsize=None)(lambda e: quantize_expert_nv(cfg, e, scales)[0])


# Calibration bound of |h| per layer shape (hidden size): above the largest
# |silu(gate) * up| of the synthetic layers, so no block of h saturates.
H_AMAX = {256: 2.0, 512: 4.0, 768: 6.0, 1024: 8.0, 4096: 64.0}

# Tensor scales of the DSV4-shaped synthetic weights (N(0, 0.02^2): every
# |w| is far below 6 * 448 * g), the same constants for every expert.
NV_WEIGHT_SCALES = (np.float32(6.1e-5), np.float32(5.3e-5))


def nv_act_scales(cfg, x_bits):
    """(g_x, g_h): x's tensor scale from its absolute maximum, h's from the
    shape's calibration bound."""
    return (nvfp4.tensor_scale(np.abs(synth.bf16_bits_to_f32(x_bits)).max()),
            nvfp4.tensor_scale(H_AMAX[cfg.hidden]))

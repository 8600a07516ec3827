"""Test-side assembly of oracle inputs: synthetic fp32 weights quantized by the
oracle's own MXFP4 quantizer (never by the device path)."""
import functools

import numpy as np

import synth
from oracle import mxfp4


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

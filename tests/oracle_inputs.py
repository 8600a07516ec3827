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

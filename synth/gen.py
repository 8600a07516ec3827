"""Seeded generators for the five layer configurations.

Shapes follow the DeepSeek-V4-Flash routed-expert layer that the pages measure:
hidden=4096, inter=2048, 256 experts, top-6 (sglang PR "[deepseek-v4] Bump
sgl-deep-gemm for packed FP4xFP4 mega-MoE (W4A4)", Appendix: measured data).
The token counts are the decode size 64, the pages' single-rank operating point
ntok=512 (same page, section B "NCU Speed-of-Light"), a 4x1024-token prefill and
a 16384-token prefill with Zipf(1.1) expert popularity.

Streams: every draw uses numpy PCG64 seeded with SeedSequence((1000*idx + stream,
*sub)); stream 0 = tokens, 1 = routing (idx = the config index), 2 = weights
(idx = the config's weight set, sub = expert index, so any single expert can be
regenerated on its own).  The four DeepSeek-V4-Flash-shaped configs are one
layer at four token counts and share weight set 1; the tiny layer has set 0.

Value distributions:
  x        fp32 ~ N(0, 1), rounded to bfloat16 (round to nearest, ties to even)
  weights  fp32 ~ N(0, 0.02^2) for W1 [2I, H] (gate rows first, then up rows)
           and W2 [H, I] of every expert
  routing  'logits':  router logits ~ N(0,1) [T, E]; top-k by value (ties go to
                      the lower expert index); weights = softmax of the k chosen
                      logits (fp64, stored fp32)
           'uniform': k distinct experts per token, uniform without replacement;
                      weights = softmax of k fresh N(0,1) logits
           'zipf':    expert popularity p(rank) ~ rank^-s over a seeded random
                      permutation of experts; k distinct experts per token by
                      Gumbel-top-k on log p; weights as for 'uniform'
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    index: int
    name: str
    tokens: int
    hidden: int
    inter: int
    experts: int
    topk: int
    routing: str           # 'logits' | 'uniform' | 'zipf'
    weight_set: int = 0
    zipf_s: float = 1.1

    @property
    def routed_rows(self) -> int:
        return self.tokens * self.topk


CONFIGS = (
    LayerConfig(0, "tiny_t16_h256_i128_e8_k2", 16, 256, 128, 8, 2, "logits"),
    LayerConfig(1, "dsv4flash_t64_decode", 64, 4096, 2048, 256, 6, "uniform", 1),
    LayerConfig(2, "dsv4flash_t512", 512, 4096, 2048, 256, 6, "uniform", 1),
    LayerConfig(3, "dsv4flash_t4096_prefill", 4096, 4096, 2048, 256, 6, "uniform", 1),
    LayerConfig(4, "dsv4flash_t16384_zipf1.1", 16384, 4096, 2048, 256, 6, "zipf", 1),
)


def _rng(cfg_index: int, stream: int, *sub: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence((1000 * cfg_index + stream, *sub))))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns, round to nearest, ties to even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_tokens(cfg: LayerConfig, tokens: int | None = None) -> np.ndarray:
    """x as bf16 bit patterns, uint16 [T, H]."""
    T = cfg.tokens if tokens is None else tokens
    x = _rng(cfg.index, 0).standard_normal((T, cfg.hidden), dtype=np.float32)
    return f32_to_bf16_bits(x)


def _softmax_rows(logits: np.ndarray) -> np.ndarray:
    z = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(z)
    return p / p.sum(axis=1, keepdims=True)


def make_routing(cfg: LayerConfig, tokens: int | None = None):
    """(topk_ids int32 [T, k], topk_weights fp32 [T, k])."""
    T = cfg.tokens if tokens is None else tokens
    E, k = cfg.experts, cfg.topk
    rng = _rng(cfg.index, 1)
    if cfg.routing == "logits":
        logits = rng.standard_normal((T, E))
        ids = np.argsort(-logits, axis=1, kind="stable")[:, :k]
        chosen = np.take_along_axis(logits, ids, axis=1)
    elif cfg.routing == "uniform":
        ids = np.argsort(rng.random((T, E)), axis=1, kind="stable")[:, :k]
        chosen = rng.standard_normal((T, k))
    elif cfg.routing == "zipf":
        perm = rng.permutation(E)
        logp = np.empty(E)
        logp[perm] = -cfg.zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))
        gumbel = -np.log(-np.log(rng.random((T, E))))
        ids = np.argsort(-(logp[None, :] + gumbel), axis=1, kind="stable")[:, :k]
        chosen = rng.standard_normal((T, k))
    else:
        raise ValueError(cfg.routing)
    w = _softmax_rows(chosen).astype(np.float32)
    return ids.astype(np.int32), w


def expert_weights_f32(cfg: LayerConfig, e: int):
    """(W1 fp32 [2I, H], W2 fp32 [H, I]) for expert e; rows [0, I) of W1 are gate, [I, 2I) are up."""
    rng = _rng(cfg.weight_set, 2, e)
    std = np.float32(0.02)
    w1 = rng.standard_normal((2 * cfg.inter, cfg.hidden), dtype=np.float32)
    w1 *= std
    w2 = rng.standard_normal((cfg.hidden, cfg.inter), dtype=np.float32)
    w2 *= std
    return w1, w2

"""Device-side fixtures for the GPU tier: synthetic inputs copied to the GPU,
weights quantized there by the library (moe_w4a4_quantize) and re-laid by
moe_w4a4_prepare_weights.  The oracle side never sees a device result as an
input: it regenerates the same synthetic values and quantizes them itself."""
import functools
import sys

import numpy as np
import torch

import synth


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dev(a, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def layer_for(H, I, E, k, max_tokens, mma_type=0):
    from block_scaled_fp4_pre_amd.layer import MoeW4A4Layer
    return MoeW4A4Layer(H, I, E, k, max_tokens, mma_type=mma_type)


@functools.lru_cache(maxsize=2)
def synth_layer(weight_set_cfg_index: int, max_tokens: int):
    """A layer holding the synthetic weights of the config's weight set."""
    cfg = synth.CONFIGS[weight_set_cfg_index]
    log(f"[gpu_support] building layer weight_set={cfg.weight_set} H={cfg.hidden} I={cfg.inter} "
        f"E={cfg.experts} k={cfg.topk} max_tokens={max_tokens}")
    layer = layer_for(cfg.hidden, cfg.inter, cfg.experts, cfg.topk, max_tokens)
    layer.load_fp32(lambda e: synth.expert_weights_f32(cfg, e))
    torch.cuda.synchronize()
    log("[gpu_support] layer ready")
    return layer


@functools.lru_cache(maxsize=1)
def synth_layer_fp8(weight_set_cfg_index: int, max_tokens: int):
    """The same layer with the fp8xfp4 MMA type.  The prepared weights (MXFP4
    for both MMA types) are shared with synth_layer's."""
    from block_scaled_fp4_pre_amd.layer import MoeW4A4Layer
    base = synth_layer(weight_set_cfg_index, max_tokens)
    layer = MoeW4A4Layer(base.H, base.I, base.E, base.k, max_tokens, mma_type=1)
    layer.prepared = base.prepared
    return layer


def run_config(layer, cfg, tokens=None):
    """Forward of config cfg on `layer`; returns host copies of every intermediate."""
    x = synth.make_tokens(cfg, tokens)
    ids, w = synth.make_routing(cfg, tokens)
    T = x.shape[0]
    out = layer.forward(dev_bf16(x), dev(ids), dev(w))
    torch.cuda.synchronize()
    return dict(x=x, ids=ids, w=w, out=host_bits(out), **workspace_host(layer, T))


def rows_from_planes(planes, nrows):
    """[K steps, rows, bytes] K-step planes (the workspace layout of the
    sorted-row activations) -> [nrows, K steps * bytes] row-major on the host."""
    a = planes[:, :nrows].cpu().numpy()
    return np.ascontiguousarray(a.transpose(1, 0, 2)).reshape(nrows, -1)


def planes_from_rows(rows, nplanes):
    """Inverse of rows_from_planes for an injected [nrows, nplanes * b] array."""
    n = rows.shape[0]
    return np.ascontiguousarray(rows.reshape(n, nplanes, -1).transpose(1, 0, 2))


def workspace_host(layer, T):
    H, I, E, k = layer.H, layer.I, layer.E, layer.k
    R = T * k
    ws = layer.ws
    f8 = layer.mma_type == 1             # E4M3 activations: one byte per element
    counts = ws("counts", (E,), torch.int32).cpu().numpy()
    nv = int(counts.sum())
    return dict(
        xq=ws("xq", (layer.max_tokens, H if f8 else H // 2), torch.uint8)[:T].cpu().numpy(),
        xsf=ws("xsf", (layer.max_tokens, H // 32), torch.uint8)[:T].cpu().numpy(),
        counts=counts,
        offsets=ws("offsets", (E + 1,), torch.int32).cpu().numpy(),
        sorted_rows=ws("sorted_rows", (layer.max_tokens * k,), torch.int32)[:nv].cpu().numpy(),
        pos=ws("pos", (layer.max_tokens * k,), torch.int32)[:R].cpu().numpy(),
        hq=rows_from_planes(ws("hq", (I // 128, layer.max_tokens * k, 128 if f8 else 64), torch.uint8), nv),
        hsf=rows_from_planes(ws("hsf", (I // 128, layer.max_tokens * k, 4), torch.uint8), nv),
        xsf_planes=rows_from_planes(ws("xsf_planes", (H // 128, layer.max_tokens * k, 4), torch.uint8), nv),
        y=ws("y", (layer.max_tokens * k, H), torch.bfloat16)[:nv].float().cpu().numpy().astype(np.float64),
    )

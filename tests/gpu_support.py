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
def _weights_layer(weight_set_cfg_index: int):
    """A layer holding the synthetic weights of the config's weight set (and
    a workspace for one token); the layers of synth_layer share its weights."""
    cfg = synth.CONFIGS[weight_set_cfg_index]
    log(f"[gpu_support] loading weight_set={cfg.weight_set} H={cfg.hidden} I={cfg.inter} E={cfg.experts} "
        f"k={cfg.topk}")
    layer = layer_for(cfg.hidden, cfg.inter, cfg.experts, cfg.topk, 1)
    layer.load_fp32(lambda e: synth.expert_weights_f32(cfg, e))
    torch.cuda.synchronize()
    log("[gpu_support] weights ready")
    return layer


@functools.lru_cache(maxsize=8)
def synth_layer(weight_set_cfg_index: int, max_tokens: int, mma_type: int = 0):
    """A layer over the synthetic weights of the config's weight set with a
    workspace for max_tokens tokens; both MMA types use the same MXFP4
    weights, so every such layer shares one prepared buffer."""
    return _weights_layer(weight_set_cfg_index).with_capacity(max_tokens, mma_type=mma_type)


def run_inputs(layer, x, ids, w, acc=False, acc_rows=None, mega=False):
    """Forward of host inputs on `layer`; returns host copies of every
    intermediate.  acc: run the same launches through moe_w4a4_run_stages
    with GEMM1's raw accumulators captured as "acc" (sorted-row order; only
    the rows acc_rows, default all, are copied back).  mega: through the
    single-launch forward (moe_w4a4_forward_mega) instead."""
    from block_scaled_fp4_pre_amd import _lib
    T = x.shape[0]
    xd, idd, wd = dev_bf16(x), dev(ids), dev(w)
    res = {}
    if acc:
        out = torch.empty((T, layer.H), dtype=torch.bfloat16, device="cuda")
        buf = torch.full((T * layer.k, 2 * layer.I), float("nan"), device="cuda")
        layer.run_stages(_lib.MOE_STAGE_ALL, T, x=xd, topk_ids=idd, topk_weights=wd, out=out, gemm1_acc=buf)
        torch.cuda.synchronize()
        rows = slice(None) if acc_rows is None else torch.from_numpy(np.asarray(acc_rows, np.int64)).cuda()
        a = buf[rows].cpu().numpy()
        if acc_rows is not None:
            full = np.full((T * layer.k, 2 * layer.I), np.nan, np.float32)
            full[np.asarray(acc_rows)] = a
            a = full
        res["acc"] = a
        del buf
    else:
        out = layer.forward_mega(xd, idd, wd) if mega else layer.forward(xd, idd, wd)
    torch.cuda.synchronize()
    return dict(x=x, ids=ids, w=w, out=host_bits(out), **res, **workspace_host(layer, T))


def run_config(layer, cfg, tokens=None, acc=False, acc_rows=None, mega=False):
    """Forward of config cfg on `layer`; returns host copies of every intermediate."""
    x = synth.make_tokens(cfg, tokens)
    ids, w = synth.make_routing(cfg, tokens)
    return run_inputs(layer, x, ids, w, acc=acc, acc_rows=acc_rows, mega=mega)


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

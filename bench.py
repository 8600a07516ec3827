"""Benchmark of the W4A4 MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--mma-type {mxf4xmxf4,fp8xfp4,nvf4xnvf4}]
                    [--no-cpu-baseline] [--no-ceiling] [--no-prefill] [--no-decode]

A step is one whole forward of the layer (pre-dispatch quantization, routing,
GEMM1 + SwiGLU + requant, GEMM2, combine) on one batch of synthetic tokens whose
inputs are already resident in HBM.  The default workload is the pages'
single-rank operating point: DeepSeek-V4-Flash shape (hidden 4096, inter 2048,
256 experts, top-6), ntok = 512, uniform routing, all 256 experts' MXFP4
weights resident.

Prints ONE JSON line.  `value` is the time of one layer forward in us (lower is
better): K calls of moe_w4a4_forward, bracketed by synchronizations and HIP
events on the stream the kernels run on.  Throughput in TFLOP/s and
algorithmic HBM GB/s ride along.  "roofline" is GEMM1's, the dominant kernel
(gemm1_swiglu_kernel up to 16 routed rows per expert, gemm_lds_kernel above;
gemm1_nv_kernel and gemm_lds_nv_kernel for the NVFP4 type), and
"roofline_gemm2" GEMM2's, each
against the HBM or the MFMA peak of the MMA type (MXFP4, FP8 for the fp8xfp4
type, fp16 for NVFP4, whose products run on the dense fp16 MFMA), whichever
bounds its algorithmic bytes and flops.  Their durations come from K further steps of the same
launches in which events on the same stream bracket each GEMM launch
("split_step_us" is the step time of that loop).  "forward_us" gives the
median, minimum and maximum of K more forwards, each bracketed by its own
events.  With the default workload the metric's second operating point,
ntok = 4096, rides along as the object "dsv4flash_t4096_prefill" (same
weights, same measurements), and (MX types) a decode batch of 8 tokens run
as one kernel launch (moe_w4a4_forward_mega, mega_moe_kernel), as
"dsv4flash_t8_decode_single_launch", with the same forward's time as four
launches beside it and whether moe_w4a4_forward takes the single launch at
that size.  "context" holds the pages' own figure for
ntok = 512 (another machine: not a baseline, so "vs_baseline" is null).
"ceiling" holds this GPU's measured ceilings (libmoe_ceiling.so): the
streaming-read rate of a 2 GiB buffer with non-temporal and with default loads
(best over 2 to 16 workgroups per CU), the rate of back-to-back MFMAs of each
MMA type and of dense bf16.  Each roofline object then carries
"ceiling_frac", its achieved rate over the measured ceiling of its bound (the
read, or the MFMA rate of its MMA type), and "gemm1_frac" repeats the
headline GEMM1's.  "cpu_baseline" times the fp64 CPU oracle over one whole
forward of the same workload, with the BLAS it runs on.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "mega-MoE layer µs + TFLOPS + HBM GB/s at ntok=512/4096, DSV4-Flash shape"
HBM_PEAK_GBPS = 8000.0            # MI355X HBM3E
FP4_PEAK_TFLOPS = 10100.0         # MI355X dense MXFP4 MFMA
FP8_PEAK_TFLOPS = 5000.0          # MI355X dense FP8 MFMA: the rate of the FP8 x FP4 mixed form
F16_PEAK_TFLOPS = 2500.0          # MI355X dense fp16 / bf16 MFMA: the NVFP4 type's products
# Tensor scales of the NVFP4 workload (calibration constants, like weights):
# x ~ N(0, 1) stays below 6 * 448 * 2^-8 = 10.5, |h| below 64 (6 * 448 * g_h),
# and the N(0, 0.02^2) weights below 0.164 (W1) and 0.142 (W2).
NV_X_SCALE = 2.0 ** -8
NV_H_SCALE = 64.0 / 2688.0
NV_W_SCALES = (6.1e-5, 5.3e-5)
COPY_BYTES = 256 << 20           # calibration copy size
PAGES_US_NTOK512 = 537.6          # W4A4 mega-MoE kernel, 1 B200, 1-rank isolation, ntok=512 (context)
PAGES_US_NTOK512_W4A8 = 753.2     # the same measurement of the W4A8 (FP8 activations) kernel


def expert_bytes(H, I, group=32):
    """Bytes of one expert: W1 (2I x H) and W2 (H x I) E2M1 codes + one scale
    byte per `group` elements (32 for MXFP4, 16 for NVFP4)."""
    return 2 * I * H // 2 + 2 * I * H // group + H * I // 2 + H * I // group


def algorithmic(cfg, counts, fp8=False, nv=False):
    """fp8: the fp8xfp4 MMA type, whose x-hat and h-hat take one byte per
    element; nv: NVFP4, one scale byte per 16 elements everywhere (the tensor
    scales are a few bytes)."""
    H, I, k, T = cfg.hidden, cfg.inter, cfg.topk, cfg.tokens
    cb = 1 if fp8 else 2          # elements per activation code byte
    G = 16 if nv else 32          # elements per scale byte
    active = int((counts > 0).sum())
    R = int(counts.sum())
    layer_bytes = active * expert_bytes(H, I, G) + T * (2 * H + 8 * k + 2 * H)
    flops = R * (2 * H * 2 * I + 2 * I * H)
    w1 = 2 * I * H // 2 + 2 * I * H // G
    gemm1_bytes = active * w1 + T * (H // cb + H // G) + R * (I // cb + I // G)
    w2 = H * I // 2 + H * I // G
    gemm2_bytes = active * w2 + R * (I // cb + I // G) + R * 2 * H      # W2, h-hat in, y out (bf16)
    return dict(active=active, R=R, layer_bytes=layer_bytes, flops=flops, gemm1_bytes=gemm1_bytes,
                gemm1_flops=R * 2 * H * 2 * I, gemm2_bytes=gemm2_bytes, gemm2_flops=R * 2 * I * H)


PREFILL = "dsv4flash_t4096_prefill"   # the metric's second operating point
DECODE_TOKENS = 8                 # decode batch of the single-launch record (48 routed rows)
STREAM_MAX_ROWS = 16              # mean routed rows per expert up to which the GEMMs are the streaming kernels
# Each GEMM's kernel on each path, with the sources its code comes from.  The
# label names the committed HBM-counter file of that kernel
# (profiles/<label>_<workload>[_fp8xfp4]_hbm_counters.txt).
KERNELS = {
    ("gemm1", "stream"): ("gemm1_swiglu_kernel", "gemm1_swiglu_kernel",
                          ("gemm1.hip", "stream_ring.h", "gemm_common.h", "epilogue.h", "device_common.h", "tiles.h")),
    ("gemm2", "stream"): ("gemm2_kernel", "gemm2_kernel",
                          ("gemm2.hip", "stream_ring.h", "gemm_common.h", "epilogue.h", "device_common.h", "tiles.h")),
    ("gemm1", "prefill"): ("gemm_lds_kernel", "gemm_lds_kernel",
                           ("gemm_lds.hip", "gemm_common.h", "epilogue.h", "device_common.h", "tiles.h")),
    ("gemm2", "prefill"): ("gemm_lds_kernel", "gemm_lds_kernel_gemm2",
                           ("gemm_lds.hip", "gemm_common.h", "epilogue.h", "device_common.h", "tiles.h")),
    ("gemm1", "nv"): ("gemm1_nv_kernel", "gemm1_nv_kernel",
                      ("gemm_nv.hip", "nvfp4.h", "gemm_common.h", "epilogue.h", "device_common.h", "tiles.h",
                       "e4m3.h", "epilogue_nv.h")),
    ("gemm2", "nv"): ("gemm2_nv_kernel", "gemm2_nv_kernel",
                      ("gemm_nv.hip", "nvfp4.h", "gemm_common.h", "epilogue.h", "device_common.h", "tiles.h",
                       "e4m3.h", "epilogue_nv.h")),
    ("gemm1", "nv_prefill"): ("gemm_lds_nv_kernel", "gemm_lds_nv_kernel",
                              ("gemm_lds_nv.hip", "nvfp4.h", "gemm_common.h", "epilogue.h", "device_common.h",
                               "tiles.h", "e4m3.h", "epilogue_nv.h")),
    ("gemm2", "nv_prefill"): ("gemm_lds_nv_kernel", "gemm_lds_nv_kernel_gemm2",
                              ("gemm_lds_nv.hip", "nvfp4.h", "gemm_common.h", "epilogue.h", "device_common.h",
                               "tiles.h", "e4m3.h", "epilogue_nv.h")),
    # the single-launch forward: the whole layer in one kernel
    ("layer", "single"): ("mega_moe_kernel", "mega_moe_kernel",
                          ("mega.hip", "epilogue.h", "gemm_common.h", "quant_group.h", "nvfp4.h", "tiles.h",
                           "device_common.h", "e4m3.h")),
}
COUNTERS_FILE = os.path.join(ROOT, "profiles", "{}_{}_hbm_counters.txt")


def gemm_path(cfg, nv=False):
    """The GEMM kernels a workload runs on: streaming or LDS-staged, each with
    its own kernels for the NVFP4 type (whose LDS-staged form needs an even
    number of weight blocks: hidden % 512 and inter % 256)."""
    rows_hint = -(-cfg.tokens * cfg.topk // cfg.experts)
    if nv:
        tiled = rows_hint > STREAM_MAX_ROWS and cfg.hidden % 512 == 0 and cfg.inter % 256 == 0
        return "nv_prefill" if tiled else "nv"
    return "stream" if rows_hint <= STREAM_MAX_ROWS else "prefill"


def measured_traffic(workload, gemm, path, fp8=False):
    """HBM bytes per launch of one GEMM kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE runs, each scaled by the same counter on a copy of
    known size; None if there are none for this workload and MMA type or the
    kernel's sources changed since."""
    import hashlib
    _, label, sources = KERNELS[(gemm, path)]
    path = COUNTERS_FILE.format(label, workload + ("_fp8xfp4" if fp8 else ""))
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    h = hashlib.sha256()
    for name in sources:
        with open(os.path.join(ROOT, "block_scaled_fp4_pre_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    if kv.get("kernel_sources_sha256") != h.hexdigest():
        return None
    cb = float(kv["copy_bytes"])
    fetch = float(kv["fetch_kib"]) * cb / float(kv["copy_fetch_kib"])
    write = float(kv["write_kib"]) * cb / float(kv["copy_write_kib"])
    return int(round(fetch + write))


def blas_info():
    """(threads, vendor string) of the BLAS that numpy uses for the oracle's products."""
    try:
        import threadpoolctl
        blas = [b for b in threadpoolctl.threadpool_info() if b.get("user_api") == "blas"]
    except Exception:  # pragma: no cover
        blas = []
    if not blas:
        return os.cpu_count() or 1, "unknown"
    b = blas[0]
    return int(b.get("num_threads", 1)), f"{b.get('internal_api', '?')} {b.get('version', '?')} " \
                                         f"({b.get('architecture', '?')} kernels, {b.get('threading_layer', '?')})"


def cpu_baseline(cfg, x, ids, w, mma_type="mxf4xmxf4", weight_pool=2):
    """The oracle as it stands, timed over one whole forward of the workload:
    quantization of all tokens, the route, GEMM1/SwiGLU/requant/GEMM2 of
    every routed row of every active expert, and the combine.  Expert weights
    are load-time work and are not timed; the oracle quantizes weight_pool
    experts' weights and every expert uses one of them in turn (its arithmetic
    and cost do not depend on the weight values, and quantizing all 256
    experts' 3.4 GB with the oracle's brute-force quantizer would take tens of
    CPU-minutes)."""
    import synth
    from oracle import mxfp4, nvfp4
    from oracle.forward import forward
    from oracle.route import route

    threads, vendor = blas_info()
    counts = route(ids, cfg.experts)[0]
    active = int((counts > 0).sum())
    nv = mma_type == "nvf4xnvf4"
    pool = []
    for e in range(weight_pool):
        w1, w2 = synth.expert_weights_f32(cfg, e)
        if nv:
            pool.append(nvfp4.quantize_packed(w1, NV_W_SCALES[0]) + nvfp4.quantize_packed(w2, NV_W_SCALES[1]))
        else:
            pool.append(mxfp4.quantize_packed(w1) + mxfp4.quantize_packed(w2))
    E = cfg.experts
    ts = (NV_X_SCALE, NV_H_SCALE, np.full(E, NV_W_SCALES[0], np.float32),
          np.full(E, NV_W_SCALES[1], np.float32)) if nv else None
    t0 = time.perf_counter()
    forward(x, ids, w, lambda e: pool[e % weight_pool], cfg.experts, cfg.inter, mma_type=mma_type, tensor_scales=ts)
    secs = time.perf_counter() - t0
    return {"value": round(secs * 1e6, 1), "unit": "us", "cores": threads, "kind": "oracle", "blas": vendor,
            "sample": f"one whole forward of the {cfg.name} workload ({cfg.tokens} tokens, {int(counts.sum())} "
                      f"routed rows over {active} active experts, combine included), measured, not scaled; the "
                      f"experts use {weight_pool} experts' oracle-quantized weights in turn",
            "measured_s": round(secs, 2)}


def mfma_peak_of(mma_type):
    """Published dense MFMA peak (TFLOP/s) of the instruction an MMA type's GEMMs run on."""
    return {"fp8xfp4": FP8_PEAK_TFLOPS, "nvf4xnvf4": F16_PEAK_TFLOPS}.get(mma_type, FP4_PEAK_TFLOPS)


def roofline(kernel, nbytes, flops, us, mma_type, traffic):
    """Roofline object of one kernel: HBM-bound unless its flops take longer
    at the MFMA peak of the MMA type than its algorithmic bytes at the HBM peak."""
    mfma_peak = mfma_peak_of(mma_type)
    mfma_bound = flops / (mfma_peak * 1e12) > nbytes / (HBM_PEAK_GBPS * 1e9)
    if mfma_bound:
        ach, peak, unit = flops / (us * 1e-6) / 1e12, mfma_peak, "TFLOP/s"
    else:
        ach, peak, unit = nbytes / (us * 1e-6) / 1e9, HBM_PEAK_GBPS, "GB/s"
    return {"kernel": kernel, "bound": "mfma" if mfma_bound else "hbm", "achieved": round(ach, 1), "peak": peak,
            "unit": unit, "frac": round(ach / peak, 4), "traffic": traffic, "avg_us": round(us, 2),
            "bytes_per_launch": int(nbytes), "flops_per_launch": int(flops)}


def measure(layer, cfg, x, ids, w, out, steps, warmup):
    """Times the forward: K forwards through the single entry point (the
    timed region), K more split into the stage groups so that events on the
    kernels' stream bracket GEMM1 and GEMM2, and K more each bracketed by its
    own events."""
    import torch

    from block_scaled_fp4_pre_amd import _lib
    T = cfg.tokens
    S_A = _lib.MOE_STAGE_QUANT | _lib.MOE_STAGE_ROUTE

    def split_step(ev=None):
        # The launches of moe_w4a4_forward, in four calls, with events
        # between them on the same stream.
        layer.run_stages(S_A, T, x=x, topk_ids=ids)
        if ev is not None:
            ev[0].record()
        layer.run_stages(_lib.MOE_STAGE_GEMM1, T)
        if ev is not None:
            ev[1].record()
        layer.run_stages(_lib.MOE_STAGE_GEMM2, T)
        if ev is not None:
            ev[2].record()
        layer.run_stages(_lib.MOE_STAGE_COMBINE, T, topk_weights=w, out=out)

    ev_t = lambda: torch.cuda.Event(enable_timing=True)
    for _ in range(warmup):
        layer.forward(x, ids, w, out)
    torch.cuda.synchronize()
    start, end = ev_t(), ev_t()
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        layer.forward(x, ids, w, out)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    us = start.elapsed_time(end) / steps * 1e3

    # Kernel attribution.  The event packets add a few us of idle time around
    # each bracketed launch, so these averages are upper bounds on the
    # kernels' durations (the kernel traces in profiles/ agree).
    for _ in range(2):
        split_step()
    evs = [(ev_t(), ev_t(), ev_t()) for _ in range(steps)]
    split_s, split_e = ev_t(), ev_t()
    torch.cuda.synchronize()
    split_s.record()
    for i in range(steps):
        split_step(evs[i])
    split_e.record()
    torch.cuda.synchronize()
    gemm1_us = float(np.mean([a.elapsed_time(b) for a, b, _ in evs])) * 1e3
    gemm2_us = float(np.mean([b.elapsed_time(c) for _, b, c in evs])) * 1e3
    split_us = split_s.elapsed_time(split_e) / steps * 1e3

    fwd = [(ev_t(), ev_t()) for _ in range(steps)]
    for a, b in fwd:
        a.record()
        layer.forward(x, ids, w, out)
        b.record()
    torch.cuda.synchronize()
    fwd_us = np.array([a.elapsed_time(b) for a, b in fwd]) * 1e3
    return dict(us=us, wall=wall, gemm1_us=gemm1_us, gemm2_us=gemm2_us, split_us=split_us, fwd_us=fwd_us)


def workload_record(layer, cfg, steps, warmup, mma_type):
    """Times one workload on `layer` and returns (its record, its inputs)."""
    import torch

    import synth
    x_h = synth.make_tokens(cfg)
    ids_h, w_h = synth.make_routing(cfg)
    x = torch.from_numpy(x_h.view(np.int16)).cuda().view(torch.bfloat16)
    ids = torch.from_numpy(ids_h).cuda()
    w = torch.from_numpy(w_h).cuda()
    out = torch.empty((cfg.tokens, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    m = measure(layer, cfg, x, ids, w, out, steps, warmup)
    counts = layer.ws("counts", (cfg.experts,), torch.int32).cpu().numpy()
    fp8, nv = mma_type == "fp8xfp4", mma_type == "nvf4xnvf4"
    alg = algorithmic(cfg, counts, fp8, nv)
    us = m["us"]
    mfma_peak = mfma_peak_of(mma_type)
    tflops = alg["flops"] / (us * 1e-6) / 1e12
    gbps = alg["layer_bytes"] / (us * 1e-6) / 1e9
    path = gemm_path(cfg, nv)
    rec = {
        "value": round(us, 2),
        "tflops": round(tflops, 2),
        "tflops_frac": round(tflops / mfma_peak, 4),
        "hbm_gbps": round(gbps, 1),
        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "split_step_us": round(m["split_us"], 2),
        "forward_us": {"median": round(float(np.median(m["fwd_us"])), 2), "min": round(float(m["fwd_us"].min()), 2),
                       "max": round(float(m["fwd_us"].max()), 2)},
        "roofline": roofline(KERNELS[("gemm1", path)][0], alg["gemm1_bytes"], alg["gemm1_flops"], m["gemm1_us"],
                             mma_type, measured_traffic(cfg.name, "gemm1", path, fp8)),
        "roofline_gemm2": roofline(KERNELS[("gemm2", path)][0], alg["gemm2_bytes"], alg["gemm2_flops"],
                                   m["gemm2_us"], mma_type, measured_traffic(cfg.name, "gemm2", path, fp8)),
        "wall_s": round(m["wall"], 3),
    }
    return rec, alg, (x_h, ids_h, w_h)


def decode_record(layer, cfg, steps, warmup):
    """The DeepSeek-V4-Flash layer at a decode batch (cfg: its shape and
    routing recipe, cfg.tokens tokens) as the single-launch kernel
    (moe_w4a4_forward_mega, mega_moe_kernel), beside the same forward as the
    four launches of the stage sequence (moe_w4a4_run_stages).
    "forward_takes_single_launch": whether moe_w4a4_forward runs the single
    launch at this size."""
    import torch

    import synth
    from block_scaled_fp4_pre_amd import _lib
    T = cfg.tokens
    x_h = synth.make_tokens(cfg)
    ids_h, w_h = synth.make_routing(cfg)
    x = torch.from_numpy(x_h.view(np.int16)).cuda().view(torch.bfloat16)
    ids = torch.from_numpy(ids_h).cuda()
    w = torch.from_numpy(w_h).cuda()
    out = torch.empty((T, cfg.hidden), dtype=torch.bfloat16, device="cuda")

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps * 1e3

    us = timed(lambda: layer.forward_mega(x, ids, w, out))
    multi = timed(lambda: layer.run_stages(_lib.MOE_STAGE_ALL, T, x=x, topk_ids=ids, topk_weights=w, out=out))
    counts = layer.ws("counts", (cfg.experts,), torch.int32).cpu().numpy()
    alg = algorithmic(cfg, counts)
    gbps = alg["layer_bytes"] / (us * 1e-6) / 1e9
    traffic = measured_traffic(cfg.name, "layer", "single", layer.mma_type == _lib.MOE_MMA_FP8_X_MXF4)
    return {
        "value_us": round(us, 2),
        "multi_launch_us": round(multi, 2),
        "speedup_over_multi_launch": round(multi / us, 3),
        "forward_takes_single_launch": T * cfg.topk <= (_lib.MOE_MEGA_AUTO_ROWS_FP8 if layer.mma_type == 1
                                                        else _lib.MOE_MEGA_AUTO_ROWS),
        "hbm_gbps": round(gbps, 1),
        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "roofline": {"kernel": "mega_moe_kernel", "bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": traffic, "avg_us": round(us, 2),
                     "bytes_per_launch": int(alg["layer_bytes"])},
        "config": {"tokens": T, "routing": cfg.routing, "active_experts": alg["active"], "routed_rows": alg["R"]},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="dsv4flash_t512")
    ap.add_argument("--mma-type", default="mxf4xmxf4", choices=("mxf4xmxf4", "fp8xfp4", "nvf4xnvf4"),
                    help="MXFP4 activations and weights (the default, W4A4), MXFP8 E4M3 activations "
                         "(W4A8), or NVFP4 activations and weights")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the streaming-read and FP4 MFMA probes (libmoe_ceiling.so)")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode-batch record of the single-launch forward")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the ntok=4096 prefill record that rides along with the ntok=512 headline")
    ap.add_argument("--threads", type=int, default=16)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after timing, run a 256 MiB device-to-device copy (reference for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this layer runs on one GPU (all experts resident); --gpus {args.gpus} is not "
              f"supported.  Sharding is by expert and is described, not built.", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    from block_scaled_fp4_pre_amd import _lib
    from block_scaled_fp4_pre_amd.layer import MoeW4A4Layer

    configs = {c.name: c for c in synth.CONFIGS}
    cfg = configs[args.workload]
    torch.cuda.set_device(0)
    t_setup = time.perf_counter()
    fp8, nv = args.mma_type == "fp8xfp4", args.mma_type == "nvf4xnvf4"
    mma = {"mxf4xmxf4": _lib.MOE_MMA_MXF4_X_MXF4, "fp8xfp4": _lib.MOE_MMA_FP8_X_MXF4,
           "nvf4xnvf4": _lib.MOE_MMA_NVF4_X_NVF4}[args.mma_type]
    layer = MoeW4A4Layer(cfg.hidden, cfg.inter, cfg.experts, cfg.topk, cfg.tokens, mma_type=mma)
    E = cfg.experts
    ts = (NV_X_SCALE, NV_H_SCALE, np.full(E, NV_W_SCALES[0], np.float32),
          np.full(E, NV_W_SCALES[1], np.float32)) if nv else None
    layer.load_fp32(lambda e: synth.expert_weights_f32(cfg, e), threads=args.threads, tensor_scales=ts)
    torch.cuda.synchronize()
    print(f"[bench] setup {time.perf_counter() - t_setup:.1f}s workload={cfg.name}", file=sys.stderr, flush=True)

    rec, alg, (x_h, ids_h, w_h) = workload_record(layer, cfg, args.steps, args.warmup, args.mma_type)
    print(f"[bench] {cfg.name}: {rec['value']} us", file=sys.stderr, flush=True)
    us = rec["value"]
    pages_us = PAGES_US_NTOK512_W4A8 if fp8 else PAGES_US_NTOK512
    res = {
        "metric": METRIC,
        "value": us,
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 4),
        "higher_is_better": False,
        "scaling": "weak",
        # The pages' figure was measured on another machine (one B200): it is
        # context, not the baseline (see "context" and "cpu_baseline").
        "vs_baseline": None,
        "dtype": {"mxf4xmxf4": "mxfp4", "fp8xfp4": "mxfp8 x mxfp4", "nvf4xnvf4": "nvfp4"}[args.mma_type],
        "data": "synthetic",
        "config": {"workload": cfg.name, "mma_type": args.mma_type, "tokens": cfg.tokens, "hidden": cfg.hidden,
                   "inter": cfg.inter, "experts": cfg.experts, "topk": cfg.topk, "routing": cfg.routing,
                   "active_experts": alg["active"], "routed_rows": alg["R"]},
    }
    res.update({k: v for k, v in rec.items() if k != "value"})
    if cfg.name == "dsv4flash_t512" and not nv:      # the pages give no NVFP4 figure
        res["context"] = {"pages_us": pages_us, "pages_hardware": "1x B200, 1-rank isolation",
                          "value_over_pages": round(us / pages_us, 4)}
    if not args.no_prefill and cfg.name == "dsv4flash_t512":
        # The metric's second operating point, ntok=4096 (uniform routing, about
        # 96 rows per expert: the LDS-staged GEMMs), on the same prepared
        # weights with a workspace for 4096 tokens.
        pcfg = configs[PREFILL]
        player = layer.with_capacity(pcfg.tokens)
        prec, palg, _ = workload_record(player, pcfg, args.steps, args.warmup, args.mma_type)
        prec = {("value_us" if k == "value" else k): v for k, v in prec.items()}
        prec["config"] = {"tokens": pcfg.tokens, "routing": pcfg.routing, "active_experts": palg["active"],
                          "routed_rows": palg["R"]}
        res[pcfg.name] = prec
        print(f"[bench] {pcfg.name}: {prec['value_us']} us", file=sys.stderr, flush=True)
        del player
        torch.cuda.synchronize()
    if not args.no_decode and cfg.name == "dsv4flash_t512" and args.mma_type != "nvf4xnvf4":
        # A decode batch as one kernel launch (the single-launch forward) and
        # as the four launches, on the same prepared weights.
        import dataclasses
        dcfg = dataclasses.replace(configs["dsv4flash_t64_decode"], name=f"dsv4flash_t{DECODE_TOKENS}_decode",
                                   tokens=DECODE_TOKENS)
        dlayer = layer.with_capacity(DECODE_TOKENS)
        res[dcfg.name + "_single_launch"] = decode_record(dlayer, dcfg, args.steps, args.warmup)
        print(f"[bench] {dcfg.name}: {res[dcfg.name + '_single_launch']['value_us']} us", file=sys.stderr,
              flush=True)
        del dlayer
    if args.calibrate_copy:
        # A plain copy of known size: its FETCH_SIZE / WRITE_SIZE per dispatch
        # calibrate the counters read for the layer's kernels.
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_ceiling:
        # Measured ceilings of this GPU, beside the published peaks the
        # roofline fraction uses.
        from block_scaled_fp4_pre_amd import ceiling
        ceil = ceiling.measure()
        # the NVFP4 type's products run on the dense fp16 MFMA, whose rate is bf16's
        mfma_ref = ceil["mfma_fp8xfp4_TFLOPs" if fp8 else "mfma_bf16_TFLOPs" if nv else "mfma_fp4_TFLOPs"]
        for r in [res] + ([res[PREFILL]] if PREFILL in res else []):
            # both GEMMs against the read ceiling or the MFMA rate (GEMM2
            # also writes y, which the read ceiling does not include)
            for key in ("roofline", "roofline_gemm2"):
                roof = r[key]
                ref = mfma_ref if roof["bound"] == "mfma" else ceil["read_nt_GBps"]
                roof["ceiling_frac"] = round(roof["achieved"] / ref, 4)
        ceil["gemm1_frac"] = res["roofline"]["ceiling_frac"]
        res["ceiling"] = ceil
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (the oracle, one whole forward)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(cfg, x_h, ids_h, w_h, mma_type=args.mma_type)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

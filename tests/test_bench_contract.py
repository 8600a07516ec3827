"""bench.py's command-line contract: more than one GPU is refused with a
message (CPU tier), and one short run prints exactly one JSON line with the
fields and types the benchmark record needs, plus the per-forward spread,
both GEMMs' rooflines, the ntok=4096 record, the decode record of the
single-launch forward and the measured ceilings (GPU tier); the CPU baseline is the oracle over one whole forward (CPU tier, at the
tiny size)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.gpu
@pytest.mark.parametrize("mma", ["mxf4xmxf4", "fp8xfp4"])
def test_one_json_line_with_the_record_fields(mma):
    r = subprocess.run([sys.executable, BENCH, "--steps", "3", "--warmup", "1", "--no-cpu-baseline",
                        "--mma-type", mma], capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key, typ in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                     ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                     ("dtype", str), ("data", str), ("config", dict), ("roofline", dict)):
        assert isinstance(d[key], typ), key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1 and d["unit"] == "us"
    assert d["higher_is_better"] is False and d["data"] == "synthetic"
    assert d["config"]["workload"] == "dsv4flash_t512" and d["config"]["mma_type"] == mma
    assert abs(d["value"] - 1e3 * d["ms_per_step"]) <= 0.01 * d["value"]
    assert d["vs_baseline"] is None                 # the pages' figure is another machine's: context only
    assert d["context"]["pages_us"] in (537.6, 753.2)
    for roof in (d["roofline"], d["roofline_gemm2"]):
        assert roof["bound"] in ("hbm", "mfma") and roof["unit"] in ("GB/s", "TFLOP/s")
        assert 0 < roof["achieved"] and roof["peak"] > 0
        assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
        assert roof["traffic"] is None or roof["traffic"] > 0
    roof = d["roofline"]
    pre = d["dsv4flash_t4096_prefill"]                # the metric's second operating point
    assert pre["config"]["tokens"] == 4096 and pre["value_us"] > 0
    assert pre["roofline"]["kernel"] == "gemm_lds_kernel" and pre["roofline_gemm2"]["avg_us"] > 0
    assert "cpu_baseline" not in d
    dec = d.get("dsv4flash_t8_decode_single_launch")     # the MX types: a decode batch as one launch
    assert (dec is not None) == (mma != "nvf4xnvf4")
    if dec is not None:
        assert dec["config"]["tokens"] == 8 and dec["roofline"]["kernel"] == "mega_moe_kernel"
        assert 0 < dec["value_us"] and 0 < dec["multi_launch_us"]
        assert abs(dec["roofline"]["frac"] - dec["roofline"]["achieved"] / dec["roofline"]["peak"]) < 1e-3
    fw = d["forward_us"]
    assert 0 < fw["min"] <= fw["median"] <= fw["max"]
    ceil = d["ceiling"]                                         # measured ceilings beside the published peaks
    assert 0 < ceil["read_GBps"] and 0 < ceil["read_nt_GBps"] and 0 < ceil["mfma_fp4_TFLOPs"]
    ref = (ceil["read_nt_GBps"] if roof["bound"] == "hbm"
           else ceil["mfma_fp8xfp4_TFLOPs" if mma == "fp8xfp4" else "mfma_fp4_TFLOPs"])
    assert abs(ceil["gemm1_frac"] - roof["achieved"] / ref) < 1e-3


def test_cpu_baseline_times_one_whole_forward():
    import synth
    sys.path.insert(0, ROOT)
    import bench
    cfg = synth.CONFIGS[0]
    x = synth.make_tokens(cfg)
    ids, w = synth.make_routing(cfg)
    cb = bench.cpu_baseline(cfg, x, ids, w)
    assert cb["kind"] == "oracle" and cb["unit"] == "us" and cb["value"] > 0 and cb["cores"] >= 1
    assert "whole forward" in cb["sample"] and "blas" in cb

"""The committed rocprofv3 summaries agree with the bench lines they were taken
with (CPU tier, reads profiles/ only).

Each kernel-trace summary holds the trace's per-kernel durations and the bench
line of the same run.  Each GEMM's average duration in the trace, over the
dispatches that bench.py's events bracket, must agree with the event-timed
duration its roofline uses; the events also bracket the launch, so they may
read a little longer, never shorter by more than the timers' noise."""
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TRACES = sorted(glob.glob(os.path.join(ROOT, "profiles", "moe_layer_*_kernel_trace.md")))


def test_every_workload_and_mma_type_has_a_trace():
    names = {os.path.basename(p) for p in TRACES}
    for wl in ("dsv4flash_t64_decode", "dsv4flash_t512", "dsv4flash_t4096_prefill", "dsv4flash_t16384_zipf1.1"):
        for sfx in ("", "_fp8xfp4"):
            assert f"moe_layer_{wl}{sfx}_kernel_trace.md" in names


@pytest.mark.parametrize("path", TRACES, ids=os.path.basename)
@pytest.mark.parametrize("gemm", ["GEMM1", "GEMM2"])
def test_gemm_trace_duration_agrees_with_the_event_timing(path, gemm):
    """The trace's average over the split-loop dispatches that the events
    bracket; the events also time the gaps around each launch, so they may
    read up to 3 % or 6 us longer, never shorter by more than 1 %."""
    text = open(path).read()
    m = re.search(gemm + r" \(`(\w+)`, \w+-bound\): ([\d.]+) us per launch from events", text)
    assert m, f"no {gemm} bench line"
    events_us = float(m.group(2))
    w = re.search(gemm + r" kernel-trace average over the \d+ split-loop dispatches that the events bracket: "
                  r"([\d.]+) us", text)
    assert w, f"no windowed {gemm} trace average"
    trace_us = float(w.group(1))
    assert -0.01 * trace_us <= events_us - trace_us <= max(0.03 * trace_us, 6.0), (trace_us, events_us)


@pytest.mark.parametrize("path", TRACES, ids=os.path.basename)
def test_gemm1_kernel_row_agrees_with_its_split_loop_average(path):
    """The table's average over all dispatches is close to the split-loop
    average (the first, warm-up dispatches of the prefill GEMMs run a few %
    slower)."""
    text = open(path).read()
    kernel = re.search(r"- GEMM1 \(`(\w+)`", text).group(1)
    # the LDS-staged kernels serve both GEMMs: GEMM1 is the <true, ...> instantiation
    tiled = kernel in ("gemm_lds_kernel", "gemm_lds_nv_kernel")
    pat = r"\| `moe::" + kernel + (r"<true, [^`]*" if tiled else r"<[^`]*") + r"` \| (\d+) \| ([\d.]+) \|"
    rows = re.findall(pat, text)
    assert len(rows) == 1, rows
    all_us = float(rows[0][1])
    split_us = float(re.search(r"GEMM1 kernel-trace average over the \d+ split-loop dispatches that the events "
                               r"bracket: ([\d.]+) us", text).group(1))
    assert abs(all_us - split_us) / split_us <= 0.05, (all_us, split_us)


COUNTERS = sorted(glob.glob(os.path.join(ROOT, "profiles", "*_hbm_counters.txt")))


@pytest.mark.parametrize("path", COUNTERS, ids=os.path.basename)
def test_hbm_counters_match_the_current_kernel_sources(path):
    """bench.py reports a kernel's HBM traffic from these files only while
    their source hash matches: a kernel changed without retaking its
    counters would silently drop the bench line's "traffic"."""
    import bench
    kv = dict(l.split("=", 1) for l in open(path) if "=" in l and not l.lstrip().startswith("#"))
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    name = os.path.basename(path)[:-len("_hbm_counters.txt")]
    matches = [(g, p) for (g, p), (_, label, _) in bench.KERNELS.items() if name.startswith(label + "_dsv4flash")
               and (label != "gemm_lds_kernel" or not name.startswith("gemm_lds_kernel_gemm2"))]
    assert len(matches) == 1, (name, matches)
    gemm, kpath = matches[0]
    workload = name[len(bench.KERNELS[matches[0]][1]) + 1:]
    fp8 = workload.endswith("_fp8xfp4")
    traffic = bench.measured_traffic(workload[:-len("_fp8xfp4")] if fp8 else workload, gemm, kpath, fp8)
    assert traffic is not None, f"{name}: kernel sources changed since the counters were taken"
    assert traffic > 0

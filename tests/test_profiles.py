"""The committed rocprofv3 summaries agree with the bench lines they were taken
with (CPU tier, reads profiles/ only).

Each kernel-trace summary holds the trace's per-kernel durations and the bench
line of the same run.  GEMM1's average duration in the trace must agree with
the event-timed GEMM1 duration that bench.py's roofline uses; the events also
bracket the launch, so they may read a little longer, never shorter by more
than the timers' noise."""
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
def test_gemm1_trace_duration_agrees_with_the_event_timing(path):
    text = open(path).read()
    m = re.search(r"- GEMM1 \(`(\w+)`, \w+-bound\): ([\d.]+) us per launch from events", text)
    assert m, "no GEMM1 bench line"
    kernel, events_us = m.group(1), float(m.group(2))
    # the GEMM1 form of the kernel: gemm1_swiglu_kernel, or gemm_lds_kernel<true, ...>
    pat = r"\| `moe::" + kernel + (r"<true, [^`]*" if kernel == "gemm_lds_kernel" else r"<[^`]*") + r"` \| (\d+) \| ([\d.]+) \|"
    rows = re.findall(pat, text)
    assert len(rows) == 1, rows
    trace_us = float(rows[0][1])
    assert -0.01 <= (events_us - trace_us) / trace_us <= 0.03, (trace_us, events_us)

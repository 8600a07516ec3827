"""CPU check of the generated gfx950 code of the LDS-staged prefill GEMMs.

Their direct-to-LDS loads are issued from inline assembly, with M0 set in the
same statement (followed by the one wait state a DMA that reads a freshly
written M0 needs) and completion tracked by explicit in-order vmcnt waits.  That
is only sound while the compiler's own code neither uses M0 nor waits on
vmcnt inside these kernels (a compiler wait would count only the loads it
knows of and drain the ring), and while nothing spills to scratch.  The test
compiles the source to assembly with hipcc (cross-compiling; no GPU needed).
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_scaled_fp4_pre_amd", "csrc")


def _hipcc():
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return None


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "gemm_lds.s"
    cmd = [hipcc, "-O3", "-std=c++17", "-I", os.path.join(ROOT, "include"), "--offload-arch=gfx950",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "--cuda-device-only", "-S",
           "-o", str(out), os.path.join(CSRC, "gemm_lds.hip")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    text = out.read_text()
    found = {}
    for m in re.finditer(r"^(_ZN3moe\w*gemm_lds\w*):(?:\s*;.*)?$", text, re.M):
        end = text.find("s_endpgm", m.end())
        found[m.group(1)] = text[m.end():end]
    meta = {}
    for m in re.finditer(r"^\s+\.name:\s+(_ZN3moe\w*gemm_lds\w*)\s*$", text, re.M):
        blk = text[max(0, m.start() - 3000):m.start() + 3000]
        sc = re.search(r"\.private_segment_fixed_size:\s+(\d+)", blk)
        meta[m.group(1)] = int(sc.group(1)) if sc else None
    assert found, "no gemm_lds kernels in the assembly"
    return found, meta


def _split_asm(body):
    """(compiler lines, list of inline-asm blocks, compiler lines after the
    first inline-asm DMA) of one kernel body."""
    compiler, blocks, after, cur, seen_dma = [], [], [], None, False
    for line in body.splitlines():
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            cur = []
            continue
        if t.startswith(";;#ASMEND"):
            blocks.append(cur)
            seen_dma = seen_dma or any(x.startswith("global_load_lds") for x in cur)
            cur = None
            continue
        if not t or t.startswith(";") or t.startswith("."):
            continue
        if cur is not None:
            cur.append(t)
        else:
            compiler.append(t)
            if seen_dma:
                after.append(t)
    return compiler, blocks, after


def test_m0_only_in_dma_statements(kernels):
    found, _ = kernels
    for name, body in found.items():
        compiler, blocks, _ = _split_asm(body)
        assert not [t for t in compiler if re.search(r"\bm0\b", t)], name
        for b in blocks:
            if any(re.search(r"\bm0\b", t) for t in b):
                # M0 written, one wait state, then the DMA that reads it
                assert len(b) == 3 and b[0].startswith("s_mov_b32 m0,"), (name, b)
                assert b[1].startswith("s_nop"), (name, b)
                assert b[2].startswith("global_load_lds_dword"), (name, b)


def test_no_compiler_vmcnt_waits_once_the_ring_runs(kernels):
    # (the routed-row index loads before the first DMA may be waited for)
    found, _ = kernels
    for name, body in found.items():
        _, _, after = _split_asm(body)
        waits = [t for t in after if t.startswith("s_waitcnt") and "vmcnt" in t]
        assert not waits, (name, waits[:4])


def test_no_scratch(kernels):
    found, meta = kernels
    for name in found:
        assert meta.get(name) == 0, (name, meta.get(name))

"""Build libmoe_w4a4.so in-tree with hipcc for gfx950.

    python block_scaled_fp4_pre_amd/build.py      (or __graft_entry__.build())

Each source of the layer under csrc/ is compiled to an object in _build/ and the
objects are linked into block_scaled_fp4_pre_amd/libmoe_w4a4.so next to the
binding.  The measurement probes (csrc/ceiling.hip) become a library of their
own, libmoe_ceiling.so, so that the layer's library holds the layer only.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmoe_w4a4.so")
PROBE_LIB = os.path.join(HERE, "libmoe_ceiling.so")
PROBE_SOURCES = ("ceiling.hip",)
# The MFMA probe keeps its accumulators in VGPRs: in AGPRs the compiler
# rotated them through copies on every loop iteration.
SOURCE_FLAGS = {"ceiling.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
ARCH = "gfx950"

DEVICE_SOURCES = ("quant.hip", "route.hip", "predispatch.hip", "gemm1.hip", "gemm2.hip", "gemm_lds.hip",
                  "gemm_nv.hip", "gemm_lds_nv.hip", "combine.hip",
                  "prepare.hip", "noalloc.hip", "mega.hip")
HOST_SOURCES = ("abi.cpp", "validate.cpp")
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include")]
# Packed fp32 VALU ops are kept out of the device code.
DEVICE_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# abi.cpp and validate.cpp hold host code only: plain C++ (abi.cpp against the HIP runtime headers).
HOST_FLAGS = ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(args):
    cmd, src = args
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    jobs, objs, probe_objs = [], [], []
    for src in DEVICE_SOURCES + HOST_SOURCES + PROBE_SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        flags = COMMON + (DEVICE_FLAGS if src.endswith(".hip") else HOST_FLAGS) + SOURCE_FLAGS.get(src, [])
        jobs.append(([hipcc, *flags, "-c", os.path.join(CSRC, src), "-o", obj], src))
        (probe_objs if src in PROBE_SOURCES else objs).append(obj)
    workers = min(len(jobs), max(1, (os.cpu_count() or 4)))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        for out in ex.map(_compile, jobs):
            if verbose and out.strip():
                print(out)
    for lib, lib_objs in ((LIB, objs), (PROBE_LIB, probe_objs)):
        tmp = lib + ".tmp"
        link = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *lib_objs]
        r = subprocess.run(link, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"linking failed:\n{' '.join(link)}\n{r.stdout}{r.stderr}")
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

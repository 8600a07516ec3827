"""The C ABI's host-side argument checks (block_scaled_fp4_pre_amd/csrc/validate.cpp,
which abi.cpp runs before any HIP call) built on their own with g++ under
the address and undefined-behaviour sanitizers, and driven through every
error path by tests/abi_host_check.cpp.  No GPU and no HIP runtime involved."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "block_scaled_fp4_pre_amd", "csrc")


def test_every_validation_path_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = tmp_path / "abi_host_check"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "validate.cpp"), os.path.join(HERE, "abi_host_check.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    assert r.stdout.strip().endswith("0 failed"), r.stdout
    n = int(r.stdout.split()[-4])
    assert n >= 100, r.stdout

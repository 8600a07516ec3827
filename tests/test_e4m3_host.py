"""The device E4M3 quantizer's arithmetic (csrc/e4m3.h), built for the host
with g++, against the oracle (oracle.mxfp8): every bfloat16 value as a lone
value in a group, every midpoint between neighbouring E4M3 magnitudes, and
random groups over a wide range of scales.  Codes and scale bytes must be
identical."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import mxfp8

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def quantizer(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = tmp_path_factory.mktemp("e4m3") / "e4m3_host"
    r = subprocess.run([gxx, "-std=c++17", "-O2", "-o", str(exe), os.path.join(HERE, "e4m3_host.cpp")],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr

    def run(groups):
        g = np.ascontiguousarray(groups, dtype=np.float32)
        out = subprocess.run([str(exe)], input=g.tobytes(), capture_output=True, check=True).stdout
        a = np.frombuffer(out, dtype=np.uint8).reshape(-1, 33)
        return a[:, :32], a[:, 32]
    return run


def check(run, groups):
    codes, scales = run(groups)
    want_c, want_s = mxfp8.quantize(np.asarray(groups, dtype=np.float32).astype(np.float64))
    assert np.array_equal(scales, want_s[:, 0])
    assert np.array_equal(codes, want_c)


def test_every_bf16_lone_value(quantizer):
    bits = np.arange(1 << 16, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    f = f[np.isfinite(f)]
    g = np.zeros((f.size, 32), dtype=np.float32)
    g[:, 7] = f
    check(quantizer, g)


def test_midpoints_and_neighbours(quantizer):
    mags = mxfp8.E4M3_MAGNITUDES
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)     # exact in fp32
    rows = []
    for e in (-127, -126, -20, 0, 9, 100):
        for m in (mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(-np.inf))):
            g = np.zeros((m.size, 32), dtype=np.float32)
            g[:, 0] = np.float32(np.ldexp(448.0, e))                # fixes the scale 2^e
            g[:, 1] = np.ldexp(m.astype(np.float64), e).astype(np.float32)
            g[:, 2] = -g[:, 1]
            rows.append(g)
    g = np.concatenate(rows)
    keep = np.all(np.isfinite(g), axis=1)
    check(quantizer, g[keep])


def test_random_groups_wide_scales(quantizer):
    rng = np.random.default_rng(3)
    g = (rng.standard_normal((20000, 32)) * np.exp2(rng.integers(-130, 120, (20000, 1)))).astype(np.float32)
    g[::7, 3] = 0.0
    g[::11, 4] = -0.0
    check(quantizer, g)

"""Pins for oracle.bf16: against torch's fp32->bf16 conversion (round to nearest
even) on fp32-exact inputs, and by brute force over neighbouring bf16 values."""
import numpy as np
import torch

from oracle import bf16


def test_encode_matches_torch_on_fp32_values():
    rng = np.random.default_rng(0)
    f = (rng.standard_normal(200000) * np.exp(rng.uniform(-80, 80, 200000))).astype(np.float32)
    # add exact ties: bf16 value + half an ulp
    base = (rng.integers(0x0080, 0x7F00, 5000).astype(np.uint32) << 16)
    ties = (base | 0x8000).view(np.float32)
    f = np.concatenate([f, ties, -ties, np.array([0.0, -0.0], np.float32)])
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = bf16.encode(f.astype(np.float64))
    assert np.array_equal(got, want)


def test_decode_matches_torch():
    bits = np.arange(1 << 16, dtype=np.uint16)
    f = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy().astype(np.float64)
    d = bf16.decode(bits)
    fin = np.isfinite(f)
    assert np.array_equal(d[fin], f[fin])


def test_encode_is_nearest_fp64():
    rng = np.random.default_rng(1)
    v = rng.standard_normal(20000) * np.exp(rng.uniform(-60, 60, 20000))
    b = bf16.encode(v).astype(np.int64)
    here = bf16.decode(b.astype(np.uint16))
    for step in (-1, 1):
        nb = b + step
        ok = ((nb & 0x7FFF) < 0x7F80) & (nb >= 0) & (nb < 0x10000)
        other = bf16.decode(nb[ok].astype(np.uint16))
        d_here = np.abs(v[ok] - here[ok])
        d_other = np.abs(v[ok] - other)
        assert np.all(d_here <= d_other)
        tie = d_here == d_other
        assert np.all((b[ok][tie] & 1) == 0)

"""The measurement probes of libmoe_ceiling.so (include/moe_ceiling.h).

CPU: the library exports every declared symbol and rejects bad arguments
before any HIP call.  GPU: the streaming read visits every byte of every chunk
exactly once (its per-workgroup XOR equals numpy's, also for chunks that end
inside a ring round), and the three MFMA loops run every MFMA (exact sums)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "moe_ceiling.h")).read()
    return sorted(set(re.findall(r"\bint\s+(moe_ceiling_\w+)\s*\(", text)))


def test_probe_library_exports_every_declared_symbol():
    from block_scaled_fp4_pre_amd import ceiling
    names = _declared()
    assert names == ["moe_ceiling_mfma_bf16", "moe_ceiling_mfma_fp4", "moe_ceiling_mfma_fp8xfp4",
                     "moe_ceiling_stream_read"]
    for n in names:
        assert hasattr(ceiling._lib, n), n


def test_probe_arguments_checked_before_any_hip_call():
    from block_scaled_fp4_pre_amd import ceiling
    lib, EINVAL = ceiling._lib, ceiling.MOE_CEILING_EINVAL
    fake = ctypes.c_void_p(1 << 20)          # never dereferenced: every call below fails its checks
    assert lib.moe_ceiling_stream_read(None, 1 << 20, 4, 1, fake, None) == EINVAL
    assert lib.moe_ceiling_stream_read(fake, 1 << 20, 4, 1, None, None) == EINVAL
    assert lib.moe_ceiling_stream_read(fake, 1 << 20, 0, 1, fake, None) == EINVAL
    assert lib.moe_ceiling_stream_read(fake, 0, 4, 1, fake, None) == EINVAL
    assert lib.moe_ceiling_stream_read(fake, 16 * 4 + 8, 4, 1, fake, None) == EINVAL        # not 16 B per workgroup
    assert lib.moe_ceiling_stream_read(ctypes.c_void_p((1 << 20) + 4), 1 << 20, 4, 1, fake, None) == EINVAL
    assert lib.moe_ceiling_stream_read(fake, 1 << 32, 1, 1, fake, None) == EINVAL          # chunk >= 2^31
    assert lib.moe_ceiling_mfma_fp4(4, 0, fake, None) == EINVAL
    assert lib.moe_ceiling_mfma_fp4(4, 16385, fake, None) == EINVAL
    assert lib.moe_ceiling_mfma_fp4(0, 10, fake, None) == EINVAL
    assert lib.moe_ceiling_mfma_fp4(4, 10, None, None) == EINVAL
    assert lib.moe_ceiling_mfma_fp8xfp4(4, 0, fake, None) == EINVAL
    assert lib.moe_ceiling_mfma_fp8xfp4(4, 10, None, None) == EINVAL
    assert lib.moe_ceiling_mfma_bf16(4, 0, fake, None) == EINVAL
    assert lib.moe_ceiling_mfma_bf16(4, 16385, fake, None) == EINVAL
    assert lib.moe_ceiling_mfma_bf16(4, 10, None, None) == EINVAL


@pytest.mark.gpu
@pytest.mark.parametrize("chunk", [32768 * 4, 40976, 16])
@pytest.mark.parametrize("non_temporal", [True, False])
def test_stream_read_xors_every_word(chunk, non_temporal):
    import torch
    from block_scaled_fp4_pre_amd import ceiling
    from tests.gpu_support import log
    wgs = 96
    log(f"[test] stream-read probe: {wgs} workgroups x {chunk} B, non_temporal={non_temporal}")
    rng = np.random.default_rng(chunk)
    host = rng.integers(0, 2**32, size=wgs * chunk // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    digest = torch.zeros(wgs, dtype=torch.int32, device="cuda")
    ceiling.moe_ceiling_stream_read(src, wgs, non_temporal, digest)
    torch.cuda.synchronize()
    expect = np.bitwise_xor.reduce(host.reshape(wgs, -1), axis=1)
    assert np.array_equal(digest.cpu().numpy().view(np.uint32), expect)


@pytest.mark.gpu
@pytest.mark.parametrize("form,k", [("fp4", 128), ("fp8xfp4", 128), ("bf16", 32)])
def test_mfma_probe_sums_are_exact(form, k):
    import torch
    from block_scaled_fp4_pre_amd import ceiling
    from tests.gpu_support import log
    log(f"[test] {form} MFMA probe: 40 workgroups x 1000 iterations")
    out = torch.full((160,), -1.0, dtype=torch.float32, device="cuda")
    getattr(ceiling, f"moe_ceiling_mfma_{form}")(40, 1000, out)
    torch.cuda.synchronize()
    assert bool((out == 8 * k * 1000).all())


@pytest.mark.gpu
def test_measure_reports_checked_rates():
    from block_scaled_fp4_pre_amd import ceiling
    from tests.gpu_support import log
    log("[test] ceiling.measure at reduced sizes")
    res = ceiling.measure(read_bytes=256 << 20, workgroups=(256, 512), reps=2, mfma_workgroups=512,
                          mfma_iterations=256)
    log(f"    {res}")
    assert res["read_nt_GBps"] > 0 and res["read_GBps"] > 0
    assert res["mfma_fp4_TFLOPs"] > 0 and res["mfma_fp8xfp4_TFLOPs"] > 0 and res["mfma_bf16_TFLOPs"] > 0

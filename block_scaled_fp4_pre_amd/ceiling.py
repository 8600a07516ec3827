"""ctypes binding of libmoe_ceiling.so (include/moe_ceiling.h) and the two
measurements built on it: the practical HBM streaming-read rate and the
practical FP4 MFMA rate of the GPU, timed with events on the stream the probes
run on.  Argument marshalling and timing only; the probes are HIP kernels."""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads torch's HIP runtime before the library binds to it)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_ceiling.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                      "(or python block_scaled_fp4_pre_amd/build.py)")
_lib = ctypes.CDLL(LIB_PATH)
_lib.moe_ceiling_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int,
                                         ctypes.c_void_p, ctypes.c_void_p]
_lib.moe_ceiling_stream_read.restype = ctypes.c_int
_lib.moe_ceiling_mfma_fp4.argtypes = [ctypes.c_uint32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
_lib.moe_ceiling_mfma_fp4.restype = ctypes.c_int
_lib.moe_ceiling_mfma_fp8xfp4.argtypes = _lib.moe_ceiling_mfma_fp4.argtypes
_lib.moe_ceiling_mfma_fp8xfp4.restype = ctypes.c_int
_lib.moe_ceiling_mfma_bf16.argtypes = _lib.moe_ceiling_mfma_fp4.argtypes
_lib.moe_ceiling_mfma_bf16.restype = ctypes.c_int

MOE_CEILING_OK, MOE_CEILING_EINVAL, MOE_CEILING_EHIP = 0, 1, 2
FLOPS_PER_MFMA = 2 * 16 * 16 * 128
FLOPS_PER_MFMA_BF16 = 2 * 16 * 16 * 32
CHAINS = 8


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _check(st: int, what: str) -> None:
    if st != MOE_CEILING_OK:
        raise RuntimeError(f"{what} failed with status {st}")


def moe_ceiling_stream_read(src: torch.Tensor, workgroups: int, non_temporal: bool, digest: torch.Tensor) -> None:
    assert src.is_cuda and digest.is_cuda and digest.dtype == torch.int32 and digest.numel() >= workgroups
    _check(_lib.moe_ceiling_stream_read(src.data_ptr(), src.numel() * src.element_size(), workgroups,
                                        int(non_temporal), digest.data_ptr(), _stream()), "moe_ceiling_stream_read")


def moe_ceiling_mfma_bf16(workgroups: int, iterations: int, out: torch.Tensor) -> None:
    assert out.is_cuda and out.dtype == torch.float32 and out.numel() >= 4 * workgroups
    _check(_lib.moe_ceiling_mfma_bf16(workgroups, iterations, out.data_ptr(), _stream()), "moe_ceiling_mfma_bf16")


def moe_ceiling_mfma_fp4(workgroups: int, iterations: int, out: torch.Tensor) -> None:
    assert out.is_cuda and out.dtype == torch.float32 and out.numel() >= 4 * workgroups
    _check(_lib.moe_ceiling_mfma_fp4(workgroups, iterations, out.data_ptr(), _stream()), "moe_ceiling_mfma_fp4")


def moe_ceiling_mfma_fp8xfp4(workgroups: int, iterations: int, out: torch.Tensor) -> None:
    assert out.is_cuda and out.dtype == torch.float32 and out.numel() >= 4 * workgroups
    _check(_lib.moe_ceiling_mfma_fp8xfp4(workgroups, iterations, out.data_ptr(), _stream()),
           "moe_ceiling_mfma_fp8xfp4")


def _timed_ms(fn, reps: int) -> list[float]:
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    return times


def measure(read_bytes: int = 2 << 30, workgroups=(512, 1024, 2048, 4096), reps: int = 5,
            mfma_workgroups: int = 2048, mfma_iterations: int = 2048) -> dict:
    """Best-of-`reps` rates of the two probes on cuda:0: a streaming read of a
    `read_bytes` random buffer, each workgroup reading one contiguous chunk,
    with non-temporal and with default loads, best over the `workgroups`
    counts (2 to 16 per CU); and `mfma_workgroups` x 4 waves of back-to-back
    MFMAs of each MMA type (E2M1 x E2M1, E2M1 x E4M3) and of dense bf16.
    Each result is checked: the read's per-workgroup XOR against the same
    XOR taken by torch, the MFMA sums against their exact value."""
    src = torch.randint(-2**31, 2**31 - 1, (read_bytes // 4,), dtype=torch.int32, device="cuda")
    res = {"read_bytes": read_bytes}
    for wgs in workgroups:
        digest = torch.zeros(wgs, dtype=torch.int32, device="cuda")
        expect = _xor_rows(src.view(wgs, -1))
        for nt in (True, False):
            moe_ceiling_stream_read(src, wgs, nt, digest)            # warm-up, and the check
            torch.cuda.synchronize()
            if not torch.equal(digest, expect):
                raise RuntimeError("stream-read probe: digests differ from the buffer's XOR")
            ms = min(_timed_ms(lambda: moe_ceiling_stream_read(src, wgs, nt, digest), reps))
            key = "read_nt_GBps" if nt else "read_GBps"
            gbps = round(read_bytes / (ms * 1e-3) / 1e9, 1)
            if gbps > res.get(key, 0.0):
                res[key], res[key.replace("GBps", "workgroups")] = gbps, wgs
        del digest, expect
    del src
    out = torch.zeros(4 * mfma_workgroups, dtype=torch.float32, device="cuda")
    flops = 4 * mfma_workgroups * mfma_iterations * CHAINS * FLOPS_PER_MFMA
    for name, fn in (("mfma_fp4_TFLOPs", moe_ceiling_mfma_fp4), ("mfma_fp8xfp4_TFLOPs", moe_ceiling_mfma_fp8xfp4)):
        out.fill_(-1.0)
        fn(mfma_workgroups, mfma_iterations, out)
        torch.cuda.synchronize()
        if not bool((out == float(CHAINS * 128 * mfma_iterations)).all()):
            raise RuntimeError(f"MFMA probe ({name}): sums differ from 8*128*iterations")
        ms = min(_timed_ms(lambda: fn(mfma_workgroups, mfma_iterations, out), reps))
        res[name] = round(flops / (ms * 1e-3) / 1e12, 1)
    out.fill_(-1.0)
    moe_ceiling_mfma_bf16(mfma_workgroups, mfma_iterations, out)
    torch.cuda.synchronize()
    if not bool((out == float(CHAINS * 32 * mfma_iterations)).all()):
        raise RuntimeError("MFMA probe (bf16): sums differ from 8*32*iterations")
    ms = min(_timed_ms(lambda: moe_ceiling_mfma_bf16(mfma_workgroups, mfma_iterations, out), reps))
    res["mfma_bf16_TFLOPs"] = round(4 * mfma_workgroups * mfma_iterations * CHAINS * FLOPS_PER_MFMA_BF16 /
                                    (ms * 1e-3) / 1e12, 1)
    return res


def _xor_rows(x: torch.Tensor) -> torch.Tensor:
    """XOR along dim 1 of an int32 [rows, n] tensor, n a power of two, by halving."""
    n = x.shape[1]
    assert n & (n - 1) == 0
    while n > 1:
        n //= 2
        x = torch.bitwise_xor(x[:, :n], x[:, n:2 * n])
    return x[:, 0].contiguous()

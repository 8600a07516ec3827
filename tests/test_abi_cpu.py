"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every symbol include/moe_w4a4.h declares, and rejects bad arguments before any
HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_symbols():
    text = open(os.path.join(ROOT, "include", "moe_w4a4.h")).read()
    return sorted(set(re.findall(r"\b(moe_w4a4_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    from block_scaled_fp4_pre_amd import _lib
    declared = header_symbols()
    assert set(declared) == set(_lib.EXPORTED)
    for name in declared:
        assert hasattr(_lib.lib(), name), name


def test_query_sizes_dsv4():
    from block_scaled_fp4_pre_amd import _lib
    cfg = _lib.make_cfg(4096, 2048, 256, 6, 512)
    prepared, ws = _lib.moe_w4a4_query(cfg)
    assert prepared == 256 * 13369344          # all experts' MXFP4 codes + scales
    lay = _lib.moe_w4a4_workspace_layout(cfg)
    assert lay["total"] == ws
    assert all(v % 256 == 0 for v in lay.values())
    assert lay["y"] + 512 * 6 * 4096 * 2 <= ws               # y is bf16 [R, H]


@pytest.mark.parametrize("field,value,status", [
    ("hidden", 4000, 2), ("inter", 100, 2), ("group_size", 16, 2), ("mma_type", 2, 2),
    ("activation", 3, 2), ("num_experts", 0, 1), ("num_experts", 513, 2), ("topk", 0, 1),
    ("topk", 17, 2), ("max_tokens", -1, 1)])
def test_query_rejects_bad_config(field, value, status):
    from block_scaled_fp4_pre_amd import _lib
    cfg = _lib.make_cfg(256, 128, 8, 2, 16)
    setattr(cfg, field, value)
    with pytest.raises(_lib.MoeError) as ei:
        _lib.moe_w4a4_query(cfg)
    assert ei.value.status == status


def test_forward_validation_before_any_hip_call():
    from block_scaled_fp4_pre_amd import _lib
    L = _lib.lib()
    cfg = _lib.make_cfg(256, 128, 8, 2, 16)
    _, ws = _lib.moe_w4a4_query(cfg)
    P = ctypes.c_void_p
    fake = P(1 << 20)                       # never dereferenced: validation fails first
    # num_tokens above capacity
    st = L.moe_w4a4_forward(ctypes.byref(cfg), fake, 17, fake, fake, fake, fake, fake, ws, None)
    assert st == _lib.MOE_ECAPACITY
    # negative tokens
    st = L.moe_w4a4_forward(ctypes.byref(cfg), fake, -1, fake, fake, fake, fake, fake, ws, None)
    assert st == _lib.MOE_EINVAL
    # workspace too small
    st = L.moe_w4a4_forward(ctypes.byref(cfg), fake, 4, fake, fake, fake, fake, fake, ws - 1, None)
    assert st == _lib.MOE_EWORKSPACE
    # zero tokens: no pointer is looked at (empty tensors may be NULL)
    st = L.moe_w4a4_forward(ctypes.byref(cfg), None, 0, None, None, None, None, None, 0, None)
    assert st == _lib.MOE_OK
    st = L.moe_w4a4_forward(ctypes.byref(cfg), fake, 4, fake, fake, fake, fake, fake, ws - 1, None)
    assert st == _lib.MOE_EWORKSPACE
    # null / misaligned pointers
    st = L.moe_w4a4_forward(ctypes.byref(cfg), fake, 4, None, fake, fake, fake, fake, ws, None)
    assert st == _lib.MOE_EINVAL
    st = L.moe_w4a4_forward(ctypes.byref(cfg), fake, 4, P((1 << 20) + 2), fake, fake, fake, fake, ws, None)
    assert st == _lib.MOE_EINVAL
    st = L.moe_w4a4_forward(ctypes.byref(cfg), fake, 4, fake, fake, fake, fake, P((1 << 20) + 128), ws, None)
    assert st == _lib.MOE_EINVAL
    # unknown stage bits
    st = L.moe_w4a4_run_stages(ctypes.byref(cfg), fake, 4, fake, fake, fake, fake, fake, ws, 64, None, None)
    assert st == _lib.MOE_EINVAL
    # zero tokens is a no-op that succeeds without touching the device
    st = L.moe_w4a4_forward(ctypes.byref(cfg), fake, 0, fake, fake, fake, fake, fake, ws, None)
    assert st == _lib.MOE_OK
    # quantize argument checks
    assert L.moe_w4a4_quantize(2, fake, 4, 64, fake, fake, None) == _lib.MOE_EUNSUPPORTED
    assert L.moe_w4a4_quantize(0, fake, 4, 48, fake, fake, None) == _lib.MOE_EUNSUPPORTED
    assert L.moe_w4a4_quantize(0, fake, -1, 64, fake, fake, None) == _lib.MOE_EINVAL
    assert L.moe_w4a4_quantize(0, fake, 0, 64, fake, fake, None) == _lib.MOE_OK
    assert _lib.status_string(_lib.MOE_ECAPACITY).startswith("num_tokens")


def test_fp8_activations_double_the_token_regions():
    """mma_type fp8xfp4: x and h take one E4M3 byte per element instead of half."""
    from block_scaled_fp4_pre_amd import _lib
    c4 = _lib.make_cfg(4096, 2048, 256, 6, 512)
    c8 = _lib.make_cfg(4096, 2048, 256, 6, 512)
    c8.mma_type = _lib.MOE_MMA_FP8_X_MXF4
    l4, l8 = _lib.moe_w4a4_workspace_layout(c4), _lib.moe_w4a4_workspace_layout(c8)
    size = lambda lay, a, b: lay[b] - lay[a]
    assert size(l8, "xq", "xsf") == 2 * size(l4, "xq", "xsf") == 512 * 4096
    assert size(l8, "hq", "hsf") == 2 * size(l4, "hq", "hsf") == 512 * 6 * 2048
    assert _lib.moe_w4a4_query(c8)[0] == _lib.moe_w4a4_query(c4)[0]      # same MXFP4 weights


def test_prepare_weights_validation():
    from block_scaled_fp4_pre_amd import _lib
    L = _lib.lib()
    cfg = _lib.make_cfg(256, 128, 8, 2, 16)
    prepared, _ = _lib.moe_w4a4_query(cfg)
    P = ctypes.c_void_p
    fake = P(1 << 20)
    st = L.moe_w4a4_prepare_weights(ctypes.byref(cfg), None, fake, fake, fake, fake, prepared, None)
    assert st == _lib.MOE_EINVAL
    st = L.moe_w4a4_prepare_weights(ctypes.byref(cfg), fake, fake, fake, fake, P((1 << 20) + 64), prepared, None)
    assert st == _lib.MOE_EINVAL                       # prepared must be 256-byte aligned
    st = L.moe_w4a4_prepare_weights(ctypes.byref(cfg), fake, fake, fake, fake, fake, prepared - 1, None)
    assert st == _lib.MOE_EWORKSPACE
    bad = _lib.make_cfg(256, 128, 8, 2, 16)
    bad.mma_type = 7
    st = L.moe_w4a4_prepare_weights(ctypes.byref(bad), fake, fake, fake, fake, fake, prepared, None)
    assert st == _lib.MOE_EUNSUPPORTED


def test_valid_call_without_a_gfx950_reports_no_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: the call would run")
    from block_scaled_fp4_pre_amd import _lib
    L = _lib.lib()
    cfg = _lib.make_cfg(256, 128, 8, 2, 16)
    _, ws = _lib.moe_w4a4_query(cfg)
    fake = ctypes.c_void_p(1 << 20)                    # aligned, never dereferenced
    st = L.moe_w4a4_forward(ctypes.byref(cfg), fake, 4, fake, fake, fake, fake, fake, ws, None)
    assert st == _lib.MOE_ENODEVICE

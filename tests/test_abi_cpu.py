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
    return sorted(set(re.findall(r"\b(moe_w4a4_[a-z0-9_]+)\s*\(", text)))


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
    # all experts' MXFP4 codes + scales, then the 64 KiB tail the weight streams' read-ahead may touch
    assert prepared == 256 * 13369344 + 65536
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


def test_single_launch_forward_validation():
    """moe_w4a4_forward_mega checks its arguments as moe_w4a4_forward does and
    then refuses what it does not support, before any HIP call."""
    from block_scaled_fp4_pre_amd import _lib
    L = _lib.lib()
    P = ctypes.c_void_p
    fake = P(1 << 20)
    cfg = _lib.make_cfg(4096, 2048, 256, 6, 64)
    _, ws = _lib.moe_w4a4_query(cfg)
    fwd = lambda c, T, wsb=ws: L.moe_w4a4_forward_mega(ctypes.byref(c), fake, T, fake, fake, fake, fake, fake,
                                                         wsb, None)
    assert fwd(cfg, 43) == _lib.MOE_EUNSUPPORTED               # 258 routed rows
    assert fwd(cfg, 65) == _lib.MOE_ECAPACITY
    assert fwd(cfg, 4, ws - 1) == _lib.MOE_EWORKSPACE
    assert fwd(cfg, 0) == _lib.MOE_OK
    assert fwd(cfg, 4) == _lib.MOE_ENODEVICE                    # valid: only the device is missing
    fp8 = _lib.make_cfg(4096, 2048, 256, 6, 64, mma_type=_lib.MOE_MMA_FP8_X_MXF4)
    _, ws8 = _lib.moe_w4a4_query(fp8)
    assert fwd(fp8, 4, ws8) == _lib.MOE_ENODEVICE               # fp8xfp4: supported
    assert fwd(fp8, 43, ws8) == _lib.MOE_EUNSUPPORTED
    nv = _lib.make_cfg(4096, 2048, 256, 6, 64, mma_type=_lib.MOE_MMA_NVF4_X_NVF4)
    _, wsn = _lib.moe_w4a4_query(nv)
    assert fwd(nv, 4, wsn) == _lib.MOE_EUNSUPPORTED
    for H, I in ((768, 512), (1536, 512), (512, 1536), (3072, 2048)):   # K slices of 1, 2, 4 or 8 steps only
        odd = _lib.make_cfg(H, I, 8, 2, 16)
        _, wso = _lib.moe_w4a4_query(odd)
        assert fwd(odd, 4, wso) == _lib.MOE_EUNSUPPORTED, (H, I)
    lay = _lib.moe_w4a4_workspace_layout(cfg)
    assert lay["mega"] == 0 and lay["xq"] >= _lib.MOE_MEGA_STATE_BYTES


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


def test_prepared_buffer_has_the_read_ahead_tail():
    """The streaming GEMMs read up to 4 K steps (4 x 16 KiB of codes) past a
    unit's last step without consuming them; for the last expert those reads
    run past the four weight regions, into a 64 KiB tail of the buffer."""
    from block_scaled_fp4_pre_amd import _lib
    for H, I, E in ((256, 128, 8), (4096, 2048, 256), (768, 384, 5)):
        cfg = _lib.make_cfg(H, I, E, 2, 16)
        prepared, _ = _lib.moe_w4a4_query(cfg)
        regions = 0
        for nbytes in (E * 2 * I * H // 2, E * 2 * I * H // 32, E * H * I // 2, E * H * I // 32):
            regions = -(-(regions + nbytes) // 256) * 256
        assert prepared - regions == 65536, (H, I, E)


def _t(shape, dtype):
    import torch
    return torch.zeros(shape, dtype=dtype)


@pytest.mark.parametrize("case", ["ids_int64", "weights_bf16", "x_fp32", "x_narrow", "ids_short", "out_short",
                                  "out_narrow", "ids_wrong_k", "x_1d", "cpu_tensors"])
def test_binding_rejects_bad_tensors_before_the_library(case):
    """The binding hands the library raw pointers only, so it checks dtype,
    shape and device itself: topk_ids straight from torch.topk (int64) would
    otherwise be read as int32 pairs, and a short x or out would be read or
    written past its end by the kernels."""
    import torch
    from block_scaled_fp4_pre_amd import _lib
    T, H, k = 8, 256, 2
    cfg = _lib.make_cfg(H, 128, 8, k, 16)
    a = dict(x=_t((T, H), torch.bfloat16), topk_ids=_t((T, k), torch.int32), topk_weights=_t((T, k), torch.float32),
             out=_t((T, H), torch.bfloat16))
    bad = {"ids_int64": ("topk_ids", _t((T, k), torch.int64)),
           "weights_bf16": ("topk_weights", _t((T, k), torch.bfloat16)),
           "x_fp32": ("x", _t((T, H), torch.float32)),
           "x_narrow": ("x", _t((T, H // 2), torch.bfloat16)),
           "ids_short": ("topk_ids", _t((T - 1, k), torch.int32)),
           "out_short": ("out", _t((T - 1, H), torch.bfloat16)),
           "out_narrow": ("out", _t((T, H - 32), torch.bfloat16)),
           "ids_wrong_k": ("topk_ids", _t((T, k + 1), torch.int32)),
           "x_1d": ("x", _t((T * H,), torch.bfloat16)),
           "cpu_tensors": (None, None)}[case]
    if bad[0] is not None:
        a[bad[0]] = bad[1]
    ws = _t((1 << 20,), torch.uint8)
    prep = _t((1 << 20,), torch.uint8)
    with pytest.raises(ValueError):
        _lib.moe_w4a4_forward(cfg, prep, T, a["x"], a["topk_ids"], a["topk_weights"], a["out"], ws)
    with pytest.raises(ValueError):
        _lib.moe_w4a4_run_stages(cfg, prep, T, a["x"], a["topk_ids"], a["topk_weights"], a["out"], ws,
                                 _lib.MOE_STAGE_ALL)


def test_binding_rejects_bad_weight_and_quantize_buffers():
    import torch
    from block_scaled_fp4_pre_amd import _lib
    cfg = _lib.make_cfg(256, 128, 8, 2, 16)
    E, H, I = 8, 256, 128
    ok = [_t((E, 2 * I, H // 2), torch.uint8), _t((E, 2 * I, H // 32), torch.uint8),
          _t((E, H, I // 2), torch.uint8), _t((E, H, I // 32), torch.uint8)]
    for i in range(4):
        w = list(ok)
        w[i] = _t(tuple(w[i].shape[:-1]) + (w[i].shape[-1] - 1,), torch.uint8)
        with pytest.raises(ValueError):
            _lib.moe_w4a4_prepare_weights(cfg, *w, _t((1 << 20,), torch.uint8))
    with pytest.raises(ValueError):
        _lib.moe_w4a4_quantize(_t((4, 64), torch.float32), _t((4, 31), torch.uint8), _t((4, 2), torch.uint8))
    with pytest.raises(ValueError):
        _lib.moe_w4a4_quantize(_t((4, 64), torch.float64), _t((4, 32), torch.uint8), _t((4, 2), torch.uint8))


def test_binding_constants_match_the_header():
    """The binding's copies of the header's #define values."""
    import re
    from block_scaled_fp4_pre_amd import _lib
    text = open(os.path.join(os.path.dirname(__file__), "..", "include", "moe_w4a4.h")).read()
    for name in ("MOE_MEGA_MAX_ROWS", "MOE_MEGA_AUTO_ROWS", "MOE_MEGA_AUTO_ROWS_FP8", "MOE_MEGA_ERR_WORD",
                 "MOE_MEGA_HCOUNT_WORD", "MOE_NOALLOC_SCRATCH_BYTES",
                 "MOE_MEGA_STATE_BYTES"):
        m = re.search(rf"#define {name} \(?(\d+)u?(?: << (\d+))?\)?", text)
        assert m, name
        value = int(m.group(1)) << int(m.group(2) or 0)
        assert getattr(_lib, name) == value, name

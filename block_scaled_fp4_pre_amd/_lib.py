"""ctypes binding of libmoe_w4a4.so (C ABI in include/moe_w4a4.h).

Argument marshalling only: tensors are passed as raw device pointers, the
current torch stream as the HIP stream, and status codes become MoeError.
Every step of the layer runs in the library's HIP kernels; if the library is
missing this module raises at import time -- there is no other code path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_w4a4.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_ECAPACITY, MOE_EWORKSPACE, MOE_ENODEVICE, MOE_EHIP, MOE_ESCRATCH = range(8)
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20
MOE_MMA_MXF4_X_MXF4, MOE_MMA_FP8_X_MXF4, MOE_MMA_NVF4_X_NVF4 = 0, 1, 2
MOE_ACT_SWIGLU = 0
MOE_STAGE_QUANT, MOE_STAGE_ROUTE, MOE_STAGE_GEMM1, MOE_STAGE_GEMM2, MOE_STAGE_COMBINE = 1, 2, 4, 8, 16
MOE_STAGE_ALL = 31
MOE_MEGA_MAX_ROWS = 256          # routed rows the single-launch forward takes
MOE_MEGA_AUTO_ROWS = 48          # routed rows up to which moe_w4a4_forward takes it (MXFP4)
MOE_MEGA_AUTO_ROWS_FP8 = 24      # the same for fp8xfp4
MOE_MEGA_STATE_BYTES = 144 << 10  # its workspace state region (offset 0), zero before its first call
MOE_MEGA_ERR_WORD = 800           # uint64 word of that region that a wait which gave up sets
MOE_MEGA_HCOUNT_WORD = 816        # first per-expert h count of that region (words hcount + e)

# Every symbol include/moe_w4a4.h declares.
EXPORTED = (
    "moe_w4a4_query",
    "moe_w4a4_quantize",
    "moe_w4a4_quantize_nvfp4",
    "moe_w4a4_prepare_weights",
    "moe_w4a4_prepare_weights_nvfp4",
    "moe_w4a4_forward",
    "moe_w4a4_forward_mega",
    "moe_w4a4_forward_noalloc",
    "moe_w4a4_status_string",
    "moe_w4a4_workspace_layout",
    "moe_w4a4_run_stages",
)


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


class moe_w4a4_cfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "hidden", "inter", "num_experts", "topk", "max_tokens", "group_size", "mma_type", "activation")]


class moe_w4a4_ws_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "xq", "xsf", "counts", "offsets", "sorted_rows", "pos", "hist", "hq", "hsf", "y", "tiles",
        "num_tiles", "xsf_planes", "mega", "total")]


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                      "(python block_scaled_fp4_pre_amd/build.py)")
# torch ships its own HIP runtime.  Loading torch first makes the library bind
# to that same runtime (same devices, streams and allocations); loading the
# library first would bring in a second runtime next to torch's.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_sz = ctypes.c_size_t
_i32 = ctypes.c_int32
_CFG = ctypes.POINTER(moe_w4a4_cfg)
_lib.moe_w4a4_query.argtypes = [_CFG, ctypes.POINTER(_sz), ctypes.POINTER(_sz)]
_lib.moe_w4a4_quantize.argtypes = [_i32, _P, ctypes.c_int64, _i32, _P, _P, _P]
_lib.moe_w4a4_quantize_nvfp4.argtypes = [_i32, _P, ctypes.c_int64, _i32, ctypes.c_float, _P, _P, _P]
_lib.moe_w4a4_prepare_weights.argtypes = [_CFG, _P, _P, _P, _P, _P, _sz, _P]
_lib.moe_w4a4_prepare_weights_nvfp4.argtypes = [_CFG, _P, _P, _P, _P, _P, _P, ctypes.c_float, ctypes.c_float, _P,
                                                _sz, _P]
_lib.moe_w4a4_forward.argtypes = [_CFG, _P, _i32, _P, _P, _P, _P, _P, _sz, _P]
_lib.moe_w4a4_forward_mega.argtypes = [_CFG, _P, _i32, _P, _P, _P, _P, _P, _sz, _P]
_lib.moe_w4a4_forward_noalloc.argtypes = [_CFG, _P, _i32, _P, _P, _P, _P, _P]
_lib.moe_w4a4_status_string.argtypes = [ctypes.c_int]
_lib.moe_w4a4_status_string.restype = ctypes.c_char_p
_lib.moe_w4a4_workspace_layout.argtypes = [_CFG, ctypes.POINTER(moe_w4a4_ws_layout)]
_lib.moe_w4a4_run_stages.argtypes = [_CFG, _P, _i32, _P, _P, _P, _P, _P, _sz, ctypes.c_uint32, _P, _P]
for _n in EXPORTED:
    if _n != "moe_w4a4_status_string":
        getattr(_lib, _n).restype = ctypes.c_int


def lib() -> ctypes.CDLL:
    return _lib


def status_string(status: int) -> str:
    return _lib.moe_w4a4_status_string(int(status)).decode()


def _check(st: int, where: str) -> None:
    if st != MOE_OK:
        raise MoeError(st, where)


def _ptr(t) -> int | None:
    """Device address of a tensor (None -> NULL); no copies, no conversions."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


_BF16_LIKE = ("bfloat16", "int16", "uint16")   # bf16 values or their bit patterns


def _expect(t, name: str, dtypes, shape=None, min_rows=None) -> None:
    """Raise ValueError unless tensor t (if given) has one of the dtypes (by
    name), the exact shape (None entries match any size) or at least min_rows
    rows, and lives on the current device.  The library sees only pointers:
    a wrong dtype or a short buffer would be read or written out of bounds
    by the kernels, so it is refused here."""
    if t is None or isinstance(t, int):
        return
    dt = str(t.dtype).replace("torch.", "")
    if dt not in dtypes:
        raise ValueError(f"{name}: dtype {dt}, expected {' or '.join(dtypes)}")
    if shape is not None:
        if t.dim() != len(shape) or any(w is not None and w != g for g, w in zip(t.shape, shape)):
            raise ValueError(f"{name}: shape {tuple(t.shape)}, expected "
                             f"({', '.join('*' if w is None else str(w) for w in shape)})")
        if min_rows is not None and t.shape[0] < min_rows:
            raise ValueError(f"{name}: {t.shape[0]} rows, at least {min_rows} needed")
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a device tensor, got one on {t.device}")
    import torch
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name}: on {t.device}, but the current device is cuda:{torch.cuda.current_device()}")


def _check_forward_tensors(cfg, num_tokens, x, topk_ids, topk_weights, out, workspace, prepared,
                           gemm1_acc=None) -> None:
    T, H, k, I = int(num_tokens), cfg.hidden, cfg.topk, cfg.inter
    _expect(x, "x", _BF16_LIKE, (None, H), T)
    _expect(topk_ids, "topk_ids", ("int32",), (None, k), T)
    _expect(topk_weights, "topk_weights", ("float32",), (None, k), T)
    _expect(out, "out", _BF16_LIKE, (None, H), T)
    _expect(workspace, "workspace", ("uint8",))
    _expect(prepared, "prepared", ("uint8",))
    _expect(gemm1_acc, "gemm1_acc", ("float32",), (None, 2 * I), T * k)


def _stream(stream) -> int | None:
    if stream is not None:
        return int(stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


def make_cfg(hidden: int, inter: int, num_experts: int, topk: int, max_tokens: int,
             group_size: int | None = None, mma_type: int = MOE_MMA_MXF4_X_MXF4,
             activation: int = MOE_ACT_SWIGLU) -> moe_w4a4_cfg:
    """group_size None: the MMA type's own (16 for NVFP4, else 32)."""
    if group_size is None:
        group_size = 16 if mma_type == MOE_MMA_NVF4_X_NVF4 else 32
    return moe_w4a4_cfg(hidden, inter, num_experts, topk, max_tokens, group_size, mma_type, activation)


def scale_group(cfg) -> int:
    """Elements per scale byte of cfg's MMA type."""
    return 16 if cfg.mma_type == MOE_MMA_NVF4_X_NVF4 else 32


def moe_w4a4_query(cfg: moe_w4a4_cfg):
    """(prepared_bytes, workspace_bytes)."""
    p, w = _sz(), _sz()
    _check(_lib.moe_w4a4_query(ctypes.byref(cfg), ctypes.byref(p), ctypes.byref(w)), "moe_w4a4_query")
    return p.value, w.value


def moe_w4a4_workspace_layout(cfg: moe_w4a4_cfg) -> dict:
    lay = moe_w4a4_ws_layout()
    _check(_lib.moe_w4a4_workspace_layout(ctypes.byref(cfg), ctypes.byref(lay)), "moe_w4a4_workspace_layout")
    return {n: getattr(lay, n) for n, _ in moe_w4a4_ws_layout._fields_}


def moe_w4a4_quantize(src, codes, scales, stream=None) -> None:
    """src: device bf16 (or uint16 bit patterns) / float32 [rows, cols];
    codes uint8 [rows, cols/2]; scales uint8 [rows, cols/32]."""
    import torch
    if src.dtype in (torch.bfloat16, torch.uint16, torch.int16):
        dt = 0
    elif src.dtype == torch.float32:
        dt = 1
    else:
        raise ValueError(f"unsupported dtype {src.dtype}")
    if src.dim() != 2:
        raise ValueError(f"src: expected [rows, cols], got shape {tuple(src.shape)}")
    rows, cols = src.shape
    _expect(src, "src", ("bfloat16", "int16", "uint16", "float32"))
    _expect(codes, "codes", ("uint8",), (rows, cols // 2))
    _expect(scales, "scales", ("uint8",), (rows, cols // 32))
    _check(_lib.moe_w4a4_quantize(dt, _ptr(src), rows, cols, _ptr(codes), _ptr(scales), _stream(stream)),
           "moe_w4a4_quantize")


def moe_w4a4_quantize_nvfp4(src, g: float, codes, scales, stream=None) -> None:
    """NVFP4 with tensor scale g: src device bf16 (or uint16 bit patterns) /
    float32 [rows, cols]; codes uint8 [rows, cols/2]; scales uint8 [rows, cols/16]."""
    import torch
    if src.dtype in (torch.bfloat16, torch.uint16, torch.int16):
        dt = 0
    elif src.dtype == torch.float32:
        dt = 1
    else:
        raise ValueError(f"unsupported dtype {src.dtype}")
    if src.dim() != 2:
        raise ValueError(f"src: expected [rows, cols], got shape {tuple(src.shape)}")
    rows, cols = src.shape
    _expect(src, "src", ("bfloat16", "int16", "uint16", "float32"))
    _expect(codes, "codes", ("uint8",), (rows, cols // 2))
    _expect(scales, "scales", ("uint8",), (rows, cols // 16))
    _check(_lib.moe_w4a4_quantize_nvfp4(dt, _ptr(src), rows, cols, float(g), _ptr(codes), _ptr(scales),
                                        _stream(stream)), "moe_w4a4_quantize_nvfp4")


def moe_w4a4_prepare_weights_nvfp4(cfg, w1_codes, w1_scales, w1_tensor_scales, w2_codes, w2_scales,
                                   w2_tensor_scales, x_tensor_scale: float, h_tensor_scale: float, prepared,
                                   stream=None) -> None:
    E, H, I = cfg.num_experts, cfg.hidden, cfg.inter
    _expect(w1_codes, "w1_codes", ("uint8",), (E, 2 * I, H // 2))
    _expect(w1_scales, "w1_scales", ("uint8",), (E, 2 * I, H // 16))
    _expect(w1_tensor_scales, "w1_tensor_scales", ("float32",), (E,))
    _expect(w2_codes, "w2_codes", ("uint8",), (E, H, I // 2))
    _expect(w2_scales, "w2_scales", ("uint8",), (E, H, I // 16))
    _expect(w2_tensor_scales, "w2_tensor_scales", ("float32",), (E,))
    _expect(prepared, "prepared", ("uint8",))
    _check(_lib.moe_w4a4_prepare_weights_nvfp4(
        ctypes.byref(cfg), _ptr(w1_codes), _ptr(w1_scales), _ptr(w1_tensor_scales), _ptr(w2_codes), _ptr(w2_scales),
        _ptr(w2_tensor_scales), float(x_tensor_scale), float(h_tensor_scale), _ptr(prepared),
        prepared.numel() * prepared.element_size(), _stream(stream)), "moe_w4a4_prepare_weights_nvfp4")


def moe_w4a4_prepare_weights(cfg, w1_codes, w1_scales, w2_codes, w2_scales, prepared, stream=None) -> None:
    E, H, I = cfg.num_experts, cfg.hidden, cfg.inter
    _expect(w1_codes, "w1_codes", ("uint8",), (E, 2 * I, H // 2))
    _expect(w1_scales, "w1_scales", ("uint8",), (E, 2 * I, H // 32))
    _expect(w2_codes, "w2_codes", ("uint8",), (E, H, I // 2))
    _expect(w2_scales, "w2_scales", ("uint8",), (E, H, I // 32))
    _expect(prepared, "prepared", ("uint8",))
    _check(_lib.moe_w4a4_prepare_weights(ctypes.byref(cfg), _ptr(w1_codes), _ptr(w1_scales), _ptr(w2_codes),
                                         _ptr(w2_scales), _ptr(prepared), prepared.numel() * prepared.element_size(),
                                         _stream(stream)), "moe_w4a4_prepare_weights")


def moe_w4a4_forward(cfg, prepared, num_tokens: int, x, topk_ids, topk_weights, out, workspace,
                     stream=None) -> None:
    """x bf16 [>= T, H], topk_ids int32 [>= T, k], topk_weights float32
    [>= T, k], out bf16 [>= T, H], all on the current device; T = num_tokens."""
    _check_forward_tensors(cfg, num_tokens, x, topk_ids, topk_weights, out, workspace, prepared)
    _check(_lib.moe_w4a4_forward(ctypes.byref(cfg), _ptr(prepared), int(num_tokens), _ptr(x), _ptr(topk_ids),
                                 _ptr(topk_weights), _ptr(out), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream)),
           "moe_w4a4_forward")


def moe_w4a4_forward_mega(cfg, prepared, num_tokens: int, x, topk_ids, topk_weights, out, workspace,
                          stream=None) -> None:
    """The forward as one kernel launch (decode sizes); arguments as moe_w4a4_forward."""
    _check_forward_tensors(cfg, num_tokens, x, topk_ids, topk_weights, out, workspace, prepared)
    _check(_lib.moe_w4a4_forward_mega(ctypes.byref(cfg), _ptr(prepared), int(num_tokens), _ptr(x), _ptr(topk_ids),
                                      _ptr(topk_weights), _ptr(out), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), _stream(stream)),
           "moe_w4a4_forward_mega")


def moe_w4a4_forward_noalloc(cfg, prepared, num_tokens: int, x, topk_ids, topk_weights, out,
                             stream=None) -> None:
    """The forward on the library's static scratch instead of a workspace."""
    _check_forward_tensors(cfg, num_tokens, x, topk_ids, topk_weights, out, None, prepared)
    _check(_lib.moe_w4a4_forward_noalloc(ctypes.byref(cfg), _ptr(prepared), int(num_tokens), _ptr(x),
                                         _ptr(topk_ids), _ptr(topk_weights), _ptr(out), _stream(stream)),
           "moe_w4a4_forward_noalloc")


def moe_w4a4_run_stages(cfg, prepared, num_tokens: int, x, topk_ids, topk_weights, out, workspace,
                        stages: int, gemm1_acc=None, stream=None) -> None:
    _check_forward_tensors(cfg, num_tokens, x, topk_ids, topk_weights, out, workspace, prepared, gemm1_acc)
    _check(_lib.moe_w4a4_run_stages(ctypes.byref(cfg), _ptr(prepared), int(num_tokens), _ptr(x), _ptr(topk_ids),
                                    _ptr(topk_weights), _ptr(out), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), int(stages), _ptr(gemm1_acc),
                                    _stream(stream)), "moe_w4a4_run_stages")

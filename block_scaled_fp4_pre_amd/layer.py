"""MoeW4A4Layer: owns the device buffers of one layer and calls the C ABI.

PyTorch provides the device memory and the stream; every computation runs in
the library's HIP kernels.  Weights can be loaded either as canonical MXFP4
(codes + scale bytes) or as fp32 matrices, which are quantized on the device by
moe_w4a4_quantize and then re-laid by moe_w4a4_prepare_weights.  An NVFP4
layer (MOE_MMA_NVF4_X_NVF4) takes NVFP4 codes, E4M3 scale bytes per 16 and the
tensor scales instead (moe_w4a4_quantize_nvfp4, moe_w4a4_prepare_weights_nvfp4).
"""
from __future__ import annotations

import concurrent.futures

import torch

from . import _lib


class MoeW4A4Layer:
    def __init__(self, hidden: int, inter: int, num_experts: int, topk: int, max_tokens: int,
                 device: str | torch.device = "cuda", mma_type: int = _lib.MOE_MMA_MXF4_X_MXF4,
                 prepared: torch.Tensor | None = None):
        """mma_type: MOE_MMA_MXF4_X_MXF4 (MXFP4 activations) or MOE_MMA_FP8_X_MXF4
        (MXFP8 E4M3 activations), the weights MXFP4 in both; or
        MOE_MMA_NVF4_X_NVF4 (NVFP4 activations and weights).  prepared: an
        existing prepared-weights buffer of the same shape to share (see
        with_capacity), else a new one is allocated."""
        self.H, self.I, self.E, self.k, self.max_tokens = hidden, inter, num_experts, topk, max_tokens
        self.mma_type = mma_type
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.cfg = _lib.make_cfg(hidden, inter, num_experts, topk, max_tokens, mma_type=mma_type)
        pb, wb = _lib.moe_w4a4_query(self.cfg)
        if prepared is None:
            prepared = torch.empty(pb, dtype=torch.uint8, device=self.device)
        elif prepared.numel() * prepared.element_size() < pb or prepared.device != self.device:
            raise ValueError("shared prepared buffer is too small or on another device")
        self.prepared = prepared
        self.workspace = torch.empty(wb, dtype=torch.uint8, device=self.device)
        self.layout = _lib.moe_w4a4_workspace_layout(self.cfg)
        # the single-launch forward's state region: zero before its first call
        # (every call leaves it zero)
        m = self.layout["mega"]
        self.workspace[m:m + _lib.MOE_MEGA_STATE_BYTES].zero_()

    @property
    def nvfp4(self) -> bool:
        return self.mma_type == _lib.MOE_MMA_NVF4_X_NVF4

    def with_capacity(self, max_tokens: int, mma_type: int | None = None) -> "MoeW4A4Layer":
        """A layer over the same prepared weights (shared, not copied) with its
        own workspace for max_tokens tokens; mma_type may switch between the
        two MX types, which use the same MXFP4 weights."""
        mma = self.mma_type if mma_type is None else mma_type
        if (mma == _lib.MOE_MMA_NVF4_X_NVF4) != self.nvfp4:
            raise ValueError("NVFP4 and MXFP4 layers cannot share prepared weights")
        return MoeW4A4Layer(self.H, self.I, self.E, self.k, max_tokens, self.device, mma, prepared=self.prepared)

    # ---- weights ------------------------------------------------------------
    def canonical_buffers(self):
        H, I, E, G = self.H, self.I, self.E, _lib.scale_group(self.cfg)
        u8 = dict(dtype=torch.uint8, device=self.device)
        return (torch.empty((E, 2 * I, H // 2), **u8), torch.empty((E, 2 * I, H // G), **u8),
                torch.empty((E, H, I // 2), **u8), torch.empty((E, H, I // G), **u8))

    def load_canonical(self, w1_codes, w1_scales, w2_codes, w2_scales, tensor_scales=None) -> None:
        """tensor_scales (NVFP4 only): (g_x, g_h, g_w1 fp32 [E], g_w2 fp32 [E])."""
        if self.nvfp4:
            gx, gh, gw1, gw2 = tensor_scales
            gw1 = torch.as_tensor(gw1, dtype=torch.float32).to(self.device)
            gw2 = torch.as_tensor(gw2, dtype=torch.float32).to(self.device)
            _lib.moe_w4a4_prepare_weights_nvfp4(self.cfg, w1_codes, w1_scales, gw1, w2_codes, w2_scales, gw2,
                                                gx, gh, self.prepared)
            torch.cuda.current_stream(self.device).synchronize()   # gw1/gw2 are temporaries
        else:
            assert tensor_scales is None
            _lib.moe_w4a4_prepare_weights(self.cfg, w1_codes, w1_scales, w2_codes, w2_scales, self.prepared)

    def quantize_fp32_weights(self, expert_source, threads: int = 16, weight_scales=None):
        """expert_source(e) -> (W1 [2I, H], W2 [H, I]) fp32 arrays (host or device).
        Returns the canonical buffers (w1c, w1s, w2c, w2s) on the device: MXFP4,
        or NVFP4 with weight_scales = (g_w1 [E], g_w2 [E]) the tensor scales."""
        bufs = self.canonical_buffers()
        w1c, w1s, w2c, w2s = bufs
        with concurrent.futures.ThreadPoolExecutor(max(1, threads)) as ex:
            futs = [ex.submit(expert_source, e) for e in range(min(self.E, 2 * threads))]
            nxt = len(futs)
            for e in range(self.E):
                w1, w2 = futs[e].result()
                futs[e] = None
                if nxt < self.E:
                    futs.append(ex.submit(expert_source, nxt))
                    nxt += 1
                d1 = torch.as_tensor(w1).to(self.device, torch.float32)
                d2 = torch.as_tensor(w2).to(self.device, torch.float32)
                if self.nvfp4:
                    _lib.moe_w4a4_quantize_nvfp4(d1, float(weight_scales[0][e]), w1c[e], w1s[e])
                    _lib.moe_w4a4_quantize_nvfp4(d2, float(weight_scales[1][e]), w2c[e], w2s[e])
                else:
                    _lib.moe_w4a4_quantize(d1, w1c[e], w1s[e])
                    _lib.moe_w4a4_quantize(d2, w2c[e], w2s[e])
        return bufs

    def load_fp32(self, expert_source, threads: int = 16, keep_canonical: bool = False, tensor_scales=None):
        """tensor_scales (NVFP4 only): (g_x, g_h, g_w1 [E], g_w2 [E])."""
        bufs = self.quantize_fp32_weights(expert_source, threads,
                                          None if tensor_scales is None else tensor_scales[2:])
        self.load_canonical(*bufs, tensor_scales=tensor_scales)
        if keep_canonical:
            return bufs
        del bufs
        return None

    # ---- forward ------------------------------------------------------------
    def forward(self, x, topk_ids, topk_weights, out=None, stream=None):
        """x bf16 [T, H]; topk_ids int32 [T, k] (ids outside [0, E) are skipped);
        topk_weights float32 [T, k]; out bf16 [T, H] or None.  Every tensor must
        be on the layer's device; anything else raises ValueError before a
        kernel is launched."""
        T = x.shape[0]
        if out is None:
            out = torch.empty((T, self.H), dtype=torch.bfloat16, device=self.device)
        with torch.cuda.device(self.device):
            _lib.moe_w4a4_forward(self.cfg, self.prepared, T, x, topk_ids, topk_weights, out, self.workspace,
                                  stream=stream)
        return out

    def forward_mega(self, x, topk_ids, topk_weights, out=None, stream=None):
        """The forward as one kernel launch (moe_w4a4_forward_mega: MXFP4 or
        fp8xfp4, at most 256 routed rows); arguments as forward."""
        T = x.shape[0]
        if out is None:
            out = torch.empty((T, self.H), dtype=torch.bfloat16, device=self.device)
        with torch.cuda.device(self.device):
            _lib.moe_w4a4_forward_mega(self.cfg, self.prepared, T, x, topk_ids, topk_weights, out, self.workspace,
                                       stream=stream)
        return out

    def run_stages(self, stages, num_tokens, x=None, topk_ids=None, topk_weights=None, out=None,
                   gemm1_acc=None, stream=None):
        with torch.cuda.device(self.device):
            _lib.moe_w4a4_run_stages(self.cfg, self.prepared, num_tokens, x, topk_ids, topk_weights, out,
                                     self.workspace, stages, gemm1_acc=gemm1_acc, stream=stream)

    def ws(self, name: str, shape, dtype) -> torch.Tensor:
        """A view of one intermediate region of the workspace (see moe_w4a4_ws_layout)."""
        off = self.layout[name]
        n = 1
        for s in shape:
            n *= s
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        return self.workspace[off:off + nbytes].view(dtype).view(*shape)

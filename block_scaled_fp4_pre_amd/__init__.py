"""MI355X (gfx950) W4A4 routed-expert MoE layer: MXFP4 tokens x MXFP4 expert
weights, SwiGLU, DeepSeek-V4-Flash shape.  The layer runs in hand-written HIP
kernels behind the C ABI of include/moe_w4a4.h; this package is its thin
Python binding (block_scaled_fp4_pre_amd._lib) plus a small helper that owns
the device buffers (block_scaled_fp4_pre_amd.layer)."""
from ._lib import (  # noqa: F401
    EXPORTED,
    MOE_STAGE_ALL,
    MOE_STAGE_COMBINE,
    MOE_STAGE_GEMM1,
    MOE_STAGE_GEMM2,
    MOE_STAGE_QUANT,
    MOE_STAGE_ROUTE,
    MoeError,
    make_cfg,
    moe_w4a4_forward,
    moe_w4a4_prepare_weights,
    moe_w4a4_quantize,
    moe_w4a4_query,
    moe_w4a4_run_stages,
    moe_w4a4_workspace_layout,
    status_string,
)

"""Seeded synthetic inputs for the W4A4 MoE layer.

This module only draws random numbers and lays them out. It holds none of the
layer's arithmetic (no MXFP4 quantization, no routing sort, no GEMM): both the
oracle side and the device side take their inputs from here and transform them
independently.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    LayerConfig,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_routing,
    make_tokens,
    expert_weights_f32,
)

"""CPU oracle for the W4A4 (MXFP4 x MXFP4) routed-expert MoE layer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links
this package: only the tests, the smoke check and the CPU-baseline leg of the
benchmark use it. It shares no code with the device path and imports nothing
from it.

Plain, slow, fp64 NumPy code that follows the method step by step:
  mxfp4    E2M1 element codes and UE8M0 block scales (one per 32 elements)
  mxfp8    E4M3 element codes with the same scales (the fp8xfp4 MMA type)
  nvfp4    E2M1 codes with E4M3 scales per 16 and an fp32 tensor scale (NVFP4)
  bf16     bfloat16 encode/decode
  route    stable counting sort of routed rows by expert
  forward  quantize -> route -> GEMM1 + SwiGLU -> requantize -> GEMM2 -> combine
  dense    brute force: every expert on every token, masked by the routing

Pages cited in this package:
  [P1] sglang PR "[deepseek-v4] Bump sgl-deep-gemm for packed FP4xFP4 mega-MoE
       (W4A4)" (pull 28210).
  [P3] prhub digest of sglang PR "bump sgl-deep-gemm to 0.1.7, MegaMoE uses the
       mma_type API for MXFP4" (pull 37279).
  [OCP-MX] OCP Microscaling Formats (MX) Specification v1.0: the FP4 E2M1
       element format, the FP8 E4M3 element format and the E8M0 scale format.
       The pages name MXFP4, FP8 and UE8M0 but do not define them; the
       definitions come from this standard.  NVFP4 (E2M1 elements, E4M3
       scales per 16, an fp32 tensor scale) is the public format of that
       name; oracle.nvfp4 states the encoding rule read into it.

Pins: tests/test_oracle_*.py check every function against closed forms, brute
force and invariants. Where no pin exists a function's docstring says
"parity unpinned".
"""
from . import bf16, dense, forward, mxfp4, mxfp8, nvfp4, route  # noqa: F401

// MXFP8 E4M3 encoding of the fp8xfp4 MMA type's activations ([P3] prhub digest
// of sglang PR "bump sgl-deep-gemm to 0.1.7, MegaMoE uses the mma_type API for
// MXFP4", "Key source snippets": the fp8xfp4 pre_dispatch quantizes to FP8 with
// quant_group_size=32).  Element format per [OCP-MX] (OCP MX v1.0) FP8 E4M3:
// bit 7 sign, bits 6..3 exponent with bias 7, bits 2..0 mantissa; exponent
// field 0 is subnormal (m/8 * 2^-6); the largest magnitude is 448 (0x7E).
// Block scale: the UE8M0 byte of MXFP4, with 2^e the smallest power of two
// such that amax <= 448 * 2^e, clamped to [-127, 127].  Elements round to the
// nearest E4M3 value, ties to the even mantissa, sign kept (-0 -> 0x80).
//
// Plain integer and fp32 arithmetic only, so that the host compiler builds
// the same functions for an exhaustive check against the rule.
#pragma once
#include <math.h>
#include <stdint.h>

namespace moe {

__host__ __device__ inline uint32_t e4m3_f32_bits(float f) { return __builtin_bit_cast(uint32_t, f); }

// Scale exponent of a block from the fp32 bits of its absolute maximum.
// amax = m * 2^E with 1 <= m < 2 and 448 = 1.75 * 2^8: the smallest e with
// amax <= 448 * 2^e is E - 8 when m <= 1.75 (mantissa field <= 0x600000) and
// E - 7 otherwise.  Zero and fp32 subnormals land on the -127 clamp.
__host__ __device__ inline int mx8_scale_exp(uint32_t amax_bits) {
  const uint32_t ef = amax_bits >> 23;
  if (ef == 0) return -127;
  const int e = (int)ef - 135 + ((amax_bits & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// 2^k as an fp32 value for k in [-127, 127] (2^-127 is an fp32 subnormal).
__host__ __device__ inline float e4m3_exp2(int k) {
  return __builtin_bit_cast(float, k > -127 ? (uint32_t)(k + 127) << 23 : 0x00400000u);
}

// E4M3 code of r, already divided by the block scale (|r| <= 448).
//  - |r| < 2^-6: subnormal steps of 2^-9; |r| * 512 is exact and rintf rounds
//    it to the nearest integer, ties to even, giving 0..8 (8 is 2^-6, the
//    smallest normal, code 0x08).
//  - otherwise: round the fp32 mantissa to 3 bits, ties to even (a carry moves
//    into the exponent), and rebias the exponent from 127 to 7.
__host__ __device__ inline uint32_t e4m3_code(float r) {
  const uint32_t b = e4m3_f32_bits(r);
  const uint32_t a = b & 0x7FFFFFFFu;
  uint32_t c;
  if (a < 0x3C800000u) {
    c = (uint32_t)rintf(fabsf(r) * 512.0f);
  } else {
    const uint32_t rnd = a + 0x7FFFFu + ((a >> 20) & 1u);
    c = (rnd >> 20) - (120u << 3);
  }
  return c | ((b >> 24) & 0x80u);
}

// Codes of four values under the block scale 2^e (inv = 2^-e), byte i = v[i].
__host__ __device__ inline uint32_t e4m3_pack4(float v0, float v1, float v2, float v3, float inv) {
  return e4m3_code(v0 * inv) | (e4m3_code(v1 * inv) << 8) | (e4m3_code(v2 * inv) << 16) |
         (e4m3_code(v3 * inv) << 24);
}

}  // namespace moe

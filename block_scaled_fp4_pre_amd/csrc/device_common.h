// Device helpers shared by the gfx950 kernels of the W4A4 MoE layer.
//
// MXFP4 ([OCP-MX] = OCP Microscaling Formats v1.0): E2M1 codes (bit 3 sign,
// bits 2..1 exponent with bias 1, bit 0 mantissa; magnitudes 0, .5, 1, 1.5, 2,
// 3, 4, 6), one UE8M0 scale byte 2^(b-127) per 32 elements, two codes per byte
// with the even element in the low nibble.  Block scale: 2^e with e the
// smallest integer such that amax <= 6 * 2^e, clamped to [-127, 127].
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "e4m3.h"

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Scale exponent of a block from the fp32 bits of its absolute maximum.
// amax = m * 2^E with 1 <= m < 2: the smallest e with amax <= 6 * 2^e is E - 2
// when m <= 1.5 (mantissa field <= 0x400000) and E - 1 otherwise.  Zero and
// fp32 subnormals (amax < 2^-126) land on the -127 clamp.
__device__ __forceinline__ int mx_scale_exp(uint32_t amax_bits) {
  const uint32_t ef = amax_bits >> 23;
  if (ef == 0) return -127;
  int e = (int)ef - 129 + ((amax_bits & 0x7FFFFFu) > 0x400000u ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// The block scale 2^e as an fp32 value, e in [-127, 127] (2^-127 is denormal).
__device__ __forceinline__ float exp2_scale(int e) {
  return e > -127 ? __uint_as_float((uint32_t)(e + 127) << 23) : __uint_as_float(0x00400000u);
}

// E2M1 codes of v0 and v1 under block scale sc = 2^e, as one byte (v0 in the
// low nibble) written into byte SEL of old.  gfx950's v_cvt_scalef32_pk_fp4_f32
// rounds |v| / sc to the nearest E2M1 magnitude, ties to the even mantissa,
// and keeps the sign bit (so -0 and negatives that round to zero give 0x8):
// the rule above.  An exhaustive check on MI355X found no difference from the
// rule for any fp32 magnitude up to 8 * 2^e at e = -127, -126, -100, -20, -3,
// 0, 5, 20, 126, 127, both signs.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pack2(uint32_t old, float v0, float v1, float sc) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, v0, v1, sc, SEL);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// fp32 -> bfloat16 bits, round to nearest even; NaN becomes a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// One gfx950 block-scaled MFMA, FP4 x FP4 (format code 4 on both sides),
// 16x16 output, K = 128.  Lane l supplies row (l % 16) and K elements
// [32 * (l / 16), +32) of each operand as 16 bytes of packed codes, and the
// UE8M0 scale of that 32-element block in byte OA / OB of its scale register.
// Output: lane l holds C[4 * (l / 16) + i][l % 16] in element i.
template <int OA, int OB>
__device__ __forceinline__ v4f mfma_fp4(const uint4& a, const uint4& b, const v4f& c, int sa, int sb) {
  const v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const v8i bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, OA, sa, OB, sb);
}

// The same MFMA with the token operand in FP8 E4M3 (format code 0; the fp8xfp4
// MMA type).  Lane l supplies 32 bytes of token column l % 16: lo = K elements
// [16g, 16g+16) and hi = K elements [64+16g, 64+16g+16), g = l / 16 -- not the
// FP4 operand's one run [32g, 32g+32) (mapped on MI355X with a single 1.0 in
// the FP4 operand against 128 distinct FP8 codes).  The scale byte of lane l
// still belongs to the 32-element block g, as for FP4.
template <int OA, int OB>
__device__ __forceinline__ v4f mfma_fp4_fp8(const uint4& a, const uint4& blo, const uint4& bhi, const v4f& c, int sa,
                                            int sb) {
  const v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const v8i bv = {(int)blo.x, (int)blo.y, (int)blo.z, (int)blo.w, (int)bhi.x, (int)bhi.y, (int)bhi.z, (int)bhi.w};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 0, OA, sa, OB, sb);
}

}  // namespace moe

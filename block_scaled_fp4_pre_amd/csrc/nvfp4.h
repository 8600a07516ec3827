// NVFP4 on gfx950 (the MOE_MMA_NVF4_X_NVF4 type): E2M1 codes, one E4M3 scale
// byte per 16 elements, one fp32 tensor scale g per tensor; value = e2m1 *
// e4m3 * g.  [P3] prhub digest of sglang PR "bump sgl-deep-gemm to 0.1.7,
// MegaMoE uses the mma_type API for MXFP4", "Motivation", names the variant
// without defining it; the public NVFP4 format is the reading, and the
// encoding rule (moe_w4a4.h) takes every decision in fp32:
//   s    = E4M3 code nearest to min(f32(amax / f32(6 g)), 448), ties to even
//   inv  = 0 for s == 0, else f32(1 / f32(e4m3(s) * g))
//   code = E2M1 code nearest to clamp(f32(v * inv), -6, 6), ties to even.
//
// The block-scaled MFMA takes power-of-two scales per 32 elements only, and an
// E2M1 value times an E4M3 scale needs up to 6 significant bits, more than any
// of its element formats holds.  Every such product is exact in fp16 (11
// bits; 2^-10 <= |product| <= 2688), so the GEMMs turn each 16-byte FP4
// operand into fp16 products e2m1 * e4m3 and run the dense 16x16x32 fp16
// MFMA, fp32 sums; the tensor scales multiply the sums.  The conversion is
// gfx950's v_cvt_scalef32_pk_f16_fp4 with scale 1 (two exact E2M1 values per
// instruction) and a packed fp16 multiply by the block scale: the scale
// operand of the FP4 conversions contributes only its power of two (an
// in-bounds check on MI355X: with 1.875 the results were the codes times 1),
// so it cannot carry an E4M3 mantissa.
#pragma once
#include "device_common.h"
#include "e4m3.h"
#include "tiles.h"

namespace moe {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

// Weight scales in the tile order of tiles.h: per (unit, K step) 512 bytes,
// lane l's 8 at l * 8, byte 2 * rb + half = the E4M3 scale of that lane's row
// of block rb and K elements [step*128 + 32*(l/16) + 16*half, +16).
constexpr int kNvStepScaleBytes = 512;
constexpr int kNvUnitScaleStride = kGroupUnits * kNvStepScaleBytes;

__host__ __device__ inline size_t nv_w1_scale_offset(int e, int u, int s, int H, int I) {
  return unit_chunk(e, u, s, I / 32, H / kStepK) * kNvStepScaleBytes;
}
__host__ __device__ inline size_t nv_w2_scale_offset(int e, int v, int s, int H, int I) {
  return unit_chunk(e, v, s, H / kUnitRows, I / kStepK) * kNvStepScaleBytes;
}

// fp32 value of an E4M3 scale byte with the sign bit clear: exponent field 0
// is subnormal (m * 2^-9), else (1 + m/8) * 2^(field - 7).
__device__ __forceinline__ float e4m3_scale_value(uint32_t c) {
  const uint32_t ex = (c >> 3) & 15u, m = c & 7u;
  return ex ? __uint_as_float(((ex + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
}

// Scale byte of a block with absolute maximum amax under tensor scale g.
__device__ __forceinline__ uint32_t nv_scale_code(float amax, float g) {
  return e4m3_code(fminf(__fdiv_rn(amax, __fmul_rn(6.0f, g)), 448.0f));
}

// Multiplier of a block's values: 0 for a zero scale, else f32(1 / f32(e4m3(s) * g)).
__device__ __forceinline__ float nv_inv(uint32_t s, float g) {
  return s ? __fdiv_rn(1.0f, __fmul_rn(e4m3_scale_value(s), g)) : 0.0f;
}

// v * inv clamped to [-6, 6]; a zero keeps its sign.
__device__ __forceinline__ float nv_q(float v, float inv) {
  return fminf(fmaxf(__fmul_rn(v, inv), -6.0f), 6.0f);
}

// E2M1 codes of v0 and v1 (v0 in the low nibble) into byte SEL of old: the
// E2M1 conversion with scale 1 rounds to the nearest code, ties to even, sign
// kept (device_common.h).
template <int SEL>
__device__ __forceinline__ uint32_t nv_pack2(uint32_t old, float v0, float v1, float inv) {
  return e2m1_pack2<SEL>(old, nv_q(v0, inv), nv_q(v1, inv), 1.0f);
}

// An E4M3 scale byte as a pair of fp16 values (exact: 2^-9 .. 448).
__device__ __forceinline__ v2h e4m3_scale_f16x2(uint32_t c) {
  const _Float16 h = (_Float16)e4m3_scale_value(c);
  return v2h{h, h};
}

// The 8 fp16 values e2m1(code) * s of the 8 codes in dword w (byte j holds
// codes 2j and 2j+1, the even one in the low nibble); s = the block's E4M3
// value as an fp16 pair.  Every product is exact.
__device__ __forceinline__ v8h nv_operand(uint32_t w, v2h s) {
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
  return v8h{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// One dense fp16 MFMA, 16x16 output, K = 32: lane l supplies row (l % 16) and
// 8 K elements of each operand; output element i of lane l is
// C[4 * (l / 16) + i][l % 16] as for the block-scaled MFMA.  Any assignment of
// the 32 K positions to (lane group, element) serves, as long as both
// operands use the same one: a 16-byte FP4 operand (K elements [32g, 32g+32)
// of lane group g) gives four MFMAs, the i-th taking its dword i.
__device__ __forceinline__ v4f mfma_f16(const v8h& a, const v8h& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

}  // namespace moe

// MXFP4 quantization of one 32-element group (pre-dispatch, stage S1a), shared
// by the stand-alone quantize kernel and the fused pre-dispatch kernel.
// [P3] prhub digest of sglang PR "bump sgl-deep-gemm to 0.1.7, MegaMoE uses the
// mma_type API for MXFP4", "Key source snippets": pre_dispatch packs E2M1 with
// group_size=32.  Formats per [OCP-MX] (OCP MX v1.0), scale rule in
// device_common.h.
#pragma once
#include "device_common.h"
#include "nvfp4.h"

namespace moe {

// Group g of a row-major source (32 consecutive values) -> 16 bytes of packed
// E2M1 codes at codes + 16g (F8: 32 bytes of E4M3 codes at codes + 32g, the
// fp8xfp4 MMA type's activations, e4m3.h) and one scale byte at scales[g].
// 64 B (bf16) or 128 B (fp32) in as 16-byte loads.
template <bool BF16>
__device__ __forceinline__ void load_group(const void* __restrict__ src, int64_t g, float (&v)[32]) {
  if (BF16) {
    const uint4* p = reinterpret_cast<const uint4*>(src) + g * 4;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 w = p[q];
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[q * 8 + 2 * i] = bf16_to_f32(ws[i] & 0xFFFFu);
        v[q * 8 + 2 * i + 1] = bf16_to_f32(ws[i] >> 16);
      }
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(src) + g * 8;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float4 w = p[q];
      v[4 * q] = w.x; v[4 * q + 1] = w.y; v[4 * q + 2] = w.z; v[4 * q + 3] = w.w;
    }
  }
}

// MXFP4 codes of 32 values whose absolute maximum has the fp32 bits amax:
// 16 bytes, two codes per byte with the even element in the low nibble; the
// return value is the scale byte.
__device__ __forceinline__ uint32_t mx_encode_group(const float (&v)[32], uint32_t amax, uint4& codes) {
  const int e = mx_scale_exp(amax);
  const float sc = exp2_scale(e);
  uint32_t packed[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t w = e2m1_pack2<0>(0u, v[8 * q], v[8 * q + 1], sc);
    w = e2m1_pack2<1>(w, v[8 * q + 2], v[8 * q + 3], sc);
    w = e2m1_pack2<2>(w, v[8 * q + 4], v[8 * q + 5], sc);
    packed[q] = e2m1_pack2<3>(w, v[8 * q + 6], v[8 * q + 7], sc);
  }
  codes = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  return (uint32_t)(e + 127);
}

// The same for 32 bf16 values as 16 words (element 2i in the low half of
// word i), without widening them all to fp32 at once: the absolute maximum
// is taken on the bit patterns (bf16 magnitudes order as their low 15 bits),
// each value widened only for its conversion.
__device__ __forceinline__ uint32_t mx_encode_bf16_group(const uint32_t (&w)[16], uint4& codes) {
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = max(amax, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  const int e = mx_scale_exp(amax << 16);
  const float sc = exp2_scale(e);
  uint32_t packed[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t* x = w + 4 * q;
    uint32_t p = e2m1_pack2<0>(0u, bf16_to_f32(x[0] & 0xFFFFu), bf16_to_f32(x[0] >> 16), sc);
    p = e2m1_pack2<1>(p, bf16_to_f32(x[1] & 0xFFFFu), bf16_to_f32(x[1] >> 16), sc);
    p = e2m1_pack2<2>(p, bf16_to_f32(x[2] & 0xFFFFu), bf16_to_f32(x[2] >> 16), sc);
    packed[q] = e2m1_pack2<3>(p, bf16_to_f32(x[3] & 0xFFFFu), bf16_to_f32(x[3] >> 16), sc);
  }
  codes = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  return (uint32_t)(e + 127);
}

// MXFP8 E4M3 codes (e4m3.h) of 32 bf16 values as 16 words: elements 0..15
// in lo, 16..31 in hi, one byte each in element order; the return value is
// the scale byte.  The same rule and arithmetic as quantize_group's F8 branch
// (the absolute maximum on the bit patterns, as above).
__device__ __forceinline__ uint32_t mx8_encode_bf16_group(const uint32_t (&w)[16], uint4& lo, uint4& hi) {
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = max(amax, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  const int e = mx8_scale_exp(amax << 16);
  const float inv = e4m3_exp2(-e);
  uint32_t c[8];
#pragma unroll
  for (int q = 0; q < 8; ++q)
    c[q] = e4m3_pack4(bf16_to_f32(w[2 * q] & 0xFFFFu), bf16_to_f32(w[2 * q] >> 16),
                      bf16_to_f32(w[2 * q + 1] & 0xFFFFu), bf16_to_f32(w[2 * q + 1] >> 16), inv);
  lo = make_uint4(c[0], c[1], c[2], c[3]);
  hi = make_uint4(c[4], c[5], c[6], c[7]);
  return (uint32_t)(e + 127);
}

// The 16 words of group g of a bf16 row-major source.
__device__ __forceinline__ void load_bf16_words(const void* __restrict__ src, int64_t g, uint32_t (&w)[16]) {
  const uint4* p = reinterpret_cast<const uint4*>(src) + g * 4;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 v = p[q];
    w[4 * q] = v.x;
    w[4 * q + 1] = v.y;
    w[4 * q + 2] = v.z;
    w[4 * q + 3] = v.w;
  }
}

template <bool BF16, bool F8 = false>
__device__ __forceinline__ void quantize_group(const void* __restrict__ src, int64_t g,
                                               uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  if constexpr (BF16 && !F8) {
    uint32_t w[16];
    load_bf16_words(src, g, w);
    uint4 c;
    scales[g] = (uint8_t)mx_encode_bf16_group(w, c);
    reinterpret_cast<uint4*>(codes)[g] = c;
    return;
  }
  float v[32];
  load_group<BF16>(src, g, v);
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = max(amax, __float_as_uint(v[i]) & 0x7FFFFFFFu);
  if constexpr (F8) {
    const int e = mx8_scale_exp(amax);
    const float inv = e4m3_exp2(-e);
    uint32_t w[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) w[q] = e4m3_pack4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3], inv);
    uint4* out = reinterpret_cast<uint4*>(codes) + 2 * g;
    out[0] = make_uint4(w[0], w[1], w[2], w[3]);
    out[1] = make_uint4(w[4], w[5], w[6], w[7]);
    scales[g] = (uint8_t)(e + 127);
    return;
  }
  uint4 c;
  scales[g] = (uint8_t)mx_encode_group(v, amax, c);
  reinterpret_cast<uint4*>(codes)[g] = c;
}

// NVFP4 (nvfp4.h): group g of 32 values -> 16 bytes of packed E2M1 codes at
// codes + 16g and the E4M3 scale bytes of its two 16-element blocks at
// scales + 2g (the first block's in the low byte), under tensor scale gs.
template <bool BF16>
__device__ __forceinline__ void quantize_group_nv(const void* __restrict__ src, int64_t g,
                                                  uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                  float gs) {
  float v[32];
  load_group<BF16>(src, g, v);
  uint32_t packed[4];
  uint32_t sc[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[16 * b + i]));
    sc[b] = nv_scale_code(amax, gs);
    const float inv = nv_inv(sc[b], gs);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const float* p = v + 16 * b + 8 * q;
      uint32_t w = nv_pack2<0>(0u, p[0], p[1], inv);
      w = nv_pack2<1>(w, p[2], p[3], inv);
      w = nv_pack2<2>(w, p[4], p[5], inv);
      packed[2 * b + q] = nv_pack2<3>(w, p[6], p[7], inv);
    }
  }
  reinterpret_cast<uint4*>(codes)[g] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  reinterpret_cast<uint16_t*>(scales)[g] = (uint16_t)(sc[0] | (sc[1] << 8));
}

}  // namespace moe

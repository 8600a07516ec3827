// Epilogues of the NVFP4 GEMMs (gemm_nv.hip, gemm_lds_nv.hip): the tensor
// scales applied to the fp32 sums, SwiGLU and the NVFP4 requantization of h
// (GEMM1), the bf16 rounding of y (GEMM2).  Accumulator layout as in
// epilogue.h: acc[nt][rb][i] holds weight row 16*rb + 4*(lane/16) + i of the
// wave's 64-row unit against token column nt*16 + lane%16.
#pragma once
#include "epilogue.h"
#include "nvfp4.h"

namespace moe {

// GEMM1 unit u (inter columns [32u, 32u+32); blocks 0, 1 gate, 2, 3 up):
// the sums times gg, h = silu(gate) * up, NVFP4 requant of h with tensor scale
// gh per 16 columns.  Lane (kb, token) holds columns 4kb..4kb+3 of each half;
// a half's absmax is reduced over the 4 lanes of the token (xor 16, xor 32).
// Codes as for MXFP4 (plane u / 4, 64 bytes a row, epilogue.h); the two scale
// bytes of unit u go to dword plane u / 2, bytes 2 * (u % 2) and + 1.
template <int NT>
__device__ __forceinline__ void gemm1_epilogue_nv(v4f (&acc)[NT][4], int u, int row0, int nrows, int I, int hrows,
                                                  int lane, float gg, float gh, uint8_t* __restrict__ hq,
                                                  uint8_t* __restrict__ hsf, float* __restrict__ acc_out) {
  const int tok_lane = lane & 15, kb = lane >> 4;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = nt * 16 + tok_lane;
    const bool live = n < nrows;
    const int p = row0 + n;
    float gate[8], up[8], h[8];
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        gate[half * 4 + i] = __fmul_rn(acc[nt][half][i], gg);
        up[half * 4 + i] = __fmul_rn(acc[nt][2 + half][i], gg);
        h[half * 4 + i] = swiglu(gate[half * 4 + i], up[half * 4 + i]);
      }
    uint32_t sc[2], packed[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(h[half * 4 + i]));
      amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
      sc[half] = nv_scale_code(amax, gh);
      const float inv = nv_inv(sc[half], gh);
      const float* v = h + 4 * half;
      packed[half] = nv_pack2<1>(nv_pack2<0>(0u, v[0], v[1], inv), v[2], v[3], inv);
    }
    if (live) {
      uint8_t* row = hq + ((size_t)(u >> 2) * hrows + p) * 64 + (u & 3) * 16;
      *reinterpret_cast<uint16_t*>(row + 2 * kb) = (uint16_t)packed[0];
      *reinterpret_cast<uint16_t*>(row + 8 + 2 * kb) = (uint16_t)packed[1];
      if (kb == 0)
        *reinterpret_cast<uint16_t*>(hsf + ((size_t)(u >> 1) * hrows + p) * 4 + (u & 1) * 2) =
            (uint16_t)(sc[0] | (sc[1] << 8));
      if (acc_out != nullptr) {
        float* arow = acc_out + (size_t)p * (2 * I) + 32 * u + 4 * kb;
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            arow[16 * half + i] = gate[half * 4 + i];
            arow[I + 16 * half + i] = up[half * 4 + i];
          }
      }
    }
  }
}

// GEMM2 unit v (hidden rows [64v, 64v+64)): y rows = bf16(sum * g2).
template <int NT>
__device__ __forceinline__ void gemm2_epilogue_nv(const v4f (&acc)[NT][4], int v, int row0, int nrows, int H,
                                                  int lane, float g2, uint16_t* __restrict__ y) {
  const int tok_lane = lane & 15, kb = lane >> 4;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = nt * 16 + tok_lane;
    if (n < nrows) {
      uint16_t* yrow = y + (size_t)(row0 + n) * H + 64 * v + 4 * kb;
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
        *reinterpret_cast<uint2*>(yrow + 16 * rb) =
            make_uint2(f32_to_bf16(__fmul_rn(acc[nt][rb][0], g2)) | (f32_to_bf16(__fmul_rn(acc[nt][rb][1], g2)) << 16),
                       f32_to_bf16(__fmul_rn(acc[nt][rb][2], g2)) | (f32_to_bf16(__fmul_rn(acc[nt][rb][3], g2)) << 16));
    }
  }
}

}  // namespace moe

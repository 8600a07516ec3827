// Epilogues of the two grouped GEMMs, shared by the streaming kernels
// (gemm1.hip, gemm2.hip) and the LDS-staged prefill kernels (gemm_lds.hip).
//
// Accumulator layout (16x16x128 MFMA, swap-AB): acc[nt][rb][i] holds weight row
// 16*rb + 4*(lane/16) + i of the wave's 64-row unit against token column
// nt*16 + lane%16 of the tile.
#pragma once
#include "device_common.h"

namespace moe {

// Store policies of the epilogues.  PlainStore: ordinary stores, made visible
// to other workgroups by the kernel's end.  CoherentStore: agent-scope stores
// (the sc1 policy on gfx950), visible to the agent-scope loads of any
// workgroup on the device once they complete, for results that another
// workgroup of the same launch reads (mega.hip).
struct PlainStore {
  template <class T>
  __device__ static void put(T* p, T v) { *p = v; }
};
struct CoherentStore {
  template <class T>
  __device__ static void put(T* p, T v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
};

// SwiGLU in fp32: silu(g) * u, silu(g) = g / (1 + e^-g).  e^-g is the hardware
// 2^x of -g * log2(e) and the quotient goes through the hardware reciprocal:
// a few ulp from the correctly rounded value, against ~20 instructions per
// element for a correctly rounded expf and division.  Very negative g gives
// e^-g = inf and h = -0 * u, the limit's sign.
__device__ __forceinline__ float swiglu(float g, float u) {
  const float t = __builtin_amdgcn_exp2f(-g * 1.44269504088896341f);
  return g * __builtin_amdgcn_rcpf(1.0f + t) * u;
}

// GEMM1 unit u (inter columns [32u, 32u+32)): blocks 0,1 are gate, 2,3 up.
// h = silu(gate) * up in fp32, requantized to MXFP4 per 32 columns: the absmax
// over the 4 lanes of a token (xor 16, xor 32), then codes packed two per byte
// (even column in the low nibble).  row0: sorted position of token column 0.
//
// F8 (the fp8xfp4 MMA type): h is requantized to E4M3 instead (e4m3.h), one
// byte per column.
//
// hq and hsf are K-step planes for GEMM2: plane c (inter columns [128c,
// 128c+128)) holds, for every sorted row p, its PB = 64 (E4M3: 128) code
// bytes at (c * hrows + p) * PB and its 4 scale bytes at (c * hrows + p) * 4,
// hrows being the rows of a plane.  A tile of consecutive rows then reads one
// contiguous run per K step.  Unit u is PB / 4 code bytes and scale byte u % 4
// of plane u / 4.
template <int NT, bool F8 = false, class St = PlainStore>
__device__ __forceinline__ void gemm1_epilogue(v4f (&acc)[NT][4], int u, int row0, int nrows, int I, int hrows,
                                               int lane, uint8_t* __restrict__ hq, uint8_t* __restrict__ hsf,
                                               float* __restrict__ acc_out) {
  const int tok_lane = lane & 15, kb = lane >> 4;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = nt * 16 + tok_lane;
    const bool live = n < nrows;
    const int p = row0 + n;
    float h[8];
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float gt = acc[nt][half][i], up = acc[nt][2 + half][i];
        h[half * 4 + i] = swiglu(gt, up);
      }
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = max(amax, __float_as_uint(h[i]) & 0x7FFFFFFFu);
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 16, 64));
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 32, 64));
    const int ex = F8 ? mx8_scale_exp(amax) : mx_scale_exp(amax);
    if (live) {
      const size_t pr = (size_t)(u >> 2) * hrows + p;   // row p of plane u / 4
      if constexpr (F8) {
        // columns 4kb..4kb+3 and 16+4kb..16+4kb+3 of the unit's 32 bytes
        const float inv = e4m3_exp2(-ex);
        uint8_t* row = hq + pr * 128 + (u & 3) * 32;
        St::put(reinterpret_cast<uint32_t*>(row + 4 * kb), e4m3_pack4(h[0], h[1], h[2], h[3], inv));
        St::put(reinterpret_cast<uint32_t*>(row + 16 + 4 * kb), e4m3_pack4(h[4], h[5], h[6], h[7], inv));
      } else {
        const float sc = exp2_scale(ex);
        const uint32_t lo = e2m1_pack2<1>(e2m1_pack2<0>(0u, h[0], h[1], sc), h[2], h[3], sc);
        const uint32_t hi = e2m1_pack2<1>(e2m1_pack2<0>(0u, h[4], h[5], sc), h[6], h[7], sc);
        uint8_t* row = hq + pr * 64 + (u & 3) * 16;
        St::put(reinterpret_cast<uint16_t*>(row + 2 * kb), (uint16_t)lo);
        St::put(reinterpret_cast<uint16_t*>(row + 8 + 2 * kb), (uint16_t)hi);
      }
      if (kb == 0) St::put(hsf + pr * 4 + (u & 3), (uint8_t)(ex + 127));
      if (acc_out != nullptr) {
        float* arow = acc_out + (size_t)p * (2 * I) + 32 * u + 4 * kb;
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            arow[16 * half + i] = acc[nt][half][i];
            arow[I + 16 * half + i] = acc[nt][2 + half][i];
          }
      }
    }
  }
}

// GEMM2 unit v (hidden rows [64v, 64v+64)): y rows in sorted order, the fp32
// accumulators rounded to bfloat16 (nearest even) -- half the bytes of the
// y round trip to the combine.
template <int NT, class St = PlainStore>
__device__ __forceinline__ void gemm2_epilogue(const v4f (&acc)[NT][4], int v, int row0, int nrows, int H,
                                               int lane, uint16_t* __restrict__ y) {
  const int tok_lane = lane & 15, kb = lane >> 4;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = nt * 16 + tok_lane;
    if (n < nrows) {
      uint16_t* yrow = y + (size_t)(row0 + n) * H + 64 * v + 4 * kb;
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
        St::put(reinterpret_cast<uint64_t*>(yrow + 16 * rb),
                (uint64_t)(f32_to_bf16(acc[nt][rb][0]) | (f32_to_bf16(acc[nt][rb][1]) << 16)) |
                    ((uint64_t)(f32_to_bf16(acc[nt][rb][2]) | (f32_to_bf16(acc[nt][rb][3]) << 16)) << 32));
    }
  }
}

template <int NT>
__device__ __forceinline__ void zero_acc(v4f (&acc)[NT][4]) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) acc[nt][rb] = v4f{0.f, 0.f, 0.f, 0.f};
}

}  // namespace moe

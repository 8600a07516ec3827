// Stage S0: canonical MXFP4 (or NVFP4) expert weights -> the device tile order
// of tiles.h (NVFP4 scales: nvfp4.h).
// A pure byte permutation, run once per weight set ([P3] prhub digest of sglang
// PR "bump sgl-deep-gemm to 0.1.7, MegaMoE uses the mma_type API for MXFP4",
// "Implementation breakdown" item 4: the weights are transformed at load time
// for the chosen mma_type).  Canonical input: W1 [E, 2I, H/2] codes with rows
// [0, I) gate and [I, 2I) up, W1 scales [E, 2I, H/32]; W2 [E, H, I/2] codes,
// W2 scales [E, H, I/32].
#include "device_common.h"
#include "launch.h"
#include "nvfp4.h"
#include "tiles.h"

namespace moe {

// Canonical W1 row of block rb (0..3) of GEMM1 unit u, row-in-block i.
__device__ __forceinline__ int w1_row(int u, int rb, int i, int I) {
  return (rb < 2 ? 0 : I) + 32 * u + 16 * (rb & 1) + i;
}

// One thread per 16-byte code chunk of the output (lane l of block rb of a step).
__global__ void __launch_bounds__(256) prepare_w1_codes(const uint8_t* __restrict__ src, int H, int I,
                                                         int64_t nchunks, uint8_t* __restrict__ dst) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= nchunks) return;
  const int S = H / kStepK, U = I / 32;
  const int lane = (int)(q & 63);
  const int64_t r1 = q >> 6;
  const int rb = (int)(r1 & 3);
  const int64_t r2 = r1 >> 2;                 // chunk index (tiles.h unit_chunk)
  const int u_lo = (int)(r2 % kGroupUnits);
  const int64_t r3 = r2 / kGroupUnits;
  const int s = (int)(r3 % S);
  const int64_t r4 = r3 / S;
  const int u = (int)(r4 % (U / kGroupUnits)) * kGroupUnits + u_lo;
  const int e = (int)(r4 / (U / kGroupUnits));
  const int row = w1_row(u, rb, lane & 15, I);
  const uint8_t* p = src + ((size_t)e * 2 * I + row) * (H / 2) + s * 64 + (lane >> 4) * 16;
  reinterpret_cast<uint4*>(dst)[q] = *reinterpret_cast<const uint4*>(p);
}

// One thread per lane dword of a step: byte rb = scale of block rb's row.
__global__ void __launch_bounds__(256) prepare_w1_scales(const uint8_t* __restrict__ src, int H, int I,
                                                          int64_t ndwords, uint8_t* __restrict__ dst) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= ndwords) return;
  const int S = H / kStepK, U = I / 32;
  const int lane = (int)(q & 63);
  const int64_t r2 = q >> 6;                  // chunk index (tiles.h unit_chunk)
  const int u_lo = (int)(r2 % kGroupUnits);
  const int64_t r3 = r2 / kGroupUnits;
  const int s = (int)(r3 % S);
  const int64_t r4 = r3 / S;
  const int u = (int)(r4 % (U / kGroupUnits)) * kGroupUnits + u_lo;
  const int e = (int)(r4 / (U / kGroupUnits));
  uint32_t word = 0;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int row = w1_row(u, rb, lane & 15, I);
    word |= (uint32_t)src[((size_t)e * 2 * I + row) * (H / 32) + s * 4 + (lane >> 4)] << (8 * rb);
  }
  reinterpret_cast<uint32_t*>(dst)[q] = word;
}

__global__ void __launch_bounds__(256) prepare_w2_codes(const uint8_t* __restrict__ src, int H, int I,
                                                         int64_t nchunks, uint8_t* __restrict__ dst) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= nchunks) return;
  const int S = I / kStepK, U = H / kUnitRows;
  const int lane = (int)(q & 63);
  const int64_t r1 = q >> 6;
  const int rb = (int)(r1 & 3);
  const int64_t r2 = r1 >> 2;                 // chunk index (tiles.h unit_chunk)
  const int v_lo = (int)(r2 % kGroupUnits);
  const int64_t r3 = r2 / kGroupUnits;
  const int s = (int)(r3 % S);
  const int64_t r4 = r3 / S;
  const int v = (int)(r4 % (U / kGroupUnits)) * kGroupUnits + v_lo;
  const int e = (int)(r4 / (U / kGroupUnits));
  const int row = kUnitRows * v + 16 * rb + (lane & 15);
  const uint8_t* p = src + ((size_t)e * H + row) * (I / 2) + s * 64 + (lane >> 4) * 16;
  reinterpret_cast<uint4*>(dst)[q] = *reinterpret_cast<const uint4*>(p);
}

__global__ void __launch_bounds__(256) prepare_w2_scales(const uint8_t* __restrict__ src, int H, int I,
                                                          int64_t ndwords, uint8_t* __restrict__ dst) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= ndwords) return;
  const int S = I / kStepK, U = H / kUnitRows;
  const int lane = (int)(q & 63);
  const int64_t r2 = q >> 6;                  // chunk index (tiles.h unit_chunk)
  const int v_lo = (int)(r2 % kGroupUnits);
  const int64_t r3 = r2 / kGroupUnits;
  const int s = (int)(r3 % S);
  const int64_t r4 = r3 / S;
  const int v = (int)(r4 % (U / kGroupUnits)) * kGroupUnits + v_lo;
  const int e = (int)(r4 / (U / kGroupUnits));
  uint32_t word = 0;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int row = kUnitRows * v + 16 * rb + (lane & 15);
    word |= (uint32_t)src[((size_t)e * H + row) * (I / 32) + s * 4 + (lane >> 4)] << (8 * rb);
  }
  reinterpret_cast<uint32_t*>(dst)[q] = word;
}

// NVFP4 scales (nvfp4.h): one thread per lane's 8 bytes of a step, byte
// 2*rb + half = the E4M3 scale of block rb's row and the lane's 16-element
// half; canonical scales are one byte per 16 elements of a row.
__global__ void __launch_bounds__(256) prepare_w1_scales_nv(const uint8_t* __restrict__ src, int H, int I,
                                                             int64_t nwords, uint8_t* __restrict__ dst) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= nwords) return;
  const int S = H / kStepK, U = I / 32;
  const int lane = (int)(q & 63);
  const int64_t r2 = q >> 6;                  // chunk index (tiles.h unit_chunk)
  const int u_lo = (int)(r2 % kGroupUnits);
  const int64_t r3 = r2 / kGroupUnits;
  const int s = (int)(r3 % S);
  const int64_t r4 = r3 / S;
  const int u = (int)(r4 % (U / kGroupUnits)) * kGroupUnits + u_lo;
  const int e = (int)(r4 / (U / kGroupUnits));
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int row = w1_row(u, rb, lane & 15, I);
    const uint8_t* p = src + ((size_t)e * 2 * I + row) * (H / 16) + s * 8 + (lane >> 4) * 2;
    w[rb >> 1] |= ((uint32_t)p[0] | ((uint32_t)p[1] << 8)) << (16 * (rb & 1));
  }
  reinterpret_cast<uint2*>(dst)[q] = make_uint2(w[0], w[1]);
}

__global__ void __launch_bounds__(256) prepare_w2_scales_nv(const uint8_t* __restrict__ src, int H, int I,
                                                             int64_t nwords, uint8_t* __restrict__ dst) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= nwords) return;
  const int S = I / kStepK, U = H / kUnitRows;
  const int lane = (int)(q & 63);
  const int64_t r2 = q >> 6;                  // chunk index (tiles.h unit_chunk)
  const int v_lo = (int)(r2 % kGroupUnits);
  const int64_t r3 = r2 / kGroupUnits;
  const int s = (int)(r3 % S);
  const int64_t r4 = r3 / S;
  const int v = (int)(r4 % (U / kGroupUnits)) * kGroupUnits + v_lo;
  const int e = (int)(r4 / (U / kGroupUnits));
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int row = kUnitRows * v + 16 * rb + (lane & 15);
    const uint8_t* p = src + ((size_t)e * H + row) * (I / 16) + s * 8 + (lane >> 4) * 2;
    w[rb >> 1] |= ((uint32_t)p[0] | ((uint32_t)p[1] << 8)) << (16 * (rb & 1));
  }
  reinterpret_cast<uint2*>(dst)[q] = make_uint2(w[0], w[1]);
}

// gsc = [g_w1[E], g_w2[E], g_x, g_h]
__global__ void __launch_bounds__(256) prepare_tensor_scales_nv(const float* __restrict__ gw1,
                                                                 const float* __restrict__ gw2, float gx, float gh,
                                                                 int E, float* __restrict__ gsc) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < E) {
    gsc[i] = gw1[i];
    gsc[E + i] = gw2[i];
  }
  if (i == 0) {
    gsc[2 * E] = gx;
    gsc[2 * E + 1] = gh;
  }
}

hipError_t launch_prepare_nv(const uint8_t* w1c, const uint8_t* w1s, const float* gw1, const uint8_t* w2c,
                             const uint8_t* w2s, const float* gw2, float gx, float gh, int H, int I, int E,
                             uint8_t* p_w1c, uint8_t* p_w1s, uint8_t* p_w2c, uint8_t* p_w2s, float* gsc,
                             hipStream_t stream) {
  const int64_t steps1 = (int64_t)E * (I / 32) * (H / kStepK);
  const int64_t steps2 = (int64_t)E * (H / kUnitRows) * (I / kStepK);
  struct Job { int64_t n; int which; };
  const Job jobs[4] = {{steps1 * 256, 0}, {steps1 * 64, 1}, {steps2 * 256, 2}, {steps2 * 64, 3}};
  for (const Job& j : jobs) {
    if (j.n == 0) continue;
    const dim3 grid((unsigned)((j.n + 255) / 256));
    switch (j.which) {
      case 0: hipLaunchKernelGGL(prepare_w1_codes, grid, dim3(256), 0, stream, w1c, H, I, j.n, p_w1c); break;
      case 1: hipLaunchKernelGGL(prepare_w1_scales_nv, grid, dim3(256), 0, stream, w1s, H, I, j.n, p_w1s); break;
      case 2: hipLaunchKernelGGL(prepare_w2_codes, grid, dim3(256), 0, stream, w2c, H, I, j.n, p_w2c); break;
      default: hipLaunchKernelGGL(prepare_w2_scales_nv, grid, dim3(256), 0, stream, w2s, H, I, j.n, p_w2s); break;
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(prepare_tensor_scales_nv, dim3((E + 255) / 256), dim3(256), 0, stream, gw1, gw2, gx, gh, E, gsc);
  return hipGetLastError();
}

hipError_t launch_prepare(const uint8_t* w1c, const uint8_t* w1s, const uint8_t* w2c, const uint8_t* w2s,
                          int H, int I, int E, uint8_t* p_w1c, uint8_t* p_w1s, uint8_t* p_w2c,
                          uint8_t* p_w2s, hipStream_t stream) {
  // W1: E * (I/32) units * (H/128) steps; W2: E * (H/64) units * (I/128) steps.
  const int64_t steps1 = (int64_t)E * (I / 32) * (H / kStepK);
  const int64_t steps2 = (int64_t)E * (H / kUnitRows) * (I / kStepK);
  struct Job { int64_t n; int which; };
  const Job jobs[4] = {{steps1 * 256, 0}, {steps1 * 64, 1}, {steps2 * 256, 2}, {steps2 * 64, 3}};
  for (const Job& j : jobs) {
    if (j.n == 0) continue;
    const dim3 grid((unsigned)((j.n + 255) / 256));
    switch (j.which) {
      case 0: hipLaunchKernelGGL(prepare_w1_codes, grid, dim3(256), 0, stream, w1c, H, I, j.n, p_w1c); break;
      case 1: hipLaunchKernelGGL(prepare_w1_scales, grid, dim3(256), 0, stream, w1s, H, I, j.n, p_w1s); break;
      case 2: hipLaunchKernelGGL(prepare_w2_codes, grid, dim3(256), 0, stream, w2c, H, I, j.n, p_w2c); break;
      default: hipLaunchKernelGGL(prepare_w2_scales, grid, dim3(256), 0, stream, w2s, H, I, j.n, p_w2s); break;
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace moe

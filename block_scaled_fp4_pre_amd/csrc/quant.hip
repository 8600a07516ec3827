// Stage S1a (pre-dispatch quantization): every 32-element group of a row becomes
// 16 bytes of packed E2M1 codes and one UE8M0 scale byte.
// [P3] prhub digest of sglang PR "bump sgl-deep-gemm to 0.1.7, MegaMoE uses the
// mma_type API for MXFP4", "Key source snippets": the mxf4xmxf4 pre_dispatch
// packs E2M1 with group_size=32.  Formats per [OCP-MX] (OCP MX v1.0).
//
// One thread per group: 64 B (bf16) or 128 B (fp32) in as 16-byte loads, 16 B
// + 1 B out; consecutive threads touch consecutive groups, so loads and stores
// coalesce.  Purely HBM-bound.
#include "device_common.h"
#include "launch.h"

namespace moe {

template <bool BF16>
__global__ void __launch_bounds__(256) quantize_kernel(const void* __restrict__ src, int64_t ngroups,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= ngroups) return;
  float v[32];
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
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = max(amax, __float_as_uint(v[i]) & 0x7FFFFFFFu);
  const int e = mx_scale_exp(amax);
  uint32_t packed[4] = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 32; ++i) packed[i >> 3] |= e2m1_code(v[i], e) << (4 * (i & 7));
  reinterpret_cast<uint4*>(codes)[g] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  scales[g] = (uint8_t)(e + 127);
}

hipError_t launch_quantize(bool src_is_bf16, const void* src, int64_t ngroups, uint8_t* codes,
                           uint8_t* scales, hipStream_t stream) {
  if (ngroups <= 0) return hipSuccess;
  const dim3 grid((unsigned)((ngroups + 255) / 256));
  if (src_is_bf16)
    hipLaunchKernelGGL(quantize_kernel<true>, grid, dim3(256), 0, stream, src, ngroups, codes, scales);
  else
    hipLaunchKernelGGL(quantize_kernel<false>, grid, dim3(256), 0, stream, src, ngroups, codes, scales);
  return hipGetLastError();
}

}  // namespace moe

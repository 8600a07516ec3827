// Stage S1a (pre-dispatch quantization): every 32-element group of a row becomes
// 16 bytes of packed E2M1 codes (the fp8xfp4 MMA type: 32 bytes of E4M3 codes)
// and one UE8M0 scale byte (NVFP4: 16 bytes of E2M1 codes and two E4M3 scale
// bytes under a tensor scale, nvfp4.h).
// [P3] prhub digest of sglang PR "bump sgl-deep-gemm to 0.1.7, MegaMoE uses the
// mma_type API for MXFP4", "Key source snippets": the mxf4xmxf4 pre_dispatch
// packs E2M1 with group_size=32.  Formats per [OCP-MX] (OCP MX v1.0).
//
// One thread per group: 64 B (bf16) or 128 B (fp32) in as 16-byte loads, 16 B
// + 1 B out; consecutive threads touch consecutive groups, so loads and stores
// coalesce.  Purely HBM-bound.
#include "launch.h"
#include "quant_group.h"

namespace moe {

template <bool BF16, bool F8>
__global__ void __launch_bounds__(256) quantize_kernel(const void* __restrict__ src, int64_t ngroups,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g < ngroups) quantize_group<BF16, F8>(src, g, codes, scales);
}

// Tensor scale: *gsp when gsp is not null (the prepared g_x of a forward),
// else gs.
template <bool BF16>
__global__ void __launch_bounds__(256) quantize_nv_kernel(const void* __restrict__ src, int64_t ngroups, float gs,
                                                          const float* __restrict__ gsp, uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g < ngroups) quantize_group_nv<BF16>(src, g, codes, scales, gsp != nullptr ? *gsp : gs);
}

hipError_t launch_quantize_nv(bool src_is_bf16, const void* src, int64_t ngroups, float gs, const float* gsp,
                              uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  if (ngroups <= 0) return hipSuccess;
  const dim3 grid((unsigned)((ngroups + 255) / 256));
  auto kern = src_is_bf16 ? quantize_nv_kernel<true> : quantize_nv_kernel<false>;
  hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, src, ngroups, gs, gsp, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quantize(bool src_is_bf16, bool fp8, const void* src, int64_t ngroups, uint8_t* codes,
                           uint8_t* scales, hipStream_t stream) {
  if (ngroups <= 0) return hipSuccess;
  const dim3 grid((unsigned)((ngroups + 255) / 256));
  if (fp8 && src_is_bf16)
    hipLaunchKernelGGL((quantize_kernel<true, true>), grid, dim3(256), 0, stream, src, ngroups, codes, scales);
  else if (fp8)
    return hipErrorInvalidValue;                // E4M3 is an activation format: bf16 input only
  else if (src_is_bf16)
    hipLaunchKernelGGL((quantize_kernel<true, false>), grid, dim3(256), 0, stream, src, ngroups, codes, scales);
  else
    hipLaunchKernelGGL((quantize_kernel<false, false>), grid, dim3(256), 0, stream, src, ngroups, codes, scales);
  return hipGetLastError();
}

}  // namespace moe

// Stage S4: top-k weighted combine.  out[t] = sum over valid slots j, in slot
// order, of w[t, j] * y[pos[t*k + j]] (y in bfloat16 from GEMM2), accumulated
// in fp32 from +0 and rounded once to bfloat16 (round to nearest even).  Slots with pos == -1 (ids outside
// [0, E)) are skipped; a token with none gives +0.
// The weighted sum back to token order is the last stage of the fused layer that
// [P1] sglang PR "[deepseek-v4] Bump sgl-deep-gemm for packed FP4xFP4 mega-MoE
// (W4A4)" measures as one kernel (Appendix, section B); the pages do not print
// it, this is the plain reading.
//
// One workgroup per token; each thread owns 8 consecutive columns (one 16-byte
// load of y per slot, one 16-byte store).  Purely HBM-bound.
#include "device_common.h"
#include "launch.h"

namespace moe {

__global__ void __launch_bounds__(256) combine_kernel(const uint16_t* __restrict__ y,
                                                      const int32_t* __restrict__ pos,
                                                      const float* __restrict__ w, int H, int k,
                                                      uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  for (int c = threadIdx.x; c < H / 8; c += 256) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    for (int j = 0; j < k; ++j) {
      const int p = pos[(size_t)t * k + j];
      if (p < 0) continue;
      const float wj = w[(size_t)t * k + j];
      const uint4 v = reinterpret_cast<const uint4*>(y + (size_t)p * H)[c];
      const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += wj * bf16_to_f32(vv[i] & 0xFFFFu);
        acc[2 * i + 1] += wj * bf16_to_f32(vv[i] >> 16);
      }
    }
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = f32_to_bf16(acc[2 * i]) | (f32_to_bf16(acc[2 * i + 1]) << 16);
    reinterpret_cast<uint4*>(out + (size_t)t * H)[c] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

hipError_t launch_combine(const uint16_t* y, const int32_t* pos, const float* w, int T, int H, int k,
                          uint16_t* out, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3(T), dim3(256), 0, stream, y, pos, w, H, k, out);
  return hipGetLastError();
}

}  // namespace moe

// Stage S4: top-k weighted combine.  out[t] = sum over valid slots j, in slot
// order, of w[t, j] * y[pos[t*k + j]] (y in bfloat16 from GEMM2), accumulated
// in fp32 from +0 and rounded once to bfloat16 (round to nearest even).  Slots
// with pos == -1 (ids outside [0, E)) are skipped; a token with none gives +0.
// The weighted sum back to token order is the last stage of the fused layer that
// [P1] sglang PR "[deepseek-v4] Bump sgl-deep-gemm for packed FP4xFP4 mega-MoE
// (W4A4)" measures as one kernel (Appendix, section B); the pages do not print
// it, this is the plain reading.
//
// One workgroup per token; each thread owns CPT pieces of 8 consecutive
// columns.  The slots' 16-byte loads of y (read once: non-temporal) are all
// issued before the first one is used, in batches of up to 8 slots, so each
// thread keeps up to 8*CPT loads in flight; the sum still runs in slot order.
// Purely HBM-bound.
#include "device_common.h"
#include "launch.h"

namespace moe {

constexpr int kCombineThreads = 256;
constexpr int kCombineBatch = 8;   // slots whose loads are in flight together

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_stream16(const uint16_t* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int CPT>
__global__ void __launch_bounds__(kCombineThreads) combine_kernel(const uint16_t* __restrict__ y,
                                                                  const int32_t* __restrict__ pos,
                                                                  const float* __restrict__ w, int H, int k,
                                                                  uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  const int pieces = H / 8;
  for (int c0 = threadIdx.x; c0 < pieces; c0 += kCombineThreads * CPT) {
    float acc[CPT][8];
#pragma unroll
    for (int q = 0; q < CPT; ++q)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[q][i] = 0.f;
    for (int j0 = 0; j0 < k; j0 += kCombineBatch) {
      uint4 v[kCombineBatch][CPT];
      float wj[kCombineBatch];
      bool use[kCombineBatch];
#pragma unroll
      for (int b = 0; b < kCombineBatch; ++b) {
        const int j = j0 + b;
        const int p = j < k ? pos[(size_t)t * k + j] : -1;   // token-uniform: scalar loads
        use[b] = p >= 0;
        wj[b] = use[b] ? w[(size_t)t * k + j] : 0.f;
        const uint16_t* row = y + (size_t)(use[b] ? p : 0) * H;
#pragma unroll
        for (int q = 0; q < CPT; ++q) {
          const int c = c0 + q * kCombineThreads;
          v[b][q] = (use[b] && c < pieces) ? load_stream16(row + 8 * c) : make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int b = 0; b < kCombineBatch; ++b) {
        if (!use[b]) continue;
#pragma unroll
        for (int q = 0; q < CPT; ++q) {
          const uint32_t vv[4] = {v[b][q].x, v[b][q].y, v[b][q].z, v[b][q].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[q][2 * i] += wj[b] * bf16_to_f32(vv[i] & 0xFFFFu);
            acc[q][2 * i + 1] += wj[b] * bf16_to_f32(vv[i] >> 16);
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int c = c0 + q * kCombineThreads;
      if (c >= pieces) continue;
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = f32_to_bf16(acc[q][2 * i]) | (f32_to_bf16(acc[q][2 * i + 1]) << 16);
      reinterpret_cast<uint4*>(out + (size_t)t * H)[c] = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

hipError_t launch_combine(const uint16_t* y, const int32_t* pos, const float* w, int T, int H, int k,
                          uint16_t* out, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  // Two pieces per thread once a row has at least 512 of them (H >= 4096).
  if (H / 8 >= 2 * kCombineThreads)
    hipLaunchKernelGGL(combine_kernel<2>, dim3(T), dim3(kCombineThreads), 0, stream, y, pos, w, H, k, out);
  else
    hipLaunchKernelGGL(combine_kernel<1>, dim3(T), dim3(kCombineThreads), 0, stream, y, pos, w, H, k, out);
  return hipGetLastError();
}

}  // namespace moe

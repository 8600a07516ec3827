// Stage S3: per-expert GEMM2 (down projection) y = h_hat . W2_hat[e]^T with fp32
// accumulation on the gfx950 block-scaled FP4 MFMA; y is written per routed row
// in expert-sorted order for the combine.
//
// [P1] sglang PR "[deepseek-v4] Bump sgl-deep-gemm for packed FP4xFP4 mega-MoE
// (W4A4)": title (packed FP4 x FP4) and section B "NCU Speed-of-Light" (the
// weight stream bounds the layer at ntok=512).
//
// Grid: one workgroup of 4 waves per (expert, 256 hidden rows); wave w owns the
// unit of 64 hidden rows v = 4g + w.  The expert's requantized rows are
// already contiguous (sorted order), so the B tile is a plain copy into LDS.
// Weights stream HBM -> VGPR with a D-step register prefetch ring as in GEMM1.
#include "device_common.h"
#include "launch.h"
#include "tiles.h"

namespace moe {

template <int NT, int D>
__global__ void __launch_bounds__(256) gemm2_kernel(
    const uint8_t* __restrict__ w2c, const uint8_t* __restrict__ w2s, const uint8_t* __restrict__ hq,
    const uint8_t* __restrict__ hsf, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, int H, int I, float* __restrict__ y) {
  const int groups = H / 256;
  const int e = blockIdx.x / groups;
  const int g = blockIdx.x - e * groups;
  const int n_e = counts[e];
  if (n_e == 0) return;
  const int base = offsets[e];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int v = g * 4 + wave;
  const int S = I / kStepK;
  const int row_bytes = I / 2, row_stride = I / 2 + 16, sc_row = I / 32;

  extern __shared__ __align__(16) uint8_t lds[];
  uint8_t* lds_codes = lds;
  uint8_t* lds_scales = lds + NT * 16 * row_stride;

  const uint4* wc = reinterpret_cast<const uint4*>(w2c + w2_code_offset(e, v, 0, H, I)) + lane;
  const uint32_t* ws = reinterpret_cast<const uint32_t*>(w2s + w2_scale_offset(e, v, 0, H, I)) + lane;
  const int tok_lane = lane & 15, kb = lane >> 4;

  for (int t0 = 0; t0 < n_e; t0 += NT * 16) {
    uint4 a[D][4];
    uint32_t sa[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (d < S) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) a[d][rb] = wc[(d * 4 + rb) * 64];
        sa[d] = ws[d * 64];
      }
    }
    const int nrows = min(NT * 16, n_e - t0);
    __syncthreads();
    const int chunks = row_bytes / 16;
    for (int idx = threadIdx.x; idx < NT * 16 * chunks; idx += 256) {
      const int n = idx / chunks, c = idx - n * chunks;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (n < nrows) val = reinterpret_cast<const uint4*>(hq + (size_t)(base + t0 + n) * row_bytes)[c];
      *reinterpret_cast<uint4*>(lds_codes + n * row_stride + c * 16) = val;
    }
    for (int idx = threadIdx.x; idx < NT * 16 * sc_row; idx += 256) {
      const int n = idx / sc_row, c = idx - n * sc_row;
      lds_scales[n * sc_row + c] = n < nrows ? hsf[(size_t)(base + t0 + n) * sc_row + c] : (uint8_t)0;
    }
    __syncthreads();

    v4f acc[NT][4];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) acc[nt][rb] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int s0 = 0; s0 < S; s0 += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const int s = s0 + d;
        if (s < S) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const int n = nt * 16 + tok_lane;
            const uint4 b = *reinterpret_cast<const uint4*>(lds_codes + n * row_stride + s * 64 + kb * 16);
            const int sb = lds_scales[n * sc_row + s * 4 + kb];
            acc[nt][0] = mfma_fp4<0, 0>(a[d][0], b, acc[nt][0], (int)sa[d], sb);
            acc[nt][1] = mfma_fp4<1, 0>(a[d][1], b, acc[nt][1], (int)sa[d], sb);
            acc[nt][2] = mfma_fp4<2, 0>(a[d][2], b, acc[nt][2], (int)sa[d], sb);
            acc[nt][3] = mfma_fp4<3, 0>(a[d][3], b, acc[nt][3], (int)sa[d], sb);
          }
          const int sn = s + D;
          if (sn < S) {
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) a[d][rb] = wc[(sn * 4 + rb) * 64];
            sa[d] = ws[sn * 64];
          }
        }
      }
    }

    // acc[nt][rb][i] = y[row t0 + nt*16 + tok_lane][64v + 16rb + 4kb + i]
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = nt * 16 + tok_lane;
      if (n < nrows) {
        float* yrow = y + (size_t)(base + t0 + n) * H + 64 * v + 4 * kb;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
          *reinterpret_cast<float4*>(yrow + 16 * rb) =
              make_float4(acc[nt][rb][0], acc[nt][rb][1], acc[nt][rb][2], acc[nt][rb][3]);
      }
    }
  }
}

template <int NT, int D>
static hipError_t launch_gemm2_t(const uint8_t* w2c, const uint8_t* w2s, const uint8_t* hq,
                                 const uint8_t* hsf, const int32_t* counts, const int32_t* offsets,
                                 int H, int I, int E, float* y, hipStream_t stream) {
  const size_t lds = (size_t)NT * 16 * (I / 2 + 16) + (size_t)NT * 16 * (I / 32);
  auto kern = gemm2_kernel<NT, D>;
  if (lds > 65536) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(kern, dim3(E * (H / 256)), dim3(256), lds, stream, w2c, w2s, hq, hsf, counts,
                     offsets, H, I, y);
  return hipGetLastError();
}

hipError_t launch_gemm2(const uint8_t* w2c, const uint8_t* w2s, const uint8_t* hq, const uint8_t* hsf,
                        const int32_t* counts, const int32_t* offsets, int H, int I, int E,
                        int rows_hint, float* y, hipStream_t stream) {
  if (rows_hint > 8) return launch_gemm2_t<2, 8>(w2c, w2s, hq, hsf, counts, offsets, H, I, E, y, stream);
  return launch_gemm2_t<1, 8>(w2c, w2s, hq, hsf, counts, offsets, H, I, E, y, stream);
}

}  // namespace moe

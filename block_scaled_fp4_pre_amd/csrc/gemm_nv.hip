// Stages S2 and S3 for the NVFP4 MMA type (nvfp4.h; [P3] prhub digest of
// sglang PR "bump sgl-deep-gemm to 0.1.7, MegaMoE uses the mma_type API for
// MXFP4", "Motivation": the NVFP4 mega-MoE variant).  The same swap-AB weight
// streaming as the MXFP4 kernels (gemm1.hip, gemm2.hip; tiles.h): one
// workgroup of 4 waves per (expert, unit groups), each wave streaming its
// units' weight tiles HBM -> VGPR through a ring of D K steps, the expert's
// token rows (up to NT*16 per pass) gathered into LDS over all of K.  What
// differs is the product: each 16-byte FP4 operand (32 K elements of one
// row) and its two E4M3 block scales become four fp16 operands of exact
// products e2m1 * e4m3, which feed four dense 16x16x32 fp16 MFMAs; the fp32
// sums are multiplied by the tensor scales in the epilogues:
//   GEMM1: gate/up = sum * f32(g_x * g_w1[e]); h = silu(gate) * up; h is
//          requantized to NVFP4 with g_h (scale bytes per 16 columns);
//   GEMM2: y = bf16(sum * f32(g_h * g_w2[e])).
// Weight scales: 8 bytes per lane and K step (nvfp4.h); token scales: one
// byte per 16 elements, two per lane and step.
#include "epilogue.h"
#include "epilogue_nv.h"
#include "gemm_common.h"
#include "launch.h"
#include "nvfp4.h"
#include "tiles.h"
#include "validate.h"

#ifndef MOE_NV_RING_DEPTH
#define MOE_NV_RING_DEPTH 2       // weight-ring slots (divides the K steps)
#endif
#ifndef MOE_NV_TWO_TILES_ABOVE
#define MOE_NV_TWO_TILES_ABOVE 16 // mean routed rows per expert above which a pass takes two token tiles
#endif

namespace moe {

static_assert(MOE_NV_RING_DEPTH * kUnitStepStride <= kPreparedTailBytes, "weight read-ahead past the prepared tail");

__device__ __forceinline__ uint2 buf_load8(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kPolicyStream);
  return make_uint2(v[0], v[1]);
}

// The wave's first D K steps of weight codes and scales.
template <int D>
__device__ __forceinline__ void fill_ring_nv(uint4 (&a)[D][4], uint2 (&sa)[D], __amdgpu_buffer_rsrc_t wr,
                                             __amdgpu_buffer_rsrc_t sr, int voff, int svoff) {
#pragma unroll
  for (int d = 0; d < D; ++d) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) a[d][rb] = buf_load16(wr, voff + rb * 1024, d * kUnitStepStride);
    sa[d] = buf_load8(sr, svoff, d * kNvUnitScaleStride);
  }
}

// The two E4M3 scale bytes of token row n, K step s, lane group kb in the LDS
// tile (one byte per 16 elements; scale dword d of row n at d ^ (n % width),
// gemm_common.h).
__device__ __forceinline__ uint32_t tile_scales_nv(const uint8_t* lds_scales, int sc_bytes, int n, int s, int kb) {
  const int scm = scale_swizzle(sc_bytes) - 1;
  const int d = 2 * s + (kb >> 1);
  return *reinterpret_cast<const uint16_t*>(lds_scales + n * sc_bytes + ((d ^ (n & scm)) << 2) + ((kb & 1) << 1));
}

// The four fp16 operands of one 16-byte FP4 operand: dword i (K elements
// 8i..8i+7 of the lane's 32) with the scale of its 16-element half.
__device__ __forceinline__ void nv_operands(const uint4& c, uint32_t scales, v8h (&o)[4]) {
  const v2h lo = e4m3_scale_f16x2(scales & 0xFFu), hi = e4m3_scale_f16x2((scales >> 8) & 0xFFu);
  o[0] = nv_operand(c.x, lo);
  o[1] = nv_operand(c.y, lo);
  o[2] = nv_operand(c.z, hi);
  o[3] = nv_operand(c.w, hi);
}

// One K step of a wave: 4 weight blocks x NT token tiles x 4 MFMAs.
template <int NT, int SWZ, int ROWS>
__device__ __forceinline__ void nv_step(v4f (&acc)[NT][4], const uint4 (&a)[4], uint2 sa, const uint8_t* lds_codes,
                                        const uint8_t* lds_scales, int row_bytes, int sc_bytes, int s, int kb,
                                        int tok_lane) {
  v8h b[NT][4];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = min(nt * 16 + tok_lane, ROWS - 1);
    nv_operands(tile_operand<SWZ>(lds_codes, row_bytes, n, s, kb), tile_scales_nv(lds_scales, sc_bytes, n, s, kb),
                b[nt]);
  }
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    v8h w[4];
    nv_operands(a[rb], ((rb < 2 ? sa.x : sa.y) >> (16 * (rb & 1))) & 0xFFFFu, w);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[nt][rb] = mfma_f16(w[i], b[nt][i], acc[nt][rb]);
  }
}

// GEMM1: grid E * (I / (128 * upw)) workgroups of 4 waves; wave w owns unit
// w of each of its upw groups of 4 units (gemm1.hip).
template <int NT, int D, int SWZ>
__global__ void __launch_bounds__(256, 2) gemm1_nv_kernel(
    const uint8_t* __restrict__ w1c, const uint8_t* __restrict__ w1s, const float* __restrict__ gsc,
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xsf, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_rows, int H, int I, int E, int k,
    int upw, int hrows, uint8_t* __restrict__ hq, uint8_t* __restrict__ hsf, float* __restrict__ acc_out) {
  const int groups = I / (128 * upw);
  const int e = blockIdx.x / groups;
  const int g = blockIdx.x - e * groups;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int u0 = g * 4 * upw + wave;
  const int S = H / kStepK;
  const int total_steps = upw * S;
  const int row_bytes = H / 2, sc_bytes = H / 16;
  constexpr int ROWS = NT == 1 ? 16 : kNvStreamRows;
  static_assert(ROWS > 16 * (NT - 1) && ROWS <= 16 * NT, "rows per pass must need NT tiles");
  extern __shared__ __align__(16) uint8_t lds[];
  uint8_t* lds_codes = lds;
  uint8_t* lds_scales = lds + ROWS * row_bytes;

  const __amdgpu_buffer_rsrc_t wr =
      make_rsrc(w1c + w1_code_offset(e, u0, 0, H, I), (uint32_t)(total_steps - 1) * kUnitStepStride + kStepCodeBytes);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(
      w1s + nv_w1_scale_offset(e, u0, 0, H, I), (uint32_t)(total_steps - 1) * kNvUnitScaleStride + kNvStepScaleBytes);
  const int voff = lane * 16, svoff = lane * 8;
  const int tok_lane = lane & 15, kb = lane >> 4;

  // Two token tiles: the first ring loads go out before the row count is read
  // (gemm1.hip); the empty asm keeps them above the branch.
  constexpr bool kEarly = NT == 2;
  uint4 a[D][4];
  uint2 sa[D];
  if constexpr (kEarly) {
    fill_ring_nv<D>(a, sa, wr, sr, voff, svoff);
    asm volatile("" ::"s"(w1c), "s"(w1s) : "memory");
  }
  const int n_e = counts[e];
  if (n_e == 0) {
    if constexpr (kEarly) wait_vmem_all();
    return;
  }
  const int base = offsets[e];
  const float gg = __fmul_rn(gsc[2 * E], gsc[e]);
  const float gh = gsc[2 * E + 1];

  for (int t0 = 0; t0 < n_e; t0 += ROWS) {
    const int nrows = min(ROWS, n_e - t0);
    if (!kEarly || t0 > 0) fill_ring_nv<D>(a, sa, wr, sr, voff, svoff);
    const int my_tok = lane < nrows ? sorted_rows[base + t0 + lane] / k : 0;
    __syncthreads();  // the previous pass has finished reading LDS
    gather_tile<ROWS, SWZ>(lds_codes, lds_scales, xq, xsf, row_bytes, sc_bytes, nrows,
                           [&](int n) { return __shfl(my_tok, n, 64); }, wave, lane, 4);
    wait_vmem_all();
    __syncthreads();

    v4f acc[NT][4];
    zero_acc<NT>(acc);
    for (int j0 = 0; j0 < total_steps; j0 += D) {
      const int s0 = j0 % S;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        int tl = tok_lane;
        asm volatile("" : "+v"(tl));   // LDS row addresses recomputed each step (gemm1.hip)
        nv_step<NT, SWZ, ROWS>(acc, a[d], sa[d], lds_codes, lds_scales, row_bytes, sc_bytes, s0 + d, kb, tl);
        const int jn = j0 + d + D;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) a[d][rb] = buf_load16(wr, voff + rb * 1024, jn * kUnitStepStride);
        sa[d] = buf_load8(sr, svoff, jn * kNvUnitScaleStride);
      }
      if (s0 + D != S) continue;
      int r0 = base + t0;
      asm volatile("" : "+s"(r0));
      gemm1_epilogue_nv<NT>(acc, u0 + kGroupUnits * (j0 / S), r0, nrows, I, hrows, lane, gg, gh, hq, hsf, acc_out);
      zero_acc<NT>(acc);
    }
  }
}

// GEMM2: grid E * (H / (256 * upw)) workgroups of 4 waves; wave w owns unit
// w of each of its upw groups of 4 units (gemm2.hip).  The expert's rows of h
// are consecutive in every plane of hq (64 code bytes a row) and in every
// dword plane of hsf, so the tile is one contiguous run per plane.
template <int NT, int D, int SWZ>
__global__ void __launch_bounds__(256, 2) gemm2_nv_kernel(
    const uint8_t* __restrict__ w2c, const uint8_t* __restrict__ w2s, const float* __restrict__ gsc,
    const uint8_t* __restrict__ hq, const uint8_t* __restrict__ hsf, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, int H, int I, int E, int upw, int hrows, uint16_t* __restrict__ y) {
  const int groups = H / (256 * upw);
  const int e = blockIdx.x / groups;
  const int g = blockIdx.x - e * groups;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int v0 = g * 4 * upw + wave;
  const int S = I / kStepK;
  const int total_steps = upw * S;
  const int row_bytes = I / 2, sc_bytes = I / 16;
  constexpr int ROWS = NT == 1 ? 16 : kNvStreamRows;
  static_assert(ROWS > 16 * (NT - 1) && ROWS <= 16 * NT, "rows per pass must need NT tiles");
  extern __shared__ __align__(16) uint8_t lds[];
  uint8_t* lds_codes = lds;
  uint8_t* lds_scales = lds + ROWS * row_bytes;

  const __amdgpu_buffer_rsrc_t wr =
      make_rsrc(w2c + w2_code_offset(e, v0, 0, H, I), (uint32_t)(total_steps - 1) * kUnitStepStride + kStepCodeBytes);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(
      w2s + nv_w2_scale_offset(e, v0, 0, H, I), (uint32_t)(total_steps - 1) * kNvUnitScaleStride + kNvStepScaleBytes);
  const int voff = lane * 16, svoff = lane * 8;
  const int tok_lane = lane & 15, kb = lane >> 4;

  constexpr bool kEarly = NT == 2;
  uint4 a[D][4];
  uint2 sa[D];
  if constexpr (kEarly) {
    fill_ring_nv<D>(a, sa, wr, sr, voff, svoff);
    asm volatile("" ::"s"(w2c), "s"(w2s) : "memory");
  }
  const int n_e = counts[e];
  if (n_e == 0) {
    if constexpr (kEarly) wait_vmem_all();
    return;
  }
  const int base = offsets[e];
  const float g2 = __fmul_rn(gsc[2 * E + 1], gsc[E + e]);

  for (int t0 = 0; t0 < n_e; t0 += ROWS) {
    const int nrows = min(ROWS, n_e - t0);
    if (!kEarly || t0 > 0) fill_ring_nv<D>(a, sa, wr, sr, voff, svoff);
    __syncthreads();
    const int row0 = base + t0;
    gather_tile<ROWS, SWZ, true, 64>(lds_codes, lds_scales, hq, hsf, row_bytes, sc_bytes, nrows,
                                     [&](int n) { return row0 + n; }, wave, lane, 4, hrows);
    wait_vmem_all();
    __syncthreads();

    v4f acc[NT][4];
    zero_acc<NT>(acc);
    for (int j0 = 0; j0 < total_steps; j0 += D) {
      const int s0 = j0 % S;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        int tl = tok_lane;
        asm volatile("" : "+v"(tl));
        nv_step<NT, SWZ, ROWS>(acc, a[d], sa[d], lds_codes, lds_scales, row_bytes, sc_bytes, s0 + d, kb, tl);
        const int jn = j0 + d + D;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) a[d][rb] = buf_load16(wr, voff + rb * 1024, jn * kUnitStepStride);
        sa[d] = buf_load8(sr, svoff, jn * kNvUnitScaleStride);
      }
      if (s0 + D == S) {
        int r0 = base + t0;
        asm volatile("" : "+s"(r0));
        gemm2_epilogue_nv<NT>(acc, v0 + kGroupUnits * (j0 / S), r0, nrows, H, lane, g2, y);
        zero_acc<NT>(acc);
      }
    }
  }
}

namespace {

// Lets kern use `lds` bytes of dynamic LDS (more than 64 KiB needs the attribute).
template <class K>
hipError_t allow_lds(K kern, size_t lds) {
  return lds > 65536 ? raise_lds_limit(reinterpret_cast<const void*>(kern), lds) : hipSuccess;
}

// Ring depth: MOE_NV_RING_DEPTH when it divides the K steps, else 2 (K % 256 == 0 for GEMM1,
// K % 128 for GEMM2: 1 is left for an odd step count).
inline int ring_depth(int steps) { return steps % MOE_NV_RING_DEPTH == 0 ? MOE_NV_RING_DEPTH : steps % 2 == 0 ? 2 : 1; }

// Swizzle width of the token code rows: the largest of 16, 8, 4 dividing the 16-byte chunks per row.
inline int swizzle(int row_bytes) {
  const int chunks = row_bytes / 16;
  return chunks % 16 == 0 ? 16 : chunks % 8 == 0 ? 8 : 4;
}

}  // namespace

#define NV_G1_ARGS w1c, w1s, gsc, xq, xsf, counts, offsets, sorted_rows, H, I, E, k, upw, hrows, hq, hsf, acc_out

template <int NT, int D, int SWZ>
static hipError_t launch_gemm1_nv_t(const uint8_t* w1c, const uint8_t* w1s, const float* gsc, const uint8_t* xq,
                                    const uint8_t* xsf, const int32_t* counts, const int32_t* offsets,
                                    const int32_t* sorted_rows, int H, int I, int E, int k, int hrows, uint8_t* hq,
                                    uint8_t* hsf, float* acc_out, size_t min_lds, hipStream_t stream) {
  constexpr int ROWS = NT == 1 ? 16 : kNvStreamRows;
  size_t lds = (size_t)ROWS * (H / 2 + H / 16);
  if (lds < min_lds) lds = min_lds;
  auto kern = gemm1_nv_kernel<NT, D, SWZ>;
  const int upw = units_per_wave(I / 32 / 4, 2);
  hipError_t err = allow_lds(kern, lds);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(kern, dim3(E * (I / (128 * upw))), dim3(256), lds, stream, NV_G1_ARGS);
  return hipGetLastError();
}

template <int NT, int D>
static hipError_t launch_gemm1_nv_d(const uint8_t* w1c, const uint8_t* w1s, const float* gsc, const uint8_t* xq,
                                    const uint8_t* xsf, const int32_t* counts, const int32_t* offsets,
                                    const int32_t* sorted_rows, int H, int I, int E, int k, int hrows, uint8_t* hq,
                                    uint8_t* hsf, float* acc_out, size_t min_lds, hipStream_t stream) {
  switch (swizzle(H / 2)) {
    case 16: return launch_gemm1_nv_t<NT, D, 16>(w1c, w1s, gsc, xq, xsf, counts, offsets, sorted_rows, H, I, E, k,
                                                 hrows, hq, hsf, acc_out, min_lds, stream);
    default: return launch_gemm1_nv_t<NT, D, 8>(w1c, w1s, gsc, xq, xsf, counts, offsets, sorted_rows, H, I, E, k,
                                                hrows, hq, hsf, acc_out, min_lds, stream);
  }
}

template <int NT>
static hipError_t launch_gemm1_nv_nt(const uint8_t* w1c, const uint8_t* w1s, const float* gsc, const uint8_t* xq,
                                     const uint8_t* xsf, const int32_t* counts, const int32_t* offsets,
                                     const int32_t* sorted_rows, int H, int I, int E, int k, int hrows, uint8_t* hq,
                                     uint8_t* hsf, float* acc_out, size_t min_lds, hipStream_t stream) {
  // H % 256 == 0: the K steps are even
  if (ring_depth(H / kStepK) == MOE_NV_RING_DEPTH)
    return launch_gemm1_nv_d<NT, MOE_NV_RING_DEPTH>(w1c, w1s, gsc, xq, xsf, counts, offsets, sorted_rows, H, I, E, k,
                                                    hrows, hq, hsf, acc_out, min_lds, stream);
  return launch_gemm1_nv_d<NT, 2>(w1c, w1s, gsc, xq, xsf, counts, offsets, sorted_rows, H, I, E, k, hrows, hq, hsf,
                                  acc_out, min_lds, stream);
}

hipError_t launch_gemm1_nv(const uint8_t* w1c, const uint8_t* w1s, const float* gsc, const uint8_t* xq,
                           const uint8_t* xsf, const int32_t* counts, const int32_t* offsets,
                           const int32_t* sorted_rows, int H, int I, int E, int k, int rows_hint, int hrows,
                           uint8_t* hq, uint8_t* hsf, float* acc_out, hipStream_t stream) {
  // With more than 8 rows per expert on average (most workgroups live), at
  // most two one-tile workgroups per CU: 56 KiB of LDS each.  At 512 tokens
  // (DeepSeek-V4-Flash shape, 12 rows per expert) GEMM1 473 -> 455 us; at
  // 64 tokens (2 rows) the same cap measured slower (310 -> 327 us), and
  // GEMM2 slower at both, so they keep the tile's own LDS size.
  const size_t min_lds = rows_hint > 8 ? (size_t)56 << 10 : 0;
  if (rows_hint > MOE_NV_TWO_TILES_ABOVE)
    return launch_gemm1_nv_nt<2>(w1c, w1s, gsc, xq, xsf, counts, offsets, sorted_rows, H, I, E, k, hrows, hq, hsf,
                                 acc_out, min_lds, stream);
  return launch_gemm1_nv_nt<1>(w1c, w1s, gsc, xq, xsf, counts, offsets, sorted_rows, H, I, E, k, hrows, hq, hsf,
                               acc_out, min_lds, stream);
}

#undef NV_G1_ARGS

template <int NT, int D, int SWZ>
static hipError_t launch_gemm2_nv_t(const uint8_t* w2c, const uint8_t* w2s, const float* gsc, const uint8_t* hq,
                                    const uint8_t* hsf, const int32_t* counts, const int32_t* offsets, int H, int I,
                                    int E, int hrows, uint16_t* y, hipStream_t stream) {
  constexpr int ROWS = NT == 1 ? 16 : kNvStreamRows;
  const size_t lds = (size_t)ROWS * (I / 2 + I / 16);
  auto kern = gemm2_nv_kernel<NT, D, SWZ>;
  const int upw = units_per_wave(H / kUnitRows / 4, 1);
  hipError_t err = allow_lds(kern, lds);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(kern, dim3(E * (H / (256 * upw))), dim3(256), lds, stream, w2c, w2s, gsc, hq, hsf, counts,
                     offsets, H, I, E, upw, hrows, y);
  return hipGetLastError();
}

template <int NT, int D>
static hipError_t launch_gemm2_nv_d(const uint8_t* w2c, const uint8_t* w2s, const float* gsc, const uint8_t* hq,
                                    const uint8_t* hsf, const int32_t* counts, const int32_t* offsets, int H, int I,
                                    int E, int hrows, uint16_t* y, hipStream_t stream) {
  switch (swizzle(I / 2)) {
    case 16: return launch_gemm2_nv_t<NT, D, 16>(w2c, w2s, gsc, hq, hsf, counts, offsets, H, I, E, hrows, y, stream);
    case 8: return launch_gemm2_nv_t<NT, D, 8>(w2c, w2s, gsc, hq, hsf, counts, offsets, H, I, E, hrows, y, stream);
    default: return launch_gemm2_nv_t<NT, D, 4>(w2c, w2s, gsc, hq, hsf, counts, offsets, H, I, E, hrows, y, stream);
  }
}

template <int NT>
static hipError_t launch_gemm2_nv_nt(const uint8_t* w2c, const uint8_t* w2s, const float* gsc, const uint8_t* hq,
                                     const uint8_t* hsf, const int32_t* counts, const int32_t* offsets, int H, int I,
                                     int E, int hrows, uint16_t* y, hipStream_t stream) {
  const int d = ring_depth(I / kStepK);
  if (d == MOE_NV_RING_DEPTH)
    return launch_gemm2_nv_d<NT, MOE_NV_RING_DEPTH>(w2c, w2s, gsc, hq, hsf, counts, offsets, H, I, E, hrows, y,
                                                    stream);
  if (d == 2) return launch_gemm2_nv_d<NT, 2>(w2c, w2s, gsc, hq, hsf, counts, offsets, H, I, E, hrows, y, stream);
  return launch_gemm2_nv_d<NT, 1>(w2c, w2s, gsc, hq, hsf, counts, offsets, H, I, E, hrows, y, stream);
}

hipError_t launch_gemm2_nv(const uint8_t* w2c, const uint8_t* w2s, const float* gsc, const uint8_t* hq,
                           const uint8_t* hsf, const int32_t* counts, const int32_t* offsets, int H, int I, int E,
                           int rows_hint, int hrows, uint16_t* y, hipStream_t stream) {
  if (rows_hint > MOE_NV_TWO_TILES_ABOVE) return launch_gemm2_nv_nt<2>(w2c, w2s, gsc, hq, hsf, counts, offsets, H, I, E, hrows, y, stream);
  return launch_gemm2_nv_nt<1>(w2c, w2s, gsc, hq, hsf, counts, offsets, H, I, E, hrows, y, stream);
}

}  // namespace moe

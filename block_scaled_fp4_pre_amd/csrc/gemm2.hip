// Stage S3: per-expert GEMM2 (down projection) y = h_hat . W2_hat[e]^T with fp32
// accumulation on the gfx950 block-scaled FP4 MFMA; y is written per routed row
// in expert-sorted order, rounded to bfloat16, for the combine.
//
// [P1] sglang PR "[deepseek-v4] Bump sgl-deep-gemm for packed FP4xFP4 mega-MoE
// (W4A4)": title (packed FP4 x FP4) and section B "NCU Speed-of-Light" (the
// weight stream bounds the layer at ntok=512).
//
// Grid: one workgroup of 4 waves per (expert, 256*upw hidden rows), i.e. upw
// groups of 4 units of 64 hidden rows; wave w owns unit w of each group and
// streams them as one sequence of K steps (one fixed stride in the tile order
// of tiles.h), writing y at each unit's end.  The expert's requantized rows are
// consecutive in every K-step plane of hq/hsf (epilogue.h), so the B tile is
// one contiguous run per plane, copied into LDS by direct-to-LDS loads;
// weights stream through the register ring of stream_ring.h; a workgroup
// whose expert has no rows exits as in gemm1.hip.  F8 (the
// fp8xfp4 MMA type): h arrives as E4M3 bytes and the MFMA's B operand takes 32
// bytes (format code 0).
#include "epilogue.h"
#include "gemm_common.h"
#include "launch.h"
#include "stream_ring.h"
#include "tiles.h"

#ifndef MOE_STREAM_RING_DEPTH
#define MOE_STREAM_RING_DEPTH 4   // weight-ring slots of the streaming GEMMs (divides the K steps)
#endif
#ifndef MOE_STREAM_ROWS2
#define MOE_STREAM_ROWS2 24       // token rows per pass of the two-tile variant (17..32)
#endif

#ifndef MOE_GEMM2_MIN_BLOCKS
#define MOE_GEMM2_MIN_BLOCKS 2    // launch bound: workgroups per CU the register budget must allow
#endif

#ifndef MOE_STREAM_EARLY
#define MOE_STREAM_EARLY 1        // two-tile form: first weight loads before the row count is read
#endif

#ifndef MOE_GEMM2_UNITS_PER_WAVE
#define MOE_GEMM2_UNITS_PER_WAVE 1
#endif

namespace moe {

template <int NT, int D, int SWZ, bool F8>
__global__ void __launch_bounds__(256, MOE_GEMM2_MIN_BLOCKS) gemm2_kernel(
    const uint8_t* __restrict__ w2c, const uint8_t* __restrict__ w2s, const uint8_t* __restrict__ hq,
    const uint8_t* __restrict__ hsf, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, int H, int I, int upw, int hrows, uint16_t* __restrict__ y) {
  const int groups = H / (256 * upw);
  const int e = blockIdx.x / groups;
  const int g = blockIdx.x - e * groups;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: keeps the buffer resources in SGPRs
  const int v0 = g * 4 * upw + wave;   // wave w owns unit w of each of the workgroup's upw unit groups
  const int S = I / kStepK;
  const int total_steps = upw * S;       // the wave's upw units: one stream at stride kUnitStepStride
  const int row_bytes = F8 ? I : I / 2, sc_bytes = I / 32;   // E4M3 bytes or packed E2M1

  // Rows per pass: 16 for one token tile; MOE_STREAM_ROWS2 (<= 32) for two.  A
  // cap below 32 trades a rare second pass for less LDS per workgroup; B-operand
  // reads clamp the row so the second tile never reads past the cap.
  constexpr int ROWS = NT == 1 ? 16 : MOE_STREAM_ROWS2;
  static_assert(ROWS > 16 * (NT - 1) && ROWS <= 16 * NT, "rows per pass must need NT tiles");
  extern __shared__ __align__(16) uint8_t lds[];
  uint8_t* lds_codes = lds;
  uint8_t* lds_scales = lds + ROWS * row_bytes;

  const __amdgpu_buffer_rsrc_t wr =
      make_rsrc(w2c + w2_code_offset(e, v0, 0, H, I), (uint32_t)(total_steps - 1) * kUnitStepStride + kStepCodeBytes);
  const __amdgpu_buffer_rsrc_t sr =
      make_rsrc(w2s + w2_scale_offset(e, v0, 0, H, I), (uint32_t)(total_steps - 1) * kUnitScaleStride + kStepScaleBytes);
  const int voff = lane * 16, svoff = lane * 4;
  const int tok_lane = lane & 15, kb = lane >> 4;

  // With two token tiles (many rows per expert) an empty expert is rare, so
  // the first pass's weight loads go out before the expert's row count is
  // known; an empty expert's workgroup waits for them and exits.  The empty
  // asm statement may, as far as the compiler knows, write the weights, so the
  // loads cannot be sunk below the branch.
  constexpr bool kEarly = NT == 2 && MOE_STREAM_EARLY;
  uint4 a[D][4];
  uint32_t sa[D];
  if constexpr (kEarly) {
    fill_weight_ring<D>(a, sa, wr, sr, voff, svoff, kUnitStepStride, kUnitScaleStride);
    asm volatile("" ::"s"(w2c), "s"(w2s) : "memory");
  }
  const int n_e = counts[e];
  if (n_e == 0) {
    if constexpr (kEarly) wait_vmem_all();
    return;
  }
  const int base = offsets[e];

  for (int t0 = 0; t0 < n_e; t0 += ROWS) {
    const int nrows = min(ROWS, n_e - t0);
    if (!kEarly || t0 > 0) fill_weight_ring<D>(a, sa, wr, sr, voff, svoff, kUnitStepStride, kUnitScaleStride);
    __syncthreads();
    const int row0 = base + t0;
    gather_tile<ROWS, SWZ, true, F8 ? 128 : 64>(lds_codes, lds_scales, hq, hsf, row_bytes, sc_bytes, nrows,
                                                [&](int n) { return row0 + n; }, wave, lane, 4, hrows);
    wait_vmem_all();
    __syncthreads();

    v4f acc[NT][4];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) acc[nt][rb] = v4f{0.f, 0.f, 0.f, 0.f};

    // Steady state without branches: D divides S.  The D steps of loads
    // issued past the wave's last step are never consumed; they read the
    // bytes after its stream (the next unit's, or the prepared buffer's tail,
    // kPreparedTailBytes), or zeros where the buffer range check drops them.
    for (int j0 = 0; j0 < total_steps; j0 += D) {
      const int s0 = j0 % S;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const int s = s0 + d;
        // The lane's token row goes through an opaque copy each step, so the
        // per-tile LDS addresses are recomputed there instead of being held
        // in registers across the loop (two fewer VGPRs; GEMM2 at T = 512
        // measured about 1 us faster).
        int tl = tok_lane;
        asm volatile("" : "+v"(tl));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int n = min(nt * 16 + tl, ROWS - 1);
          const int sb = tile_scale(lds_scales, sc_bytes, n, s, kb);
          if constexpr (F8) {
            uint4 blo, bhi;
            tile_operand8<SWZ>(lds_codes, row_bytes, n, s, kb, blo, bhi);
            acc[nt][0] = mfma_fp4_fp8<0, 0>(a[d][0], blo, bhi, acc[nt][0], (int)sa[d], sb);
            acc[nt][1] = mfma_fp4_fp8<1, 0>(a[d][1], blo, bhi, acc[nt][1], (int)sa[d], sb);
            acc[nt][2] = mfma_fp4_fp8<2, 0>(a[d][2], blo, bhi, acc[nt][2], (int)sa[d], sb);
            acc[nt][3] = mfma_fp4_fp8<3, 0>(a[d][3], blo, bhi, acc[nt][3], (int)sa[d], sb);
          } else {
            const uint4 b = tile_operand<SWZ>(lds_codes, row_bytes, n, s, kb);
            acc[nt][0] = mfma_fp4<0, 0>(a[d][0], b, acc[nt][0], (int)sa[d], sb);
            acc[nt][1] = mfma_fp4<1, 0>(a[d][1], b, acc[nt][1], (int)sa[d], sb);
            acc[nt][2] = mfma_fp4<2, 0>(a[d][2], b, acc[nt][2], (int)sa[d], sb);
            acc[nt][3] = mfma_fp4<3, 0>(a[d][3], b, acc[nt][3], (int)sa[d], sb);
          }
        }
        const int jn = j0 + d + D;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) a[d][rb] = buf_load16(wr, voff + rb * 1024, jn * kUnitStepStride);
        sa[d] = buf_load4(sr, svoff, jn * kUnitScaleStride);
      }
      if (s0 + D == S) {
        // unit finished: its 64 hidden columns of y for the tile's rows
        int r0 = base + t0;
        asm volatile("" : "+s"(r0));   // likewise: y's row addresses are computed here
        gemm2_epilogue<NT>(acc, v0 + kGroupUnits * (j0 / S), r0, nrows, H, lane, y);
        zero_acc<NT>(acc);
      }
    }
  }
}

#define MOE_GEMM2_ARGS w2c, w2s, hq, hsf, counts, offsets, H, I, E, hrows, y, stream

template <int NT, int D, int SWZ, bool F8>
static hipError_t launch_gemm2_t(const uint8_t* w2c, const uint8_t* w2s, const uint8_t* hq,
                                 const uint8_t* hsf, const int32_t* counts, const int32_t* offsets,
                                 int H, int I, int E, int hrows, uint16_t* y, hipStream_t stream) {
  constexpr int ROWS = NT == 1 ? 16 : MOE_STREAM_ROWS2;
  size_t lds = (size_t)ROWS * (F8 ? I : I / 2) + (size_t)ROWS * (I / 32);
  if (lds < kStreamMinLds) lds = kStreamMinLds;   // at most two workgroups per CU (stream_ring.h)
  auto kern = gemm2_kernel<NT, D, SWZ, F8>;
  const int upw = units_per_wave(H / kUnitRows / 4, MOE_GEMM2_UNITS_PER_WAVE);
  if (lds > 65536) {
    hipError_t err = raise_lds_limit(reinterpret_cast<const void*>(kern), lds);
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(kern, dim3(E * (H / (256 * upw))), dim3(256), lds, stream, w2c, w2s, hq, hsf, counts,
                     offsets, H, I, upw, hrows, y);
  return hipGetLastError();
}

template <int NT, int D, bool F8>
static hipError_t launch_gemm2_nt(const uint8_t* w2c, const uint8_t* w2s, const uint8_t* hq,
                                  const uint8_t* hsf, const int32_t* counts, const int32_t* offsets,
                                  int H, int I, int E, int hrows, uint16_t* y, hipStream_t stream) {
  const int chunks = F8 ? I / 16 : I / 32;  // 16-byte chunks per token row; a multiple of 4
  if (chunks % 16 == 0) return launch_gemm2_t<NT, D, 16, F8>(MOE_GEMM2_ARGS);
  if (chunks % 8 == 0) return launch_gemm2_t<NT, D, 8, F8>(MOE_GEMM2_ARGS);
  return launch_gemm2_t<NT, D, 4, F8>(MOE_GEMM2_ARGS);
}

template <int NT, bool F8>
static hipError_t launch_gemm2_d(const uint8_t* w2c, const uint8_t* w2s, const uint8_t* hq,
                                 const uint8_t* hsf, const int32_t* counts, const int32_t* offsets,
                                 int H, int I, int E, int hrows, uint16_t* y, hipStream_t stream) {
  // The ring depth must divide the number of K steps I/128.
  const int S = I / kStepK;
  if (S % MOE_STREAM_RING_DEPTH == 0) return launch_gemm2_nt<NT, MOE_STREAM_RING_DEPTH, F8>(MOE_GEMM2_ARGS);
  if (S % 2 == 0) return launch_gemm2_nt<NT, 2, F8>(MOE_GEMM2_ARGS);
  return launch_gemm2_nt<NT, 1, F8>(MOE_GEMM2_ARGS);
}

hipError_t launch_gemm2(bool fp8, const uint8_t* w2c, const uint8_t* w2s, const uint8_t* hq, const uint8_t* hsf,
                        const int32_t* counts, const int32_t* offsets, int H, int I, int E,
                        int rows_hint, int hrows, uint16_t* y, hipStream_t stream) {
  if (rows_hint > 8) return fp8 ? launch_gemm2_d<2, true>(MOE_GEMM2_ARGS) : launch_gemm2_d<2, false>(MOE_GEMM2_ARGS);
  return fp8 ? launch_gemm2_d<1, true>(MOE_GEMM2_ARGS) : launch_gemm2_d<1, false>(MOE_GEMM2_ARGS);
}

#undef MOE_GEMM2_ARGS

}  // namespace moe

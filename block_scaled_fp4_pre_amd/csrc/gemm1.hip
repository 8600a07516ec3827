// Stage S2: per-expert GEMM1 (tokens x W1^T over gate and up) with fp32
// accumulation on the gfx950 block-scaled FP4 MFMA, then SwiGLU
// h = silu(gate) * up and requantization of h to MXFP4 along the inter axis.
//
// [P1] sglang PR "[deepseek-v4] Bump sgl-deep-gemm for packed FP4xFP4 mega-MoE
// (W4A4)": title (both operands packed FP4) and section B "NCU Speed-of-Light"
// (the layer is memory-bound at ntok=512: the weight data path sets the time).
// [P3] prhub digest of sglang PR "bump sgl-deep-gemm to 0.1.7, MegaMoE uses the
// mma_type API for MXFP4", "Key source snippets": activation="swiglu"; W1 rows
// [0, I) are gate and [I, 2I) are up (the split _interleave_mega_moe_gate_up
// slices).  The pages' gate/up interleave is tied to their MMA layout; here the
// pairing is by MFMA block instead (tiles.h).
//
// Grid: one workgroup of 4 waves per (expert, 128*upw inter columns), i.e. upw
// groups of 4 units of 32 columns (64 weight rows each); wave w owns unit w of
// each group.  In the tile order of tiles.h those units' chunks follow each
// other at one fixed stride, so the wave streams them as one sequence of K
// steps, and the 4 waves read one contiguous 16 KiB per step.  A workgroup whose
// expert has no rows exits (with two token tiles, once the first ring loads it
// issued ahead of the row count have landed).  Per pass it takes up to NT*16 of
// the expert's rows: their quantized tokens are gathered into LDS (B operand)
// by direct-to-LDS loads while the wave's weight ring (stream_ring.h) fills;
// then 4 MFMAs (one per 16-row block) per token tile per K step of 128.
// Epilogue per lane: gate/up of 8 columns for one token; the 32-column absmax
// is reduced over the 4 lanes holding that token (xor 16, xor 32).
//
// F8 (the fp8xfp4 MMA type, [P3] "Implementation breakdown" items 1-3): the
// tokens are E4M3 bytes, twice the LDS per row, the B operand of each MFMA
// takes 32 bytes (format code 0), and h is requantized to E4M3.  With two
// token tiles its workgroups have 8 waves: waves 4q..4q+3 own the q-th run of
// upw unit groups, and all 8 share the token tile.
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

#ifndef MOE_STREAM_EARLY
#define MOE_STREAM_EARLY 1        // two-tile form: first weight loads before the row count is read
#endif

#ifndef MOE_G1_F8_WAVES
#define MOE_G1_F8_WAVES 8         // waves per workgroup, E4M3 tokens with two tiles (4 or 8)
#endif
#ifndef MOE_GEMM1_UNITS_PER_WAVE
#define MOE_GEMM1_UNITS_PER_WAVE 2
#endif

namespace moe {

template <int NT, int D, int SWZ, bool F8, int WAVES = 4>
__global__ void __launch_bounds__(64 * WAVES, WAVES == 4 ? 2 : 1) gemm1_swiglu_kernel(
    const uint8_t* __restrict__ w1c, const uint8_t* __restrict__ w1s, const uint8_t* __restrict__ xq,
    const uint8_t* __restrict__ xsf, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_rows, int H, int I, int k,
    int upw, int hrows, uint8_t* __restrict__ hq, uint8_t* __restrict__ hsf, float* __restrict__ acc_out) {
  const int groups = I / (32 * WAVES * upw);   // unit blocks (WAVES * upw units) per expert
  const int e = blockIdx.x / groups;
  const int g = blockIdx.x - e * groups;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: keeps the buffer resources in SGPRs
  // wave w owns unit w % 4 of each of its upw unit groups; waves 4q..4q+3
  // take the q-th run of upw groups of the workgroup's block
  const int u0 = (g * (WAVES / 4) + wave / 4) * 4 * upw + (wave & 3);
  const int S = H / kStepK;
  const int total_steps = upw * S;       // the wave's upw units: one stream at stride kUnitStepStride
  const int row_bytes = F8 ? H : H / 2, sc_bytes = H / 32;   // token row: E4M3 bytes or packed E2M1

  // Rows per pass: 16 for one token tile; MOE_STREAM_ROWS2 (<= 32) for two.  A
  // cap below 32 trades a rare second pass for less LDS per workgroup; B-operand
  // reads clamp the row so the second tile never reads past the cap.
  constexpr int ROWS = NT == 1 ? 16 : MOE_STREAM_ROWS2;
  static_assert(ROWS > 16 * (NT - 1) && ROWS <= 16 * NT, "rows per pass must need NT tiles");
  extern __shared__ __align__(16) uint8_t lds[];
  uint8_t* lds_codes = lds;                               // [NT*16][row_bytes], swizzled chunks
  uint8_t* lds_scales = lds + ROWS * row_bytes;           // [ROWS][sc_bytes]

  const __amdgpu_buffer_rsrc_t wr =
      make_rsrc(w1c + w1_code_offset(e, u0, 0, H, I), (uint32_t)(total_steps - 1) * kUnitStepStride + kStepCodeBytes);
  const __amdgpu_buffer_rsrc_t sr =
      make_rsrc(w1s + w1_scale_offset(e, u0, 0, H, I), (uint32_t)(total_steps - 1) * kUnitScaleStride + kStepScaleBytes);
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
    asm volatile("" ::"s"(w1c), "s"(w1s) : "memory");
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
    // token of each tile row: lane n < nrows holds it, broadcast by shuffle
    const int my_tok = lane < nrows ? sorted_rows[base + t0 + lane] / k : 0;
    __syncthreads();  // the previous pass has finished reading LDS
    gather_tile<ROWS, SWZ>(lds_codes, lds_scales, xq, xsf, row_bytes, sc_bytes, nrows,
                              [&](int n) { return __shfl(my_tok, n, 64); }, wave, lane, WAVES);
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
        // An opaque copy of the lane's token row each step: the per-tile LDS
        // addresses are recomputed here instead of being held in registers
        // across the loop (13 fewer VGPRs; 1-3 us per layer at T = 64 / 512).
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
      if (s0 + D != S) continue;

      // Unit finished: SwiGLU + requant of its 32 columns for the tile's rows.
      int r0 = base + t0;
      asm volatile("" : "+s"(r0));   // likewise: hq/hsf row addresses are computed here
      gemm1_epilogue<NT, F8>(acc, u0 + kGroupUnits * (j0 / S), r0, nrows, I, hrows, lane, hq, hsf, acc_out);
      zero_acc<NT>(acc);
    }
  }
}

#define MOE_GEMM1_ARGS w1c, w1s, xq, xsf, counts, offsets, sorted_rows, H, I, E, k, hrows, hq, hsf, acc_out, stream

template <int NT, int D, int SWZ, bool F8, int WAVES = 4>
static hipError_t launch_gemm1_t(const uint8_t* w1c, const uint8_t* w1s, const uint8_t* xq,
                                 const uint8_t* xsf, const int32_t* counts, const int32_t* offsets,
                                 const int32_t* sorted_rows, int H, int I, int E, int k, int hrows, uint8_t* hq,
                                 uint8_t* hsf, float* acc_out, hipStream_t stream) {
  constexpr int ROWS = NT == 1 ? 16 : MOE_STREAM_ROWS2;
  size_t lds = (size_t)ROWS * (F8 ? H : H / 2) + (size_t)ROWS * (H / 32);
  if (lds < kStreamMinLds) lds = kStreamMinLds;   // at most two workgroups per CU (stream_ring.h)
  auto kern = gemm1_swiglu_kernel<NT, D, SWZ, F8, WAVES>;
  const int upw = units_per_wave(I / 32 / WAVES, MOE_GEMM1_UNITS_PER_WAVE);
  if (lds > 65536) {
    hipError_t err = raise_lds_limit(reinterpret_cast<const void*>(kern), lds);
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(kern, dim3(E * (I / (32 * WAVES * upw))), dim3(64 * WAVES), lds, stream, w1c, w1s, xq, xsf, counts,
                     offsets, sorted_rows, H, I, k, upw, hrows, hq, hsf, acc_out);
  return hipGetLastError();
}

template <int NT, int D, bool F8>
static hipError_t launch_gemm1_nt(const uint8_t* w1c, const uint8_t* w1s, const uint8_t* xq,
                                  const uint8_t* xsf, const int32_t* counts, const int32_t* offsets,
                                  const int32_t* sorted_rows, int H, int I, int E, int k, int hrows, uint8_t* hq,
                                  uint8_t* hsf, float* acc_out, hipStream_t stream) {
  const int chunks = F8 ? H / 16 : H / 32;  // 16-byte chunks per token row; a multiple of 8
  // E4M3 tokens with two tiles: the token tile (101 KiB at H = 4096) fits
  // one workgroup per CU, so 8 waves (two unit groups) share it: at 512
  // tokens GEMM1 343 against 345 us with 4 waves.
  constexpr int W = F8 && NT == 2 ? MOE_G1_F8_WAVES : 4;
  if (W != 4 && (I / 32) % W != 0) {
    if (chunks % 16 == 0) return launch_gemm1_t<NT, D, 16, F8>(MOE_GEMM1_ARGS);
    return launch_gemm1_t<NT, D, 8, F8>(MOE_GEMM1_ARGS);
  }
  if (chunks % 16 == 0) return launch_gemm1_t<NT, D, 16, F8, W>(MOE_GEMM1_ARGS);
  return launch_gemm1_t<NT, D, 8, F8, W>(MOE_GEMM1_ARGS);
}

template <int NT, bool F8>
static hipError_t launch_gemm1_d(const uint8_t* w1c, const uint8_t* w1s, const uint8_t* xq,
                                 const uint8_t* xsf, const int32_t* counts, const int32_t* offsets,
                                 const int32_t* sorted_rows, int H, int I, int E, int k, int hrows, uint8_t* hq,
                                 uint8_t* hsf, float* acc_out, hipStream_t stream) {
  // The ring depth must divide the number of K steps H/128 (even, as H % 256 == 0).
  if ((H / kStepK) % MOE_STREAM_RING_DEPTH == 0) return launch_gemm1_nt<NT, MOE_STREAM_RING_DEPTH, F8>(MOE_GEMM1_ARGS);
  return launch_gemm1_nt<NT, 2, F8>(MOE_GEMM1_ARGS);
}

hipError_t launch_gemm1(bool fp8, const uint8_t* w1c, const uint8_t* w1s, const uint8_t* xq, const uint8_t* xsf,
                        const int32_t* counts, const int32_t* offsets, const int32_t* sorted_rows,
                        int H, int I, int E, int k, int rows_hint, int hrows, uint8_t* hq, uint8_t* hsf,
                        float* acc_out, hipStream_t stream) {
  // rows_hint: mean routed rows per expert; two token tiles per pass once a
  // single 16-row tile would often overflow (and re-stream the weights).
  if (rows_hint > 8)
    return fp8 ? launch_gemm1_d<2, true>(MOE_GEMM1_ARGS) : launch_gemm1_d<2, false>(MOE_GEMM1_ARGS);
  return fp8 ? launch_gemm1_d<1, true>(MOE_GEMM1_ARGS) : launch_gemm1_d<1, false>(MOE_GEMM1_ARGS);
}

#undef MOE_GEMM1_ARGS

}  // namespace moe

// Stages S1a + S1b fused in one launch for few routed rows (the pages'
// pre_dispatch: [P3] prhub digest of sglang PR "bump sgl-deep-gemm to 0.1.7,
// MegaMoE uses the mma_type API for MXFP4", "Key source snippets" -- one call
// that packs the tokens to E2M1 with group_size=32 and hands over the top-k ids
// and weights).
//
// Block 0 routes all R <= 8192 rows by itself.  Wave w of its 16 owns the
// contiguous rows [w*RW, (w+1)*RW), RW a multiple of 64, and reads their ids
// once.  Per-wave expert counts go to LDS (integer atomics only count, so the
// result does not depend on their order); one block scan gives counts and
// offsets (and the tile list); thread e then turns the counts of expert e into
// the first slot of each wave's rows of e.  Each wave then places its rows 64
// at a time, in order: the rank among the sub-chunk's rows of the same expert
// comes from a 64-lane match (one ballot per id bit), and the lowest lane of
// each expert advances the wave's slot for the next sub-chunk.  Blocks 1..
// quantize one 32-element group of x per thread meanwhile (E2M1, E4M3 for the
// fp8xfp4 MMA type, or NVFP4 under the layer's tensor scale g_x).
#include "launch.h"
#include "quant_group.h"
#include "route_common.h"

namespace moe {

constexpr int kPredispatchSubs = kPredispatchMaxRows / kRouteRows;  // 64-row sub-chunks per wave, at most

// ACT: the activation format, 0 = MXFP4, 1 = MXFP8 E4M3, 2 = NVFP4 with the
// tensor scale *gx.
template <int ACT>
__global__ void __launch_bounds__(kRouteRows) predispatch_kernel(
    const uint16_t* __restrict__ x, int64_t ngroups, const float* __restrict__ gx, uint8_t* __restrict__ xq,
    uint8_t* __restrict__ xsf, const int32_t* __restrict__ ids, int R, int E, int nbits,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_rows,
    int32_t* __restrict__ pos, int tile_rows, int2* __restrict__ tiles, int32_t* __restrict__ num_tiles) {
  const int tid = threadIdx.x;
  if (blockIdx.x > 0) {
    const int64_t g = (int64_t)(blockIdx.x - 1) * kRouteRows + tid;
    if (g < ngroups) {
      if constexpr (ACT == 2)
        quantize_group_nv<true>(x, g, xq, xsf, *gx);
      else
        quantize_group<true, ACT == 1>(x, g, xq, xsf);
    }
    return;
  }
  extern __shared__ int smem[];
  int* wslot = smem;                       // [16][E]: rows of e in wave w, then wave w's next slot of e
  int* wave_tot = wslot + kRouteWaves * E; // [16]
  const int lane = tid & (kWave - 1), w = tid / kWave;
  const int nsub = (R + kRouteRows - 1) / kRouteRows;   // 64-row sub-chunks per wave (<= kPredispatchSubs)
  const int r0 = w * nsub * kWave;
  int eid[kPredispatchSubs];
#pragma unroll
  for (int j = 0; j < kPredispatchSubs; ++j) {
    const int r = r0 + j * kWave + lane;
    const int e = j < nsub && r < R ? ids[r] : -1;
    eid[j] = e >= 0 && e < E ? e : -1;
  }
  for (int i = tid; i < kRouteWaves * E; i += kRouteRows) wslot[i] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPredispatchSubs; ++j)
    if (eid[j] >= 0) atomicAdd(&wslot[w * E + eid[j]], 1);
  __syncthreads();
  int tot = 0;
  if (tid < E)
    for (int ww = 0; ww < kRouteWaves; ++ww) tot += wslot[ww * E + tid];
  const int incl = block_inclusive_scan(tot, wave_tot);   // also orders the reads above before the writes below
  if (tid < E) {
    counts[tid] = tot;
    offsets[tid] = incl - tot;
    if (tid == E - 1) offsets[E] = incl;
    int run = incl - tot;
    for (int ww = 0; ww < kRouteWaves; ++ww) {
      const int c = wslot[ww * E + tid];
      wslot[ww * E + tid] = run;
      run += c;
    }
  }
  if (tile_rows > 0) write_tiles(tot, E, tile_rows, wave_tot, tiles, num_tiles);
  __syncthreads();
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
  int* slot = wslot + w * E;
#pragma unroll
  for (int j = 0; j < kPredispatchSubs; ++j) {
    if (j >= nsub) break;
    const int r = r0 + j * kWave + lane;
    const int e = eid[j];
    const bool valid = e >= 0;
    uint64_t match = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const uint64_t m1 = __ballot(valid && ((e >> bit) & 1));
      match &= ((e >> bit) & 1) ? m1 : ~m1;
    }
    const int rank = __popcll(match & below);
    const int p = valid ? slot[e] + rank : -1;
    // every lane has read its expert's slot before the lowest lane of each
    // expert moves it past this sub-chunk (one wave: LDS accesses in order)
    __builtin_amdgcn_wave_barrier();
    if (valid && rank == 0) slot[e] += __popcll(match);
    __builtin_amdgcn_wave_barrier();
    if (r < R) {
      pos[r] = p;
      if (valid) sorted_rows[p] = r;
    }
  }
}

hipError_t launch_predispatch(int act, const uint16_t* x, int64_t ngroups, const float* gx, uint8_t* xq,
                              uint8_t* xsf, const int32_t* ids, int R, int E, int32_t* counts, int32_t* offsets,
                              int32_t* sorted_rows, int32_t* pos, int tile_rows, int2* tiles, int32_t* num_tiles,
                              hipStream_t stream) {
  const int64_t qblocks = (ngroups + kRouteRows - 1) / kRouteRows;
  const size_t lds = (size_t)(kRouteWaves * E + kRouteWaves) * sizeof(int);
  auto kern = act == 2 ? predispatch_kernel<2> : act == 1 ? predispatch_kernel<1> : predispatch_kernel<0>;
  hipLaunchKernelGGL(kern, dim3((unsigned)(1 + qblocks)), dim3(kRouteRows), lds, stream, x, ngroups, gx, xq, xsf,
                     ids, R, E, id_bits(E), counts, offsets, sorted_rows, pos, tile_rows, tiles, num_tiles);
  return hipGetLastError();
}

}  // namespace moe

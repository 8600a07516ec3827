// Stages S1a + S1b fused in one launch for few routed rows (the pages'
// pre_dispatch: [P3] prhub digest of sglang PR "bump sgl-deep-gemm to 0.1.7,
// MegaMoE uses the mma_type API for MXFP4", "Key source snippets" -- one call
// that packs the tokens to E2M1 with group_size=32 and hands over the top-k ids
// and weights).
//
// Block 0 routes all R <= 8192 rows by itself: every thread reads its (up to 8)
// ids once, then an LDS histogram (integer atomics only count), one block scan
// for counts/offsets (and the tile list), then the rows in chunks of 1024 in
// order, each placed with the in-block stable ranks of route_common.h while a
// running base per expert carries the chunks before it.  Blocks 1.. quantize
// one 32-element group of x per thread meanwhile.
#include "launch.h"
#include "quant_group.h"
#include "route_common.h"

namespace moe {

constexpr int kPredispatchChunks = kPredispatchMaxRows / kRouteRows;

__global__ void __launch_bounds__(kRouteRows) predispatch_kernel(
    const uint16_t* __restrict__ x, int64_t ngroups, uint8_t* __restrict__ xq, uint8_t* __restrict__ xsf,
    const int32_t* __restrict__ ids, int R, int E, int nbits, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_rows, int32_t* __restrict__ pos, int tile_rows,
    int2* __restrict__ tiles, int32_t* __restrict__ num_tiles) {
  const int tid = threadIdx.x;
  if (blockIdx.x > 0) {
    const int64_t g = (int64_t)(blockIdx.x - 1) * kRouteRows + tid;
    if (g < ngroups) quantize_group<true>(x, g, xq, xsf);
    return;
  }
  extern __shared__ int smem[];
  int* base = smem;                        // [E] next free slot of expert e
  int* wcnt = smem + E;                    // [16][E]
  int* wave_tot = wcnt + kRouteWaves * E;  // [16]
  int eid[kPredispatchChunks];
#pragma unroll
  for (int c = 0; c < kPredispatchChunks; ++c) {
    const int r = c * kRouteRows + tid;
    eid[c] = r < R ? ids[r] : -1;
  }
  for (int i = tid; i < E; i += kRouteRows) base[i] = 0;
  for (int i = tid; i < kRouteWaves * E; i += kRouteRows) wcnt[i] = 0;
  __syncthreads();
#pragma unroll
  for (int c = 0; c < kPredispatchChunks; ++c)
    if (eid[c] >= 0 && eid[c] < E) atomicAdd(&base[eid[c]], 1);
  __syncthreads();
  const int tot = tid < E ? base[tid] : 0;
  const int incl = block_inclusive_scan(tot, wave_tot);  // also orders the reads of base above
  if (tid < E) {
    base[tid] = incl - tot;
    counts[tid] = tot;
    offsets[tid] = incl - tot;
    if (tid == E - 1) offsets[E] = incl;
  }
  if (tile_rows > 0) write_tiles(tot, E, tile_rows, wave_tot, tiles, num_tiles);
  __syncthreads();
#pragma unroll
  for (int c = 0; c < kPredispatchChunks; ++c) {
    const int r0 = c * kRouteRows;
    if (r0 >= R) break;
    place_chunk(eid[c], R, E, nbits, r0, base, wcnt, sorted_rows, pos);
    __syncthreads();
    // advance the running bases past this chunk and clear the per-wave counts
    for (int e = tid; e < E; e += kRouteRows) {
      int cnt = 0;
      for (int w = 0; w < kRouteWaves; ++w) {
        cnt += wcnt[w * E + e];
        wcnt[w * E + e] = 0;
      }
      base[e] += cnt;
    }
    __syncthreads();
  }
}

hipError_t launch_predispatch(const uint16_t* x, int64_t ngroups, uint8_t* xq, uint8_t* xsf, const int32_t* ids,
                              int R, int E, int32_t* counts, int32_t* offsets, int32_t* sorted_rows,
                              int32_t* pos, int tile_rows, int2* tiles, int32_t* num_tiles, hipStream_t stream) {
  const int64_t qblocks = (ngroups + kRouteRows - 1) / kRouteRows;
  const size_t lds = (size_t)(E + kRouteWaves * E + kRouteWaves) * sizeof(int);
  hipLaunchKernelGGL(predispatch_kernel, dim3((unsigned)(1 + qblocks)), dim3(kRouteRows), lds, stream, x, ngroups,
                     xq, xsf, ids, R, E, id_bits(E), counts, offsets, sorted_rows, pos, tile_rows, tiles,
                     num_tiles);
  return hipGetLastError();
}

}  // namespace moe

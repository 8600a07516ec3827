// Stage S1b (routing): stable counting sort of the routed rows r = t*k + j by
// expert id, giving counts[E], offsets[E+1], sorted_rows[] and pos[r].
// The pages hand topk_ids/topk_weights to the expert kernel through the
// pre-dispatch buffer ([P3] prhub digest of sglang PR "bump sgl-deep-gemm to
// 0.1.7, MegaMoE uses the mma_type API for MXFP4", "Key source snippets"); the
// ordering (expert, r) is the reading taken for a permutation they leave open.
//
// Deterministic by construction, no order-dependent atomics:
//   kernel 1 (one block per 1024 rows): per-block expert histogram.  Integer
//     LDS atomics only count, so the result does not depend on their order.
//   kernel 2 (same blocks): every block sums the histograms of all blocks and
//     of the blocks before it, scans the totals over experts, and places its
//     rows at offsets[e] + (rows of e in earlier blocks) + (rank in block).
//     The rank inside a wave comes from a 64-lane "match" built from one ballot
//     per id bit; across the 16 waves of a block from per-wave counts in LDS.
#include "device_common.h"
#include "launch.h"

namespace moe {

constexpr int kRouteRows = 1024;   // rows per block, one per thread
constexpr int kRouteWaves = kRouteRows / kWave;

__global__ void __launch_bounds__(kRouteRows) route_hist_kernel(const int32_t* __restrict__ ids, int R,
                                                                int E, int32_t* __restrict__ hist) {
  extern __shared__ int cnt[];
  for (int e = threadIdx.x; e < E; e += kRouteRows) cnt[e] = 0;
  __syncthreads();
  const int r = blockIdx.x * kRouteRows + threadIdx.x;
  if (r < R) {
    const int e = ids[r];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kRouteRows) hist[(size_t)blockIdx.x * E + e] = cnt[e];
}

// Inclusive prefix sum over the 1024 threads of a block.
__device__ __forceinline__ int block_inclusive_scan(int v, int* wave_tot) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(v, d, kWave);
    if (lane >= d) v += o;
  }
  if (lane == kWave - 1) wave_tot[w] = v;
  __syncthreads();
  if (w == 0) {
    int t = lane < kRouteWaves ? wave_tot[lane] : 0;
#pragma unroll
    for (int d = 1; d < kRouteWaves; d <<= 1) {
      const int o = __shfl_up(t, d, kWave);
      if (lane >= d) t += o;
    }
    if (lane < kRouteWaves) wave_tot[lane] = t;   // inclusive over waves
  }
  __syncthreads();
  return v + (w > 0 ? wave_tot[w - 1] : 0);
}

__global__ void __launch_bounds__(kRouteRows) route_scatter_kernel(
    const int32_t* __restrict__ ids, int R, int E, int nbits, int nblocks,
    const int32_t* __restrict__ hist, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_rows, int32_t* __restrict__ pos, int tile_rows, int2* __restrict__ tiles,
    int32_t* __restrict__ num_tiles) {
  extern __shared__ int smem[];
  int* base = smem;                       // [E]   first slot of this block's rows of e
  int* wcnt = smem + E;                   // [16][E] rows of e in each wave of this block
  int* wave_tot = wcnt + kRouteWaves * E; // [16]
  const int tid = threadIdx.x, b = blockIdx.x;

  int tot = 0, before = 0;
  if (tid < E) {
    for (int bb = 0; bb < nblocks; ++bb) {
      const int h = hist[(size_t)bb * E + tid];
      tot += h;
      if (bb < b) before += h;
    }
  }
  for (int i = tid; i < kRouteWaves * E; i += kRouteRows) wcnt[i] = 0;
  const int incl = block_inclusive_scan(tot, wave_tot);
  if (tid < E) {
    base[tid] = incl - tot + before;
    if (b == 0) {
      counts[tid] = tot;
      offsets[tid] = incl - tot;
      if (tid == E - 1) offsets[E] = incl;
    }
  }
  __syncthreads();

  if (b == 0 && tile_rows > 0) {
    // Tile list for the tiled GEMMs: expert e gets ceil(count / tile_rows)
    // consecutive entries (e, 0), (e, tile_rows), ...
    const int nt_e = tid < E ? (tot + tile_rows - 1) / tile_rows : 0;
    const int t_incl = block_inclusive_scan(nt_e, wave_tot);
    for (int i = 0; i < nt_e; ++i) tiles[t_incl - nt_e + i] = make_int2(tid, i * tile_rows);
    if (tid == kRouteRows - 1) *num_tiles = t_incl;
  }

  const int r = b * kRouteRows + tid;
  const int e = r < R ? ids[r] : -1;
  const bool valid = e >= 0 && e < E;
  uint64_t match = __ballot(valid);
  for (int bit = 0; bit < nbits; ++bit) {
    const bool one = valid && ((e >> bit) & 1);
    const uint64_t m1 = __ballot(one);
    match &= ((e >> bit) & 1) ? m1 : ~m1;
  }
  const int lane = tid & (kWave - 1), w = tid / kWave;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
  const int rank_in_wave = __popcll(match & below);
  if (valid && rank_in_wave == 0) wcnt[w * E + e] = __popcll(match);
  __syncthreads();
  if (r < R) {
    if (valid) {
      int rank = rank_in_wave;
      for (int ww = 0; ww < w; ++ww) rank += wcnt[ww * E + e];
      const int p = base[e] + rank;
      pos[r] = p;
      sorted_rows[p] = r;
    } else {
      pos[r] = -1;
    }
  }
}

hipError_t launch_route(const int32_t* ids, int R, int E, int32_t* hist, int32_t* counts,
                        int32_t* offsets, int32_t* sorted_rows, int32_t* pos, int tile_rows, int2* tiles,
                        int32_t* num_tiles, hipStream_t stream) {
  if (R <= 0) return hipSuccess;
  const int nblocks = (R + kRouteRows - 1) / kRouteRows;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  hipLaunchKernelGGL(route_hist_kernel, dim3(nblocks), dim3(kRouteRows), E * sizeof(int), stream, ids,
                     R, E, hist);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t lds = (size_t)(E + kRouteWaves * E + kRouteWaves) * sizeof(int);
  hipLaunchKernelGGL(route_scatter_kernel, dim3(nblocks), dim3(kRouteRows), lds, stream, ids, R, E,
                     nbits, nblocks, hist, counts, offsets, sorted_rows, pos, tile_rows, tiles, num_tiles);
  return hipGetLastError();
}

}  // namespace moe

// Stage S1b (routing), multi-block form for many routed rows: stable counting
// sort of the routed rows r = t*k + j by expert id, giving counts[E],
// offsets[E+1], sorted_rows[] and pos[r] (and the tile list of the tiled
// GEMMs).  The pages hand topk_ids/topk_weights to the expert kernel through the
// pre-dispatch buffer ([P3] prhub digest of sglang PR "bump sgl-deep-gemm to
// 0.1.7, MegaMoE uses the mma_type API for MXFP4", "Key source snippets"); the
// ordering (expert, r) is the reading taken for a permutation they leave open.
//
// Deterministic by construction, no order-dependent atomics:
//   kernel 1 (one block per 1024 rows): per-block expert histogram.  Integer
//     LDS atomics only count, so the result does not depend on their order.
//   kernel 2 (same blocks): every block sums the histograms of all blocks and
//     of the blocks before it (several threads per expert, then an LDS
//     reduction), scans the totals over experts, and places its rows at
//     offsets[e] + (rows of e in earlier blocks) + (rank in block).
#include "launch.h"
#include "route_common.h"

namespace moe {

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

__global__ void __launch_bounds__(kRouteRows) route_scatter_kernel(
    const int32_t* __restrict__ ids, int R, int E, int nbits, int nblocks,
    const int32_t* __restrict__ hist, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_rows, int32_t* __restrict__ pos, int tile_rows, int2* __restrict__ tiles,
    int32_t* __restrict__ num_tiles) {
  extern __shared__ int smem[];
  const int Q = kRouteRows / E;            // threads per expert summing the histograms (E <= 512)
  int* base = smem;                        // [E]   first slot of this block's rows of e
  int* wcnt = smem + E;                    // [16][E] rows of e in each wave of this block
  int* wave_tot = wcnt + kRouteWaves * E;  // [16]
  int* part_tot = wave_tot + kRouteWaves;  // [Q][E] partial sums over every Q-th block
  int* part_bef = part_tot + Q * E;        // [Q][E] the same over the blocks before this one
  const int tid = threadIdx.x, b = blockIdx.x;

  // Thread (q, e) sums the counts of expert e in blocks q, q+Q, ...: Q
  // independent load chains instead of one chain over every block.
  if (tid < Q * E) {
    const int e = tid % E, q = tid / E;
    int t = 0, bf = 0;
#pragma unroll 4
    for (int bb = q; bb < nblocks; bb += Q) {
      const int h = hist[(size_t)bb * E + e];
      t += h;
      bf += bb < b ? h : 0;
    }
    part_tot[q * E + e] = t;
    part_bef[q * E + e] = bf;
  }
  for (int i = tid; i < kRouteWaves * E; i += kRouteRows) wcnt[i] = 0;
  __syncthreads();
  int tot = 0, before = 0;
  if (tid < E) {
    for (int q = 0; q < Q; ++q) {
      tot += part_tot[q * E + tid];
      before += part_bef[q * E + tid];
    }
  }
  const int incl = block_inclusive_scan(tot, wave_tot);
  if (tid < E) {
    base[tid] = incl - tot + before;
    if (b == 0) {
      counts[tid] = tot;
      offsets[tid] = incl - tot;
      if (tid == E - 1) offsets[E] = incl;
    }
  }
  if (b == 0 && tile_rows > 0) write_tiles(tot, E, tile_rows, wave_tot, tiles, num_tiles);
  __syncthreads();
  const int r = b * kRouteRows + tid;
  place_chunk(r < R ? ids[r] : -1, R, E, nbits, b * kRouteRows, base, wcnt, sorted_rows, pos);
}

// One thread per sorted row q < offsets[E]: its token's scale row (dws
// dwords: H/128 for MXFP4, one per K step; H/64 for NVFP4, two per K step) is
// read once and its dword d goes to plane d; the lanes of a wave write
// consecutive dwords of each plane.
__global__ void __launch_bounds__(256) sorted_scales_kernel(const uint8_t* __restrict__ xsf,
                                                            const int32_t* __restrict__ sorted_rows,
                                                            const int32_t* __restrict__ offsets, int E, int dws, int k,
                                                            int hrows, uint32_t* __restrict__ planes) {
  const int q = blockIdx.x * 256 + threadIdx.x;
  if (q >= offsets[E]) return;
  const uint2* src = reinterpret_cast<const uint2*>(xsf + (size_t)(sorted_rows[q] / k) * dws * 4);
  for (int c2 = 0; c2 < dws / 2; ++c2) {   // two dwords per 8-byte load (dws is even)
    const uint2 v = src[c2];
    planes[(size_t)(2 * c2) * hrows + q] = v.x;
    planes[(size_t)(2 * c2 + 1) * hrows + q] = v.y;
  }
}

hipError_t launch_sorted_scales(const uint8_t* xsf, const int32_t* sorted_rows, const int32_t* offsets, int E,
                                int rows_bound, int sc_dwords, int k, int hrows, uint8_t* xsf_planes,
                                hipStream_t stream) {
  if (rows_bound <= 0) return hipSuccess;
  hipLaunchKernelGGL(sorted_scales_kernel, dim3((rows_bound + 255) / 256), dim3(256), 0, stream, xsf, sorted_rows,
                     offsets, E, sc_dwords, k, hrows, reinterpret_cast<uint32_t*>(xsf_planes));
  return hipGetLastError();
}

hipError_t launch_route(const int32_t* ids, int R, int E, int32_t* hist, int32_t* counts,
                        int32_t* offsets, int32_t* sorted_rows, int32_t* pos, int tile_rows, int2* tiles,
                        int32_t* num_tiles, hipStream_t stream) {
  if (R <= 0) return hipSuccess;
  const int nblocks = (R + kRouteRows - 1) / kRouteRows;
  hipLaunchKernelGGL(route_hist_kernel, dim3(nblocks), dim3(kRouteRows), E * sizeof(int), stream, ids,
                     R, E, hist);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t lds = (size_t)(E + kRouteWaves * E + kRouteWaves + 2 * (kRouteRows / E) * E) * sizeof(int);
  hipLaunchKernelGGL(route_scatter_kernel, dim3(nblocks), dim3(kRouteRows), lds, stream, ids, R, E,
                     id_bits(E), nblocks, hist, counts, offsets, sorted_rows, pos, tile_rows, tiles, num_tiles);
  return hipGetLastError();
}

}  // namespace moe

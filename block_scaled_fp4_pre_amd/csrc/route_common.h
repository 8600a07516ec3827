// Building blocks of the routing step (stage S1b): a stable counting sort of
// the routed rows r = t*k + j by expert id, deterministic by construction.
// Used by the multi-block route (route.hip) and by the single-block route of
// the fused pre-dispatch kernel (predispatch.hip).
#pragma once
#include "device_common.h"

namespace moe {

constexpr int kRouteRows = 1024;  // rows per chunk, one per thread of a 1024-thread block
constexpr int kRouteWaves = kRouteRows / kWave;

// Inclusive prefix sum over the 1024 threads of a block (wave_tot: 16 ints of LDS).
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
    if (lane < kRouteWaves) wave_tot[lane] = t;  // inclusive over waves
  }
  __syncthreads();
  const int r = v + (w > 0 ? wave_tot[w - 1] : 0);
  __syncthreads();  // wave_tot may be reused right after
  return r;
}

// Places row r = r0 + threadIdx.x of a chunk of 1024 rows, whose expert id e
// the caller read (-1 past the end): row r of expert e goes to base[e] + (rows
// of e before r in the chunk).  The rank inside a wave comes from a 64-lane
// match (one ballot per id bit), across waves from per-wave counts in
// wcnt[16][E], which must be zero on entry and are left holding the chunk's
// per-wave counts.  Called by all 1024 threads.
__device__ __forceinline__ void place_chunk(int e, int R, int E, int nbits, int r0, const int* base, int* wcnt,
                                            int32_t* __restrict__ sorted_rows, int32_t* __restrict__ pos) {
  const int tid = threadIdx.x;
  const int r = r0 + tid;
  const bool valid = r < R && e >= 0 && e < E;
  uint64_t match = __ballot(valid);
  for (int bit = 0; bit < nbits; ++bit) {
    const uint64_t m1 = __ballot(valid && ((e >> bit) & 1));
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

// Tile list for the tiled GEMMs: expert e (thread e) gets ceil(count / tile_rows)
// consecutive entries (e, 0), (e, tile_rows), ...  Called by all 1024 threads.
__device__ __forceinline__ void write_tiles(int tot, int E, int tile_rows, int* wave_tot, int2* __restrict__ tiles,
                                            int32_t* __restrict__ num_tiles) {
  const int tid = threadIdx.x;
  const int nt_e = tid < E ? (tot + tile_rows - 1) / tile_rows : 0;
  const int t_incl = block_inclusive_scan(nt_e, wave_tot);
  for (int i = 0; i < nt_e; ++i) tiles[t_incl - nt_e + i] = make_int2(tid, i * tile_rows);
  if (tid == kRouteRows - 1) *num_tiles = t_incl;
}

inline int id_bits(int E) {
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  return nbits;
}

}  // namespace moe

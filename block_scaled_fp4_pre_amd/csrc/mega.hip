// The whole forward of the layer in one launch, for decode-sized batches: the
// pages' single fused "mega" MoE kernel ([P1] sglang PR "[deepseek-v4] Bump
// sgl-deep-gemm for packed FP4xFP4 mega-MoE (W4A4)", title and section B,
// where one kernel runs the routed experts' layer).  MXFP4 x MXFP4 and the
// fp8xfp4 MMA type (E4M3 tokens and h, [P3] "Implementation breakdown" items
// 1-3), at most kMegaMaxRows routed rows, hidden and inter each 512, 1024,
// 2048 or 4096 (validate.h).
//
// Stage S1 inside the work items.  Every workgroup routes the T*k ids itself
// (the stable counting sort of route_common.h in LDS, one thread per routed
// row), so no workgroup waits for a routing stage, and the GEMM1 items
// quantize the token rows they need straight from x with the quantize
// kernel's encoder (quant_group.h).
//
// Work items, in two phases:
//   GEMM1 (active expert, W1 unit u of 64 rows): the 4 waves split K into 4
//     slices.  Each wave loads its slice of the unit's weights into VGPRs at
//     once (every load in flight together); the workgroup quantizes the
//     expert's token rows into an LDS tile (kept for the next item when that
//     is of the same expert); each wave runs 4 MFMAs per K step of its slice.
//     The slices' partial sums meet in LDS in a fixed order; wave 0 runs the
//     SwiGLU + requant epilogue (epilogue.h) with agent-scope stores, and
//     once they are complete (one pass later, when the wave has nothing else
//     outstanding) adds one to the expert's h counter.  A GEMM1 item never
//     waits.  A pass takes 16 of the expert's rows (E4M3 tokens: 8, so that
//     the tile of twice the bytes per row keeps its LDS size).
//   GEMM2 (active expert, one or two W2 units v of 64 hidden rows; two from
//     MOE_MEGA_PAIR_ROWS routed rows on, when both 4-step slices fit a wave's
//     registers): the weights as above, loaded before the wait for the
//     expert's h counter to reach its number of GEMM1 items; then each wave's
//     slice of h by agent-scope loads (one operand for both units), the
//     MFMAs, the reduction (wave u sums unit u), and y (bf16) by agent-scope
//     stores.  Once they are complete (again one pass later), one more on
//     each row's (token, v) combine counter; the item that brings it to the
//     token's number of valid slots combines those 64 columns of the token
//     (stage S4), in slot order, as combine.hip does.
// Each phase's items are dealt round-robin over kMegaQueues ticket counters
// (one fetch-and-add per item, spread over as many addresses, since
// same-address atomics from every CU serialize in the memory system).  A
// workgroup starts on the queue of its own index, moves on to the others,
// and takes GEMM2 items only once it has seen every GEMM1 queue run out:
// every GEMM1 item a GEMM2 item waits for has then been handed to a running
// workgroup, whatever order the hardware dispatches workgroups in.
//
// Hand-off between workgroups: the producer stores with the agent-scope
// policy, waits until none of its memory operations is outstanding (vmcnt
// 0: those stores have completed), then adds to the counter with an
// agent-scope atomic; the consumer reads the counter and then the data with
// agent-scope loads.  Data that only moves through agent-scope
// accesses needs no L2 write-back or invalidate.
//
// The state region (queues, counters) must be zero at the launch; the last
// workgroup to finish, found by a two-level count, zeroes it again, so a
// zeroed workspace stays valid for every later call (a replayed graph
// included).  Every wait gives up after poll_limit polls: it sets the error
// word (which the kernel never clears) and the abort word, after which no wait
// waits, so the launch always drains.
#include <climits>

#include "epilogue.h"
#include "gemm_common.h"
#include "launch.h"
#include "quant_group.h"
#include "tiles.h"
#include "validate.h"

namespace moe {
namespace {

constexpr int kMegaThreads = 256;
constexpr int kMegaWaves = kMegaThreads / kWave;   // K slices of a work item
constexpr int kMegaMaxL = 8;                        // K steps per slice, at most (1, 2, 4 or 8)
static_assert(kMegaMaxRows <= kMegaThreads, "one routed row per thread");
static_assert(kMegaMaxK / kStepK <= kMegaWaves * kMegaMaxL, "K slices");

// The state region (validate.h: kMegaStateBytes), in 8-byte words: each
// ticket and done counter on a 128-byte line of its own.
constexpr int kLine = 16;                                   // words per 128 bytes
constexpr int kQueueA = 0;                                  // GEMM1 ticket counters
constexpr int kQueueB = kQueueA + kMegaQueues * kLine;      // GEMM2 ticket counters
constexpr int kDone1 = kQueueB + kMegaQueues * kLine;       // finished workgroups, by blockIdx % kMegaQueues
constexpr int kDone2 = kDone1 + kMegaQueues * kLine;        // finished groups of kDone1
constexpr int kAbort = kDone2 + kLine;                      // nonzero: waits give up at once
constexpr int kErr = kAbort + kLine;                        // nonzero: a wait gave up (never cleared here)
constexpr int kCounters = kErr + kLine;                     // h counters [E], then combine counters
static_assert((uint64_t)(kCounters + kMaxExperts + kMegaMaxRows * (kMegaMaxK / 64)) * 8 <= kMegaStateBytes,
              "state region");
static_assert(kErr == MOE_MEGA_ERR_WORD, "error word documented in moe_w4a4.h");
static_assert(kCounters == MOE_MEGA_HCOUNT_WORD, "h counters documented in moe_w4a4.h");

constexpr int kTokStride = kMegaMaxK / 2 + 16;    // E2M1 tile: 16 rows
constexpr int kTokStride8 = kMegaMaxK + 16;       // E4M3 tile: 8 rows
constexpr int kTscStride = kMegaMaxK / 32 + 4;
static_assert(8 * kTokStride8 <= 16 * kTokStride, "the E4M3 tile fits the E2M1 tile's bytes");
static_assert(2 * (kMegaWaves - 1) * kWave * 16 * 4 <= 16 * kTokStride,
              "GEMM2's partial sums of two units fit the token tile's bytes");

// Token rows of a GEMM1 pass (the LDS tile) and of a GEMM2 pass.
template <bool G1, bool F8>
constexpr int pass_rows() { return G1 && F8 ? 8 : 16; }

struct MegaLds {
  int wcnt[kMegaWaves][kMaxExperts];   // route: rows of each expert per wave
  int off[kMaxExperts + 1];            // sorted position of each expert's first row
  int act[kMaxExperts];                // active experts, ascending
  int sorted[kMegaMaxRows];            // flat row t*k+j at each sorted position
  int pos[kMegaMaxRows];               // sorted position of each flat row, or -1
  int wave_tot[kMegaWaves];
  int nact;
  int item;
  int last;
  int tok_key;                         // (expert, first row) of the token tile, or -1
  float red[kMegaWaves - 1][kWave][16];   // partial sums of the other K slices, one unit per item
  // GEMM1's token tile: 16 quantized token rows of one expert over all of K,
  // rows kTokStride bytes apart (16 bytes of padding put the 16 rows one MFMA
  // operand read touches on distinct banks), and their scale bytes; E4M3: 8
  // rows kTokStride8 bytes apart.
  alignas(16) uint8_t tok[16 * kTokStride];
  uint8_t tsc[16 * kTscStride];
};

__device__ __forceinline__ uint64_t ld_agent(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t add_agent(uint64_t* p, uint64_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Polls *p until it equals want; false after `limit` polls, or as soon as
// the error word *err is set (err may be null), so that once one wait has
// given up the launch drains without waiting again.
__device__ __forceinline__ bool wait_eq(const uint64_t* p, uint64_t want, const uint64_t* err, uint32_t limit) {
  for (uint32_t i = 0; i < limit; ++i) {
    if (ld_agent(p) == want) return true;
    if (err != nullptr && ld_agent(err) != 0) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  return ld_agent(p) == want;
}

struct MegaArgs {
  const uint8_t* w1c;
  const uint8_t* w1s;
  const uint8_t* w2c;
  const uint8_t* w2s;
  const uint16_t* x;
  uint8_t* xq;
  uint8_t* xsf;
  const int32_t* ids;
  const float* tw;
  uint16_t* out;
  uint8_t* hq;
  uint8_t* hsf;
  uint16_t* y;
  uint64_t* state;
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_rows;
  int32_t* pos;
  int T, H, I, E, k, nbits, hrows;
  uint32_t poll_limit;
};

// The workgroup's own route: counts, offsets, the active experts and both
// directions of the permutation, as the route stage computes them.
__device__ void mega_route(const MegaArgs& A, MegaLds& sh) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const int R = A.T * A.k, E = A.E;
  int e = -1;
  if (tid < R) {
    const int id = A.ids[tid];
    e = id >= 0 && id < E ? id : -1;
  }
  for (int i = tid; i < E; i += kMegaThreads)
#pragma unroll
    for (int ww = 0; ww < kMegaWaves; ++ww) sh.wcnt[ww][i] = 0;
  __syncthreads();
  const bool valid = e >= 0;
  uint64_t match = __ballot(valid);
  for (int bit = 0; bit < A.nbits; ++bit) {
    const uint64_t m1 = __ballot(valid && ((e >> bit) & 1));
    match &= ((e >> bit) & 1) ? m1 : ~m1;
  }
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
  const int rank_w = __popcll(match & below);
  if (valid && rank_w == 0) sh.wcnt[w][e] = __popcll(match);
  __syncthreads();
  // Thread t scans experts 2t and 2t+1 (E <= 512): row count in the low 16
  // bits, 1 << 16 per active expert above.
  const int e0 = 2 * tid, e1 = 2 * tid + 1;
  int c0 = 0, c1 = 0;
#pragma unroll
  for (int ww = 0; ww < kMegaWaves; ++ww) {
    if (e0 < E) c0 += sh.wcnt[ww][e0];
    if (e1 < E) c1 += sh.wcnt[ww][e1];
  }
  const int v0 = c0 | (c0 > 0 ? 1 << 16 : 0), v1 = c1 | (c1 > 0 ? 1 << 16 : 0);
  int incl = v0 + v1;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += o;
  }
  if (lane == kWave - 1) sh.wave_tot[w] = incl;
  __syncthreads();
  for (int ww = 0; ww < w; ++ww) incl += sh.wave_tot[ww];
  const int ex0 = incl - v0 - v1, ex1 = ex0 + v0;
  if (e0 < E) {
    sh.off[e0] = ex0 & 0xFFFF;
    if (c0 > 0) sh.act[ex0 >> 16] = e0;
  }
  if (e1 < E) {
    sh.off[e1] = ex1 & 0xFFFF;
    if (c1 > 0) sh.act[ex1 >> 16] = e1;
  }
  if (tid == kMegaThreads - 1) {
    sh.off[E] = incl & 0xFFFF;
    sh.nact = incl >> 16;
  }
  __syncthreads();
  if (tid < R) {
    if (valid) {
      int rank = rank_w;
      for (int ww = 0; ww < w; ++ww) rank += sh.wcnt[ww][e];
      const int p = sh.off[e] + rank;
      sh.pos[tid] = p;
      sh.sorted[p] = tid;
    } else {
      sh.pos[tid] = -1;
    }
  }
  __syncthreads();
}

// Writes the route to the workspace and zeroes the output rows of tokens with
// no valid slot (nothing else writes them).  Called by one workgroup.
__device__ void mega_route_out(const MegaArgs& A, const MegaLds& sh) {
  const int tid = threadIdx.x, R = A.T * A.k;
  for (int e = tid; e <= A.E; e += kMegaThreads) {
    A.offsets[e] = sh.off[e];
    if (e < A.E) A.counts[e] = sh.off[e + 1] - sh.off[e];
  }
  if (tid < R) {
    A.pos[tid] = sh.pos[tid];
    if (tid < sh.off[A.E]) A.sorted_rows[tid] = sh.sorted[tid];
  }
  const int pieces = A.H / 8;
  for (int i = tid; i < A.T * pieces; i += kMegaThreads) {
    const int t = i / pieces;
    bool any = false;
    for (int j = 0; j < A.k; ++j) any |= sh.pos[t * A.k + j] >= 0;
    if (!any) reinterpret_cast<uint4*>(A.out + (size_t)t * A.H)[i - t * pieces] = make_uint4(0, 0, 0, 0);
  }
}

// K-slice w's weights of one unit: all L steps in flight at once.
template <int L>
__device__ __forceinline__ void mega_load_weights(const uint8_t* codes, const uint8_t* scales, int lane,
                                                  uint4 (&a)[L][4], uint32_t (&sa)[L]) {
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(codes, (uint32_t)(L - 1) * kUnitStepStride + kStepCodeBytes);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(scales, (uint32_t)(L - 1) * kUnitScaleStride + kStepScaleBytes);
#pragma unroll
  for (int i = 0; i < L; ++i) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) a[i][rb] = buf_load16(wr, lane * 16 + rb * 1024, i * kUnitStepStride);
    sa[i] = buf_load4(sr, lane * 4, i * kUnitScaleStride);
  }
}

// Sums the K slices of unit u into wave u's acc[u], slice 0 first (wave u's
// own slice enters in its place: fp32 addition commutes).  red: [U][waves -
// 1][kWave][16] floats, wave w's partial sums of unit u in slot w - (w > u).
// Ends with a barrier: waves u < U then own the sums, and the others may go
// on.
template <int U>
__device__ __forceinline__ void mega_reduce(float* red, int w, int lane, v4f (&acc)[U][1][4]) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (w != u) {
      float4* d = reinterpret_cast<float4*>(red + ((u * (kMegaWaves - 1) + w - (w > u)) * kWave + lane) * 16);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
        d[rb] = make_float4(acc[u][0][rb][0], acc[u][0][rb][1], acc[u][0][rb][2], acc[u][0][rb][3]);
    }
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (w == u) {
#pragma unroll
      for (int q = 0; q < kMegaWaves; ++q) {
        if (q == u) continue;
        const float4* s =
            reinterpret_cast<const float4*>(red + ((u * (kMegaWaves - 1) + q - (q > u)) * kWave + lane) * 16);
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const float4 v = s[rb];
          acc[u][0][rb][0] += v.x;
          acc[u][0][rb][1] += v.y;
          acc[u][0][rb][2] += v.z;
          acc[u][0][rb][3] += v.w;
        }
      }
    }
  }
}

// The quantized tokens as the quantize stage writes them (xq [T, H/2], E4M3:
// [T, H]; xsf [T, H/32]), for inspection only: the GEMM1 items quantize
// their own rows.
template <bool F8>
__device__ void mega_tokens_out(const MegaArgs& A) {
  const int groups = A.H / 32;
  for (int i = threadIdx.x; i < A.T * groups; i += kMegaThreads) {
    const int t = i / groups, g = i - t * groups;
    uint32_t w[16];
    load_bf16_words(A.x + (size_t)t * A.H, g, w);
    uint32_t sc;
    if constexpr (F8) {
      uint4 lo, hi;
      sc = mx8_encode_bf16_group(w, lo, hi);
      uint4* d = reinterpret_cast<uint4*>(A.xq + (size_t)t * A.H) + 2 * g;
      d[0] = lo;
      d[1] = hi;
    } else {
      uint4 c;
      sc = mx_encode_bf16_group(w, c);
      reinterpret_cast<uint4*>(A.xq + (size_t)t * (A.H / 2))[g] = c;
    }
    A.xsf[(size_t)t * groups + g] = (uint8_t)sc;
  }
}

// Combines the 64 columns of block v of token t (stage S4, as combine.hip:
// slots in order, fp32 from +0, one rounding to bf16); lane c takes column
// 64v + c.  y by agent-scope loads.
__device__ void mega_combine(const MegaArgs& A, const MegaLds& sh, int t, int v, int lane) {
  const int col = 64 * v + lane;
  float s = 0.f;
  for (int j0 = 0; j0 < A.k; j0 += 4) {
    uint32_t yv[4];
    float wj[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = j0 + q;
      const int pj = j < A.k ? sh.pos[t * A.k + j] : -1;
      wj[q] = pj >= 0 ? A.tw[(size_t)t * A.k + j] : 0.f;
      yv[q] = pj >= 0 ? __hip_atomic_load(A.y + (size_t)pj * A.H + col, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                      : 0u;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = j0 + q;
      if (j < A.k && sh.pos[t * A.k + j] >= 0) s += wj[q] * bf16_to_f32(yv[q]);
    }
  }
  A.out[(size_t)t * A.H + col] = (uint16_t)f32_to_bf16(s);
}

// Issues this wave's weight loads of item i: expert act[i / N], units
// (i % N) * U .. + U - 1, the wave's K slice of each.
template <bool G1, int U, int L>
__device__ __forceinline__ void mega_item_weights(const MegaArgs& A, const MegaLds& sh, int i, int N, int w,
                                                  int lane, uint4 (&a)[U][L][4], uint32_t (&sa)[U][L]) {
  const int e = sh.act[i / N], unit0 = (i % N) * U, s0 = w * L;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if constexpr (G1)
      mega_load_weights<L>(A.w1c + w1_code_offset(e, unit0 + u, s0, A.H, A.I),
                           A.w1s + w1_scale_offset(e, unit0 + u, s0, A.H, A.I), lane, a[u], sa[u]);
    else
      mega_load_weights<L>(A.w2c + w2_code_offset(e, unit0 + u, s0, A.H, A.I),
                           A.w2s + w2_scale_offset(e, unit0 + u, s0, A.H, A.I), lane, a[u], sa[u]);
  }
}

// GEMM1's token tile for a pass over the sorted rows p0 .. p0 + nrows - 1:
// the rows of x quantized by the workgroup with the quantize stage's encoder
// (quant_group.h) into LDS, 16 rows over all of K (rows kTokStride bytes
// apart, 16 bytes of padding putting the 16 rows one MFMA operand read
// touches on distinct banks; scale bytes kTscStride apart); E4M3: 8 rows,
// kTokStride8 bytes apart, element order.  The tile is kept while the pass
// stays the same (key: its first sorted row).  All threads call it.
template <bool F8>
__device__ __forceinline__ void mega_token_tile(const MegaArgs& A, MegaLds& sh, int p0, int nrows) {
  if (sh.tok_key == p0) return;
  const int groups = A.H / 32;
  for (int i = threadIdx.x; i < nrows * groups; i += kMegaThreads) {
    const int r = i / groups, g = i - r * groups;
    uint32_t w[16];
    load_bf16_words(A.x + (size_t)(sh.sorted[p0 + r] / A.k) * A.H, g, w);
    if constexpr (F8) {
      uint4 lo, hi;
      sh.tsc[r * kTscStride + g] = (uint8_t)mx8_encode_bf16_group(w, lo, hi);
      uint4* d = reinterpret_cast<uint4*>(sh.tok + r * kTokStride8 + g * 32);
      d[0] = lo;
      d[1] = hi;
    } else {
      uint4 c;
      sh.tsc[r * kTscStride + g] = (uint8_t)mx_encode_bf16_group(w, c);
      *reinterpret_cast<uint4*>(sh.tok + r * kTokStride + g * 16) = c;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) sh.tok_key = p0;   // read again only after a later barrier
}

// The 16 code bytes at p and the scale byte kb of the dword at s4, by
// agent-scope loads.
__device__ __forceinline__ void ld_operand(const uint8_t* p, const uint8_t* s4, int kb, uint4& b, uint32_t& sb) {
  const uint64_t* c = reinterpret_cast<const uint64_t*>(p);
  const uint64_t lo = ld_agent(c), hi = ld_agent(c + 1);
  b = make_uint4((uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32));
  const uint32_t w = __hip_atomic_load(reinterpret_cast<const uint32_t*>(s4), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  sb = (w >> (8 * kb)) & 0xFFu;
}

// The E4M3 operand of lane group kb in the 128-byte step row at p (elements
// [16kb, 16kb+16) and [64+16kb, 64+16kb+16), device_common.h) and its scale
// byte, by agent-scope loads.
__device__ __forceinline__ void ld_operand8(const uint8_t* p, const uint8_t* s4, int kb, uint4& lo, uint4& hi,
                                            uint32_t& sb) {
  const uint64_t* c = reinterpret_cast<const uint64_t*>(p + kb * 16);
  const uint64_t a0 = ld_agent(c), a1 = ld_agent(c + 1), b0 = ld_agent(c + 8), b1 = ld_agent(c + 9);
  lo = make_uint4((uint32_t)a0, (uint32_t)(a0 >> 32), (uint32_t)a1, (uint32_t)(a1 >> 32));
  hi = make_uint4((uint32_t)b0, (uint32_t)(b0 >> 32), (uint32_t)b1, (uint32_t)(b1 >> 32));
  const uint32_t w = __hip_atomic_load(reinterpret_cast<const uint32_t*>(s4), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  sb = (w >> (8 * kb)) & 0xFFu;
}

// One pass of a wave over its K slice (from step s0), rows p0 .. p0 + nrows
// - 1 (row min(r, nrows - 1) for lane row r: rows past the expert's last
// re-read it, their results are not stored): per step the token operand, then
// 4 MFMAs (one per 16-row weight block).  GEMM1: the operand from the LDS
// token tile.  GEMM2: h by agent-scope loads (K-step planes of hrows rows,
// epilogue.h).  F8: E4M3 operands of 32 bytes a lane (the FP8 MFMA form).
template <bool G1, bool F8, int U, int L>
__device__ __forceinline__ void mega_pass(const MegaArgs& A, const MegaLds& sh, int p0, int nrows, int s0,
                                          int lane, const uint4 (&a)[U][L][4], const uint32_t (&sa)[U][L],
                                          v4f (&acc)[U][1][4]) {
  const int r = lane & 15, kb = lane >> 4;
  const int rr = min(r, nrows - 1);
  const size_t pp = (size_t)s0 * A.hrows + p0 + rr;
#pragma unroll
  for (int u = 0; u < U; ++u) zero_acc<1>(acc[u]);
#pragma unroll
  for (int i = 0; i < L; ++i) {
    uint32_t sb;
    if constexpr (F8) {
      uint4 lo, hi;
      if constexpr (G1) {
        const uint8_t* row = sh.tok + rr * kTokStride8 + (s0 + i) * 128 + kb * 16;
        lo = *reinterpret_cast<const uint4*>(row);
        hi = *reinterpret_cast<const uint4*>(row + 64);
        sb = sh.tsc[rr * kTscStride + (s0 + i) * 4 + kb];
      } else {
        const size_t pr = pp + (size_t)i * A.hrows;
        ld_operand8(A.hq + pr * 128, A.hsf + pr * 4, kb, lo, hi, sb);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        acc[u][0][0] = mfma_fp4_fp8<0, 0>(a[u][i][0], lo, hi, acc[u][0][0], (int)sa[u][i], (int)sb);
        acc[u][0][1] = mfma_fp4_fp8<1, 0>(a[u][i][1], lo, hi, acc[u][0][1], (int)sa[u][i], (int)sb);
        acc[u][0][2] = mfma_fp4_fp8<2, 0>(a[u][i][2], lo, hi, acc[u][0][2], (int)sa[u][i], (int)sb);
        acc[u][0][3] = mfma_fp4_fp8<3, 0>(a[u][i][3], lo, hi, acc[u][0][3], (int)sa[u][i], (int)sb);
      }
    } else {
      uint4 b;
      if constexpr (G1) {
        b = *reinterpret_cast<const uint4*>(sh.tok + rr * kTokStride + (s0 + i) * 64 + kb * 16);
        sb = sh.tsc[rr * kTscStride + (s0 + i) * 4 + kb];
      } else {
        const size_t pr = pp + (size_t)i * A.hrows;
        ld_operand(A.hq + pr * 64 + kb * 16, A.hsf + pr * 4, kb, b, sb);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        acc[u][0][0] = mfma_fp4<0, 0>(a[u][i][0], b, acc[u][0][0], (int)sa[u][i], (int)sb);
        acc[u][0][1] = mfma_fp4<1, 0>(a[u][i][1], b, acc[u][0][1], (int)sa[u][i], (int)sb);
        acc[u][0][2] = mfma_fp4<2, 0>(a[u][i][2], b, acc[u][0][2], (int)sa[u][i], (int)sb);
        acc[u][0][3] = mfma_fp4<3, 0>(a[u][i][3], b, acc[u][0][3], (int)sa[u][i], (int)sb);
      }
    }
  }
}

// Wave 0's end of a pass: GEMM1's SwiGLU + requant epilogue (h) or GEMM2's
// y, by agent-scope stores.  Their completion is waited for later
// (mega_publish), when the wave has nothing else outstanding.
template <bool G1, bool F8>
__device__ __forceinline__ void mega_epilogue(const MegaArgs& A, int unit, int p0, int nrows, int lane,
                                              v4f (&acc)[1][4]) {
  if constexpr (G1)
    gemm1_epilogue<1, F8, CoherentStore>(acc, unit, p0, nrows, A.I, A.hrows, lane, A.hq, A.hsf, nullptr);
  else
    gemm2_epilogue<1, CoherentStore>(acc, unit, p0, nrows, A.H, lane, A.y);
}

// Wave w (< U)'s epilogue: that of unit w of the item, whose sums it holds.
template <bool G1, bool F8, int U>
__device__ __forceinline__ void mega_epilogue_u(const MegaArgs& A, int unit, int p0, int nrows, int w, int lane,
                                                v4f (&acc)[U][1][4]) {
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (w == u) mega_epilogue<G1, F8>(A, unit, p0, nrows, lane, acc[u]);
}

// What wave 0 still owes for the stores of an earlier pass: the expert's h
// counter (GEMM1, once per item), or the combine counters of the pass's rows
// (GEMM2: unit v, sorted rows p0 .. p0 + nrows - 1).  Published once the
// wave has waited for all its memory operations, one pass later, so that no
// wave waits for a store's completion on the item's critical path.
struct MegaPending {
  int e = -1, unit = 0, p0 = 0, nrows = 0;
  int tok = 0;        // GEMM2, lane r < nrows (kb == 0): the row's token
  uint64_t old = 0;   //   and the combine counter's value before this row's count
  bool counted = false;
};

// First half of a publication (wave 0): wait for every outstanding memory
// operation of the wave (the pending stores included), then count.  GEMM1
// adds one to the expert's h counter; GEMM2 adds one to each row's (token,
// block) combine counter, keeping the old values for mega_publish_end.
template <bool G1>
__device__ __forceinline__ void mega_publish(const MegaArgs& A, const MegaLds& sh, MegaPending& pd, int lane) {
  if (pd.e < 0) return;
  wait_vmem_all();
  if constexpr (G1) {
    if (lane == 0) add_agent(A.state + kCounters + pd.e, 1);
    pd.e = -1;
  } else {
    const int r = lane & 15, kb = lane >> 4;
    pd.counted = r < pd.nrows && kb == 0;
    if (pd.counted) {
      pd.tok = sh.sorted[pd.p0 + r] / A.k;
      pd.old = add_agent(A.state + kCounters + A.E + (size_t)pd.tok * (A.H / 64) + pd.unit, 1);
    }
  }
}

// Second half (GEMM2): the tokens whose last row this was get their block
// combined.
template <bool G1>
__device__ __forceinline__ void mega_publish_end(const MegaArgs& A, const MegaLds& sh, MegaPending& pd,
                                                 int lane) {
  if constexpr (!G1) {
    if (pd.e < 0) return;
    bool last = false;
    if (pd.counted) {
      int nvalid = 0;
      for (int j = 0; j < A.k; ++j) nvalid += sh.pos[pd.tok * A.k + j] >= 0;
      last = (int)pd.old + 1 == nvalid;
    }
    uint64_t m = __ballot(last);
    while (m) {
      const int src = __ffsll((long long)m) - 1;
      m &= m - 1;
      mega_combine(A, sh, __shfl(pd.tok, src, kWave), pd.unit, lane);
    }
    pd.e = -1;
  }
}

// One queue of a phase (the counter at ctr hands out items q, q +
// kMegaQueues, ... below n), pipelined: the next item's ticket is taken while
// the current item runs, and each wave issues the next item's weights as soon
// as its MFMAs have consumed the current ones, before the epilogue.  An item
// covers U weight units (GEMM2: 1 or 2); wave u < U reduces unit u, runs its
// epilogue and publishes it.
template <bool G1, bool F8, int U, int L>
__device__ void mega_queue(const MegaArgs& A, MegaLds& sh, uint64_t* ctr, int q, int n) {
  constexpr int P = pass_rows<G1, F8>();
  static_assert(U == 1 || (!G1 && U == 2), "two units per item: GEMM2 only");
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int N = G1 ? A.I / 32 : A.H / 64 / U, s0 = w * L;
  // Partial sums of the K slices: GEMM2 with two units puts them in the
  // token tile's bytes, which only GEMM1 uses.
  float* red = U == 1 ? &sh.red[0][0][0] : reinterpret_cast<float*>(sh.tok);
  if (tid == 0) sh.item = (int)min(add_agent(ctr, 1) * kMegaQueues + q, (uint64_t)INT_MAX);
  __syncthreads();
  int cur = sh.item;
  __syncthreads();
  if (cur >= n) return;
  uint4 a[U][L][4];
  uint32_t sa[U][L];
  mega_item_weights<G1, U, L>(A, sh, cur, N, w, lane, a, sa);
  MegaPending pd;   // waves u < U: unit u's
  // GEMM2: the next item's h counter, read as soon as the item is known; a
  // count already complete spares the wait's first load
  uint64_t hc_next = 0;
  for (;;) {
    uint64_t next_raw = 0;
    if (tid == 0) next_raw = add_agent(ctr, 1);
    // An opaque copy of the lane index per item: the lane-derived addresses
    // are recomputed here instead of being hoisted out of the loops and held
    // (or spilled) across them.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int e = sh.act[cur / N], unit = (cur % N) * U + min(w, U - 1);   // the wave's unit, if it has one
    const int base = sh.off[e], n_e = sh.off[e + 1] - base;
    if constexpr (!G1) {
      // h of the expert is complete once each of its I/32 GEMM1 items has
      // counted (counts only grow within a launch)
      if (hc_next != (uint64_t)(A.I / 32) &&
          !wait_eq(A.state + kCounters + e, (uint64_t)(A.I / 32), A.state + kAbort, A.poll_limit) && ln == 0) {
        st_agent(A.state + kErr, 1);
        st_agent(A.state + kAbort, 1);
      }
    }
    int nxt = INT_MAX;
    for (int t0 = 0; t0 < n_e; t0 += P) {
      const int nrows = min(P, n_e - t0);
      const bool last = t0 + P >= n_e;
      if constexpr (G1) mega_token_tile<F8>(A, sh, base + t0, nrows);
      v4f acc[U][1][4];
      mega_pass<G1, F8, U, L>(A, sh, base + t0, nrows, s0, ln, a, sa, acc);
      // The previous pass's stores are long done: waves u < U publish them
      // while the other waves reach the reduction.
      if (w < U) mega_publish<G1>(A, sh, pd, ln);
      if (last && tid == 0) sh.item = (int)min(next_raw * kMegaQueues + q, (uint64_t)INT_MAX);
      mega_reduce<U>(red, w, ln, acc);   // a barrier: sh.item is published
      if (last) nxt = sh.item;
      if constexpr (!G1) {
        if (last && nxt < n) hc_next = ld_agent(A.state + kCounters + sh.act[nxt / N]);
      }
      // (Separate paths for "no next item" and "next item", each loading the
      // weights unconditionally, so that the spent weights are dead during
      // the epilogue instead of being kept for a merge with the new ones.)
      if (last && nxt >= n) {
        if (w < U) {
          mega_epilogue_u<G1, F8, U>(A, unit, base + t0, nrows, w, ln, acc);
          mega_publish_end<G1>(A, sh, pd, ln);
          pd.e = e, pd.unit = unit, pd.p0 = base + t0, pd.nrows = nrows;
          mega_publish<G1>(A, sh, pd, ln);   // the queue's last: published at once
          mega_publish_end<G1>(A, sh, pd, ln);
        }
        __syncthreads();
        return;
      }
      if (w < U) {
        mega_epilogue_u<G1, F8, U>(A, unit, base + t0, nrows, w, ln, acc);
        mega_publish_end<G1>(A, sh, pd, ln);
        if (!G1 || last) pd.e = e, pd.unit = unit, pd.p0 = base + t0, pd.nrows = nrows;
        if (last) mega_item_weights<G1, U, L>(A, sh, nxt, N, w, ln, a, sa);
      } else if (last) {
        mega_item_weights<G1, U, L>(A, sh, nxt, N, w, ln, a, sa);
      }
      __syncthreads();   // the partial sums' LDS and sh.item are free again
    }
    cur = nxt;
  }
}

// Takes the items of one phase (n of them, item i on queue i % kMegaQueues)
// until every queue has run out: first the workgroup's own queue, then,
// after one read of all the queue counters at once, any queue still open.
template <bool G1, bool F8, int U, int L>
__device__ void mega_phase(const MegaArgs& A, MegaLds& sh, uint64_t* q0, int n) {
  const int tid = threadIdx.x;
  int q = blockIdx.x % kMegaQueues;
  for (;;) {
    mega_queue<G1, F8, U, L>(A, sh, q0 + q * kLine, q, n);
    if (tid < kWave) {
      const bool open = tid < kMegaQueues && ld_agent(q0 + tid * kLine) * kMegaQueues + tid < (uint64_t)n;
      const uint64_t m = __ballot(open);
      if (tid == 0) sh.item = (int)m;
    }
    __syncthreads();
    const uint32_t mask = (uint32_t)sh.item;
    __syncthreads();
    if (mask == 0) break;
    // the next open queue after q, cyclically
    const uint32_t rot = ((mask >> (q + 1)) | (mask << (kMegaQueues - q - 1))) & ((1u << kMegaQueues) - 1);
    q = (q + 1 + __builtin_ctz(rot)) % kMegaQueues;
  }
}

}  // namespace

// One kernel per token format, K-slice lengths (L1 = H / 512 steps for
// GEMM1, L2 = I / 512 for GEMM2) and W2 units per GEMM2 item (U2), so that
// each holds only its own two phase bodies and their registers.
template <bool F8, int L1, int L2, int U2>
__global__ void __launch_bounds__(kMegaThreads, 2) mega_moe_kernel(MegaArgs A) {
  __shared__ MegaLds sh;
  const int tid = threadIdx.x;
  mega_route(A, sh);
  if (tid == 0) sh.tok_key = -1;   // ordered before its first read by the barriers of the phases
  if (blockIdx.x == 0) {
    mega_route_out(A, sh);
    mega_tokens_out<F8>(A);
  }
  mega_phase<true, F8, 1, L1>(A, sh, A.state + kQueueA, sh.nact * (A.I / 32));
  mega_phase<false, F8, U2, L2>(A, sh, A.state + kQueueB, sh.nact * (A.H / 64 / U2));

  // Two-level count of finished workgroups; the last one zeroes the state.
  if (tid == 0) {
    wait_vmem_all();   // this workgroup's counter updates are done
    const int g = blockIdx.x % kMegaQueues;
    const int in_group = (int)(gridDim.x / kMegaQueues) + (g < (int)(gridDim.x % kMegaQueues) ? 1 : 0);
    const int groups = min((int)gridDim.x, kMegaQueues);
    int last = 0;
    if ((int)add_agent(A.state + kDone1 + g * kLine, 1) + 1 == in_group)
      last = (int)add_agent(A.state + kDone2, 1) + 1 == groups;
    sh.last = last;
  }
  __syncthreads();
  if (sh.last) {
    const int nwords = kCounters + A.E + (kMegaMaxRows / A.k) * (A.H / 64);
    for (int i = tid; i < nwords; i += kMegaThreads)
      if (i != kErr) st_agent(A.state + i, 0);
  }
}

namespace {
// Workgroups per launch of each kernel on each device: CUs x resident
// workgroups per CU.
int g_mega_grid[2][4][4][2][64];

int log2_slice(int steps) { return steps >= 8 ? 3 : steps >= 4 ? 2 : steps >= 2 ? 1 : 0; }

// Two W2 units per GEMM2 item (twice the weights per item, half the items)
// from this many routed rows on, when the wave's two slices fit its
// registers (at most 4 steps each: inter up to 2048).
#ifndef MOE_MEGA_PAIR_ROWS
#define MOE_MEGA_PAIR_ROWS 24
#endif

template <bool F8, int L1>
const void* mega_kernel_l2(int l2, bool pair) {
  switch (l2) {
    case 3: return reinterpret_cast<const void*>(mega_moe_kernel<F8, L1, 8, 1>);
    case 2: return pair ? reinterpret_cast<const void*>(mega_moe_kernel<F8, L1, 4, 2>)
                        : reinterpret_cast<const void*>(mega_moe_kernel<F8, L1, 4, 1>);
    case 1: return pair ? reinterpret_cast<const void*>(mega_moe_kernel<F8, L1, 2, 2>)
                        : reinterpret_cast<const void*>(mega_moe_kernel<F8, L1, 2, 1>);
    default: return pair ? reinterpret_cast<const void*>(mega_moe_kernel<F8, L1, 1, 2>)
                         : reinterpret_cast<const void*>(mega_moe_kernel<F8, L1, 1, 1>);
  }
}

template <bool F8>
const void* mega_kernel_l1(int l1, int l2, bool pair) {
  switch (l1) {
    case 3: return mega_kernel_l2<F8, 8>(l2, pair);
    case 2: return mega_kernel_l2<F8, 4>(l2, pair);
    case 1: return mega_kernel_l2<F8, 2>(l2, pair);
    default: return mega_kernel_l2<F8, 1>(l2, pair);
  }
}
}  // namespace

hipError_t launch_mega(const uint8_t* w1c, const uint8_t* w1s, const uint8_t* w2c, const uint8_t* w2s,
                       const uint16_t* x, const int32_t* ids, const float* tw, uint16_t* out, int T, int H, int I,
                       int E, int k, int hrows, uint8_t* xq, uint8_t* xsf, uint8_t* hq, uint8_t* hsf, uint16_t* y,
                       uint64_t* state, int32_t* counts, int32_t* offsets, int32_t* sorted_rows, int32_t* pos,
                       bool f8, uint32_t poll_limit, hipStream_t stream) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  const int l1 = log2_slice(H / kStepK / kMegaWaves), l2 = log2_slice(I / kStepK / kMegaWaves);
  const bool pair = l2 < 3 && T * k >= MOE_MEGA_PAIR_ROWS;
  const void* kern = f8 ? mega_kernel_l1<true>(l1, l2, pair) : mega_kernel_l1<false>(l1, l2, pair);
  int* cached = &g_mega_grid[f8][l1][l2][pair][dev < 64 ? dev : 0];
  int grid = dev < 64 ? __atomic_load_n(cached, __ATOMIC_RELAXED) : 0;
  if (grid == 0) {
    int cus = 0, per_cu = 0;
    err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
    err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kMegaThreads, 0);
    if (err != hipSuccess) return err;
    grid = cus * (per_cu > 0 ? per_cu : 1);
    if (dev < 64) __atomic_store_n(cached, grid, __ATOMIC_RELAXED);
  }
  const int R = T * k;
  const int64_t items = (int64_t)(R < E ? R : E) * (I / 32);
  if (items < grid) grid = (int)items;
  if (grid < 1) grid = 1;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  MegaArgs A{w1c, w1s, w2c, w2s, x, xq, xsf, ids, tw, out, hq, hsf, y, state, counts, offsets, sorted_rows, pos,
             T, H, I, E, k, nbits, hrows, poll_limit};
  void* args[] = {&A};
  err = hipLaunchKernel(kern, dim3(grid), dim3(kMegaThreads), args, 0, stream);
  if (err != hipSuccess) return err;
  return hipGetLastError();
}

}  // namespace moe

// Stages S2 / S3 for many rows per expert (prefill): tiled grouped GEMMs.
//
// [P1] sglang PR "[deepseek-v4] Bump sgl-deep-gemm for packed FP4xFP4 mega-MoE
// (W4A4)", Appendix A (prefill sweep with 1024-token inputs) and section B
// (the fused layer on packed FP4 operands); [P3] prhub digest of sglang PR
// "bump sgl-deep-gemm to 0.1.7, MegaMoE uses the mma_type API for MXFP4", "Key
// source snippets" (activation="swiglu", gate rows then up rows in W1).
//
// Work is a list of tiles (expert e, first row t0) of up to NT*16 routed rows,
// written by the route kernel, crossed with the expert's weight blocks (GEMM1:
// 128 inter columns = 4 units of 64 gate/up rows; GEMM2: 256 hidden rows = 4
// units of 64 rows).  Every tile has the same size, so a hot expert becomes
// many equal work items instead of one long one.
//
// Block order: logical id L = (blockIdx % 8) * (grid / 8) + blockIdx / 8, and
// L runs weight-block-major, tile-minor.  Blocks are dealt round-robin to the 8
// XCDs, so each XCD gets a contiguous range of L: the tiles that share a
// weight block run on one XCD at about the same time and that weight block is
// fetched from HBM once into that XCD's L2.
//
// Per workgroup (WH groups of 4 waves; the groups run the same 4 weight units,
// one unit per wave, on different NT*16-row parts of the tile, so each weight
// byte a group fetches is reused by the other group through L1/L2 while every
// wave keeps only NT*16 accumulator columns): the token operand is staged through
// LDS in chunks of CK K-steps, double-buffered: every thread loads its share of
// chunk c+2 into registers while chunk c+1 is computed from LDS, then stores it
// into the free buffer at the chunk boundary (one barrier per chunk).  Weights
// stream HBM/L2 -> VGPR through the D-slot buffer-load ring of gemm_common.h.
#include "epilogue.h"
#include "gemm_common.h"
#include "launch.h"
#include "tiles.h"

namespace moe {

// Position of 16-byte piece c of staged row n (CHUNKS pieces per row): the 16
// rows read by one MFMA operand load fall on 16 different 16-byte bank groups.
template <int CHUNKS>
__device__ __forceinline__ int stage_pos(int n, int c) {
  if constexpr (CHUNKS >= 16)
    return c ^ (n & 15);
  else
    return c ^ ((n / (16 / CHUNKS)) & (CHUNKS - 1));
}

#ifndef MOE_TILED_GROUP
#define MOE_TILED_GROUP 0        // 0: weight-block-major order; g > 0: tile groups of g, blocks inside
#endif
#ifndef MOE_TILED_MIN_BLOCKS
#define MOE_TILED_MIN_BLOCKS 2   // 4-wave groups per CU the register budget must allow
#endif

template <bool G1, int NT, int D, int CK, int WH>
__global__ void __launch_bounds__(256 * WH, (MOE_TILED_MIN_BLOCKS / WH) > 0 ? MOE_TILED_MIN_BLOCKS / WH : 1)
    gemm_tiled_kernel(
    const uint8_t* __restrict__ wc, const uint8_t* __restrict__ wsc, const uint8_t* __restrict__ act,
    const uint8_t* __restrict__ act_sf, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_rows,
    const int2* __restrict__ tiles, const int32_t* __restrict__ num_tiles, int max_tiles, int H, int I,
    int k, uint8_t* __restrict__ hq, uint8_t* __restrict__ hsf, float* __restrict__ acc_out,
    uint16_t* __restrict__ y) {
  constexpr int THREADS = 256 * WH;                 // WH groups of 4 waves
  constexpr int ROWS = NT * 16 * WH;                // tile rows; each wave group takes NT*16
  constexpr int CHUNKS = CK * 4;                    // 16-byte pieces per row per chunk
  constexpr int CODE_BYTES = ROWS * CHUNKS * 16;    // one buffer of codes
  constexpr int SC_BYTES = ROWS * CK * 4;           // one buffer of scale bytes
  constexpr int PIECES = ROWS * CHUNKS;             // 16-byte code pieces per chunk
  constexpr int PPT = (PIECES + THREADS - 1) / THREADS;  // per thread (the last may be idle)
  constexpr int U = D > CK ? D : CK;
  static_assert(ROWS * CK <= THREADS, "one scale dword per thread");
  static_assert(D % CK == 0 || CK % D == 0, "ring depth and chunk length must nest");

  const int K = G1 ? H : I;
  const int nwb = G1 ? I / 128 : H / 256;
  const int G = gridDim.x;
  const int L = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  int wb, ti;
  if constexpr (MOE_TILED_GROUP == 0) {
    wb = L / max_tiles;                        // weight-block-major over all tiles
    ti = L - wb * max_tiles;
  } else {
    // groups of MOE_TILED_GROUP consecutive tiles, weight blocks inside a group
    constexpr int TG = MOE_TILED_GROUP;
    const int grp = L / (TG * nwb), r = L - grp * (TG * nwb);
    wb = r / TG;
    ti = grp * TG + (r - wb * TG);
  }
  if (wb >= nwb || ti >= *num_tiles) return;
  const int2 tile = tiles[ti];
  const int e = tile.x, t0 = tile.y;
  const int nrows = min(ROWS, counts[e] - t0);
  const int row0 = offsets[e] + t0;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int unit = wb * 4 + (wave & 3);        // wave groups share the 4 weight units
  const int half = wave >> 2;                  // ... and split the tile's rows
  const int hrow0 = half * NT * 16;
  const int S = K / kStepK;
  const int nchunks = S / CK;
  const int row_bytes = K / 2, sc_row = K / 32;

  extern __shared__ __align__(16) uint8_t lds[];
  uint8_t* codes_buf = lds;                    // [2][ROWS][CHUNKS*16]
  uint8_t* sc_buf = lds + 2 * CODE_BYTES;      // [2][ROWS][CK*4]

  const size_t wco = G1 ? w1_code_offset(e, unit, 0, H, I) : w2_code_offset(e, unit, 0, H, I);
  const size_t wso = G1 ? w1_scale_offset(e, unit, 0, H, I) : w2_scale_offset(e, unit, 0, H, I);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(wc + wco, (uint32_t)S * kStepCodeBytes);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(wsc + wso, (uint32_t)S * kStepScaleBytes);
  const int voff = lane * 16, svoff = lane * 4;
  const int tok_lane = lane & 15, kb = lane >> 4;

  uint4 a[D][4];
  uint32_t sa[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) a[d][rb] = buf_load16<kPolicyDefault>(wr, voff + rb * 1024, d * kStepCodeBytes);
    sa[d] = buf_load4<kPolicyDefault>(sr, svoff, d * kStepScaleBytes);
  }

  // Fixed staging assignment: thread piece i = row n, piece c of every chunk.
  auto src_row = [&](int n) -> int {
    if (n >= nrows) return -1;
    return G1 ? sorted_rows[row0 + n] / k : row0 + n;
  };
  int src_off[PPT], dst_off[PPT];
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const int p = tid + i * THREADS;
    const int n = p / CHUNKS, c = p - (p / CHUNKS) * CHUNKS;
    const int r = p < PIECES ? src_row(n) : -1;
    src_off[i] = r < 0 ? -1 : r * row_bytes + c * 16;
    dst_off[i] = p < PIECES ? n * (CHUNKS * 16) + stage_pos<CHUNKS>(n, c) * 16 : -1;
  }
  int sc_src = -1;
  const int sc_dst = tid * 4;                  // row n = tid / CK, step q = tid % CK
  if (tid < ROWS * CK) {
    const int r = src_row(tid / CK);
    sc_src = r < 0 ? -1 : r * sc_row + (tid % CK) * 4;
  }
  uint4 stg[PPT];
  uint32_t stg_sc = 0;
  auto load_chunk = [&](int c) {
#pragma unroll
    for (int i = 0; i < PPT; ++i)
      stg[i] = src_off[i] < 0 ? make_uint4(0, 0, 0, 0)
                              : *reinterpret_cast<const uint4*>(act + src_off[i] + c * (CK * 64));
    stg_sc = sc_src < 0 ? 0u : *reinterpret_cast<const uint32_t*>(act_sf + sc_src + c * (CK * 4));
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PPT; ++i)
      if (dst_off[i] >= 0) *reinterpret_cast<uint4*>(codes_buf + buf * CODE_BYTES + dst_off[i]) = stg[i];
    if (tid < ROWS * CK) *reinterpret_cast<uint32_t*>(sc_buf + buf * SC_BYTES + sc_dst) = stg_sc;
  };

  load_chunk(0);
  store_chunk(0);
  if (nchunks > 1) load_chunk(1);
  __syncthreads();

  v4f acc[NT][4];
  zero_acc<NT>(acc);
  // Steady state without branches on the weight ring: U divides S, and the
  // loads issued past the last step fall outside the buffer range (zeros).
  for (int j0 = 0; j0 < S; j0 += U) {
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      const int j = j0 + uu;
      const int slot = uu % D;
      const int q = uu % CK;                   // step within the chunk (j0 is a multiple of CK)
      const int chunk = j / CK;
      const uint8_t* cb = codes_buf + (chunk & 1) * CODE_BYTES;
      const uint8_t* sb = sc_buf + (chunk & 1) * SC_BYTES;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int n = hrow0 + nt * 16 + tok_lane;
        const uint4 b =
            *reinterpret_cast<const uint4*>(cb + n * (CHUNKS * 16) + stage_pos<CHUNKS>(n, q * 4 + kb) * 16);
        const int bs = sb[n * (CK * 4) + q * 4 + kb];
        acc[nt][0] = mfma_fp4<0, 0>(a[slot][0], b, acc[nt][0], (int)sa[slot], bs);
        acc[nt][1] = mfma_fp4<1, 0>(a[slot][1], b, acc[nt][1], (int)sa[slot], bs);
        acc[nt][2] = mfma_fp4<2, 0>(a[slot][2], b, acc[nt][2], (int)sa[slot], bs);
        acc[nt][3] = mfma_fp4<3, 0>(a[slot][3], b, acc[nt][3], (int)sa[slot], bs);
      }
      const int jn = j + D;
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) a[slot][rb] = buf_load16<kPolicyDefault>(wr, voff + rb * 1024, jn * kStepCodeBytes);
      sa[slot] = buf_load4<kPolicyDefault>(sr, svoff, jn * kStepScaleBytes);
      if (q == CK - 1) {
        // Chunk boundary.  Buffer (chunk+1)&1 was last read in chunk-1, which
        // every wave finished before the previous barrier.
        if (chunk + 1 < nchunks) store_chunk((chunk + 1) & 1);
        __syncthreads();
        if (chunk + 2 < nchunks) load_chunk(chunk + 2);
      }
    }
  }

  if constexpr (G1)
    gemm1_epilogue<NT>(acc, unit, row0 + hrow0, nrows - hrow0, I, lane, hq, hsf, acc_out);
  else
    gemm2_epilogue<NT>(acc, unit, row0 + hrow0, nrows - hrow0, H, lane, y);
}

template <bool G1, int NT, int D, int CK, int WH = kTiledHalves>
static hipError_t launch_tiled_t(const uint8_t* wc, const uint8_t* wsc, const uint8_t* act,
                                 const uint8_t* act_sf, const int32_t* counts, const int32_t* offsets,
                                 const int32_t* sorted_rows, const int2* tiles, const int32_t* num_tiles,
                                 int max_tiles, int H, int I, int k, uint8_t* hq, uint8_t* hsf,
                                 float* acc_out, uint16_t* y, hipStream_t stream) {
  constexpr int ROWS = NT * 16 * WH;
  const size_t lds = 2 * ((size_t)ROWS * CK * 64 + (size_t)ROWS * CK * 4);
  const int nwb = G1 ? I / 128 : H / 256;
  const int64_t tiles_pad = MOE_TILED_GROUP > 0 ? ((int64_t)max_tiles + MOE_TILED_GROUP - 1) / MOE_TILED_GROUP *
                                                      MOE_TILED_GROUP
                                                : (int64_t)max_tiles;
  const int64_t blocks = (tiles_pad * nwb + 7) / 8 * 8;
  hipLaunchKernelGGL((gemm_tiled_kernel<G1, NT, D, CK, WH>), dim3((unsigned)blocks), dim3(256 * WH), lds, stream, wc,
                     wsc, act, act_sf, counts, offsets, sorted_rows, tiles, num_tiles, max_tiles, H, I, k, hq,
                     hsf, acc_out, y);
  return hipGetLastError();
}

int tiled_max_tiles(int R, int E) { return (R + kTiledRows - 1) / kTiledRows + E; }

#ifndef MOE_TILED_D
#define MOE_TILED_D 4    // weight-ring slots
#endif
#ifndef MOE_TILED_CK
#define MOE_TILED_CK 2   // K steps per staged token chunk
#endif

hipError_t launch_gemm1_tiled(const uint8_t* w1c, const uint8_t* w1s, const uint8_t* xq, const uint8_t* xsf,
                              const int32_t* counts, const int32_t* offsets, const int32_t* sorted_rows,
                              const int2* tiles, const int32_t* num_tiles, int max_tiles, int H, int I, int k,
                              uint8_t* hq, uint8_t* hsf, float* acc_out, hipStream_t stream) {
  // max(ring, chunk) must divide the K steps H/128 (even, as H % 256 == 0).
  // A 4-deep weight ring with 2-step token chunks fits in 256 VGPRs without
  // spills (2 waves per SIMD).
  constexpr int U = MOE_TILED_D > MOE_TILED_CK ? MOE_TILED_D : MOE_TILED_CK;
  if ((H / kStepK) % U == 0)
    return launch_tiled_t<true, kTiledNT, MOE_TILED_D, MOE_TILED_CK>(w1c, w1s, xq, xsf, counts, offsets,
                                                                    sorted_rows, tiles, num_tiles, max_tiles,
                                                                    H, I, k, hq, hsf, acc_out, nullptr, stream);
  return launch_tiled_t<true, kTiledNT, 2, 2>(w1c, w1s, xq, xsf, counts, offsets, sorted_rows, tiles, num_tiles,
                                              max_tiles, H, I, k, hq, hsf, acc_out, nullptr, stream);
}

hipError_t launch_gemm2_tiled(const uint8_t* w2c, const uint8_t* w2s, const uint8_t* hq, const uint8_t* hsf,
                              const int32_t* counts, const int32_t* offsets, const int2* tiles,
                              const int32_t* num_tiles, int max_tiles, int H, int I, uint16_t* y,
                              hipStream_t stream) {
  constexpr int U = MOE_TILED_D > MOE_TILED_CK ? MOE_TILED_D : MOE_TILED_CK;
  const int S = I / kStepK;
  if (S % U == 0)
    return launch_tiled_t<false, kTiledNT, MOE_TILED_D, MOE_TILED_CK>(w2c, w2s, hq, hsf, counts, offsets, nullptr,
                                                                     tiles, num_tiles, max_tiles, H, I, 1, nullptr,
                                                                     nullptr, nullptr, y, stream);
  if (S % 2 == 0)
    return launch_tiled_t<false, kTiledNT, 2, 2>(w2c, w2s, hq, hsf, counts, offsets, nullptr, tiles, num_tiles,
                                                 max_tiles, H, I, 1, nullptr, nullptr, nullptr, y, stream);
  return launch_tiled_t<false, kTiledNT, 1, 1>(w2c, w2s, hq, hsf, counts, offsets, nullptr, tiles, num_tiles,
                                               max_tiles, H, I, 1, nullptr, nullptr, nullptr, y, stream);
}

}  // namespace moe

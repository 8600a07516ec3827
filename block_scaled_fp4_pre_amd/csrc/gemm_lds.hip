// Stages S2 / S3 for many routed rows per expert (prefill): grouped GEMMs whose
// two operands are both staged in LDS by direct-to-LDS loads through a ring of
// P stages, one K step of 128 per stage.
//
// [P1] sglang PR "[deepseek-v4] Bump sgl-deep-gemm for packed FP4xFP4 mega-MoE
// (W4A4)", Appendix A (prefill sweep with 1024-token inputs) and section B (the
// fused layer on packed FP4 operands); [P3] prhub digest of sglang PR "bump
// sgl-deep-gemm to 0.1.7, MegaMoE uses the mma_type API for MXFP4", "Key source
// snippets" (activation="swiglu", gate rows then up rows in W1).
//
// Work item = (tile of up to NT*16 routed rows of one expert, from the route's
// tile list) x (weight block of 4 units = 256 weight rows).  Wave w of the
// 4-wave workgroup owns unit w (64 weight rows, the 16-row MFMA A side) and
// all NT*16 token rows (the B side), so each stage feeds 4*NT MFMAs per wave.
// A weight block is one unit group of the tile order (tiles.h): its 4 units'
// chunks of a step are one contiguous 16 KiB.
//
// F8 (the fp8xfp4 MMA type): the token codes are E4M3 bytes, 128 per row and
// K step instead of 64, and each MFMA's B operand is two 16-byte pieces.
//
// Per stage each wave issues its share of the DMA: its unit's 4 KiB of weight
// codes and 256 B of weight scales (already in MFMA operand order), a quarter
// of the token rows' 64-byte code pieces (gathered by row index; 16-byte piece
// c of row n lands at position c ^ ((n / 4) % 4), so the 16 rows one MFMA
// operand read touches fall on distinct banks) and a quarter of their scale
// dwords.  The DMA is issued from inline assembly: the compiler cannot tell the
// ring's stages apart and would otherwise wait for every DMA in flight before
// each LDS read.  The wait is explicit instead: before step s a wave waits
// until only the DMAs of the P-2 later stages it has issued remain
// (vmcnt, in order), then the barrier makes the whole stage visible and
// guarantees that stage s-1's buffer is no longer read, so the DMA of stage
// s+P-1 can go into it.
//
// Block order: logical id L = (blockIdx % 8) * (grid / 8) + blockIdx / 8 runs
// weight-block-major, tile-minor.  Workgroups are dealt round-robin to the 8
// XCDs, so each XCD gets a contiguous range of L: the tiles that share a
// weight block run on one XCD at about the same time and fetch it from HBM
// once into that XCD's L2.  (Tile-major order, which keeps a tile's tokens in
// L2 instead, measured 30% slower at 96 rows per expert.)  Exception: GEMM2
// with one tile per expert, where no weight block is shared: XCD x owns whole
// tiles, so each tile's rows of h reach one L2 only (E4M3 h at 96 rows per
// expert: 889 -> 866 us per layer; E2M1 about even; GEMM1 measured slower so).
//
// Occupancy: two workgroups per CU (3 stages x 26 KiB of LDS each; about 210
// VGPRs per lane with the accumulators, 245 with E4M3 tokens) measured faster
// than one workgroup with a deeper ring; the second workgroup's MFMAs cover
// the first one's waits.
#include "epilogue.h"
#include "gemm_common.h"
#include "launch.h"
#include "tiles.h"

namespace moe {

// One stage of the ring for WAVES waves (one weight unit each) and NT*16 token
// rows of TB code bytes per K step (64: E2M1; 128: E4M3, the fp8xfp4 MMA type).
template <int NT, int WAVES, int TB>
struct LdsStage {
  static constexpr int ROWS = NT * 16;
  static constexpr int W_CODES = 0;                          // WAVES units x 4 KiB
  static constexpr int W_SCALES = WAVES * kStepCodeBytes;    // WAVES units x 256 B
  static constexpr int T_CODES = W_SCALES + WAVES * kStepScaleBytes;  // ROWS x TB
  static constexpr int T_SCALES = T_CODES + ROWS * TB;       // ROWS x 4 B
  static constexpr int BYTES = T_SCALES + ROWS * 4;
};

template <bool B>
struct BoolConst {
  static constexpr bool value = B;
};

// Position of 16-byte piece c of staged token row n: 4 pieces per row (E2M1)
// or 8 (E4M3).  The 16 rows one MFMA operand read touches then fall on 16
// different 16-byte bank groups.
template <bool F8>
__device__ __forceinline__ int tok_pos(int n, int c) { return F8 ? c ^ ((n >> 1) & 7) : c ^ ((n >> 2) & 3); }

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// Direct global -> LDS copies: lane l's 16 (4) bytes land at LDS byte address
// lds + 16*l (4*l).  M0 carries the wave's LDS address (uniform; readfirstlane
// keeps it in a scalar register wherever the compiler's divergence analysis
// loses track of that).  A DMA that reads M0
// right after a scalar write of it needs one wait state (the s_nop), which the
// compiler cannot insert inside an asm statement.
__device__ __forceinline__ void dma16_asm(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}
__device__ __forceinline__ void dma4_asm(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}
// The same with the non-temporal hint (data read once).
__device__ __forceinline__ void dma16_nt_asm(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(g), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}
__device__ __forceinline__ void dma4_nt_asm(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off nt" ::"v"(g), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void stage_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

#ifndef MOE_LDS_PAIRED
#define MOE_LDS_PAIRED 1        // 1: per-XCD weight blocks, tile-major inside an XCD
#endif
#ifndef MOE_LDS_XCD_TILES
#define MOE_LDS_XCD_TILES 1     // GEMM2, one tile per expert: XCDs own whole tiles (else weight blocks)
#endif
#ifndef MOE_LDS_MFMA_PRIO
#define MOE_LDS_MFMA_PRIO 1     // several tiles per expert: raised wave priority over each MFMA block
#endif
#ifndef MOE_LDS_INTERLEAVE
#define MOE_LDS_INTERLEAVE 1    // 1: a stage's DMAs are issued between the MFMA groups of the step
#endif
#ifndef MOE_LDS_PAIR_G2_F8
#define MOE_LDS_PAIR_G2_F8 1    // fp8xfp4, one tile per expert: GEMM2 pairs weight blocks as GEMM1 does
#endif
#ifndef MOE_LDS_PAIR_MULTI_F8
#define MOE_LDS_PAIR_MULTI_F8 1 // fp8xfp4, several tiles per expert: both GEMMs pair weight blocks
#endif
#ifndef MOE_LDS_BLOCKS
#define MOE_LDS_BLOCKS 2        // workgroups per CU the launch bound asks for
#endif

// WNT: weight DMA with the non-temporal hint (each weight byte is read by one
// tile only).  WB: weight blocks per workgroup (4*WB waves, one unit each), so
// each staged token piece feeds WB weight blocks.
template <bool G1, int NT, int P, bool WNT, int WB, bool F8>
__global__ void __launch_bounds__(256 * WB, WB == 1 ? MOE_LDS_BLOCKS : 1) gemm_lds_kernel(
    const uint8_t* __restrict__ wc, const uint8_t* __restrict__ wsc, const uint8_t* __restrict__ act,
    const uint8_t* __restrict__ act_sf, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_rows,
    const int2* __restrict__ tiles, const int32_t* __restrict__ num_tiles, int max_tiles, int H, int I, int k,
    int hrows, uint8_t* __restrict__ hq, uint8_t* __restrict__ hsf, float* __restrict__ acc_out,
    uint16_t* __restrict__ y) {
  constexpr int WAVES = 4 * WB;
  constexpr int TB = F8 ? 128 : 64;                    // token code bytes per row and K step
  constexpr int PPR = TB / 16;                         // 16-byte pieces per row
  using L = LdsStage<NT, WAVES, TB>;
  constexpr int ROWS = L::ROWS;
  constexpr int TOK_INSTS = ROWS * TB / 1024 / WAVES;  // token-code DMAs (1 KiB each) per wave per stage
  constexpr int SC_LANES = ROWS / WAVES;               // token-scale dwords per wave per stage
  constexpr int DMA_PER_STAGE = 4 + 1 + TOK_INSTS + 1;
  // The waves' token DMAs tile the stage's token region exactly: ROWS rows x
  // TB bytes of codes, ROWS x 4 B of scales.
  static_assert(TOK_INSTS >= 1 && TOK_INSTS * WAVES * 1024 == ROWS * TB, "token code DMAs");
  static_assert(SC_LANES * WAVES == ROWS && SC_LANES <= 64, "token scale DMAs");
  static_assert(DMA_PER_STAGE * (P - 2) <= 63, "vmcnt range");

  const int K = G1 ? H : I;
  const int nwb = (G1 ? I / 128 : H / 256) / WB;      // weight-block groups per expert
  const int G = gridDim.x;
  constexpr bool XCD_TILES = WNT && !G1 && MOE_LDS_XCD_TILES;
  int wb, ti;
  if (XCD_TILES) {
    // GEMM2, one tile per expert: XCD x owns tiles x, x+8, ... and runs all
    // weight blocks of each before the next, so a tile's rows of h are fetched
    // into one L2 only (the launch covers ceil(max_tiles/8)*8 tiles).
    const int j = blockIdx.x >> 3, tq = j / nwb;
    ti = tq * 8 + (blockIdx.x & 7);
    wb = j - tq * nwb;
  } else if (MOE_LDS_PAIRED && nwb % 8 == 0) {
    // XCD x owns weight blocks [x*q, x*q+q); its workgroups run tile-major
    // over them, so the q workgroups of a tile share its token lines in L2.
    const int q = nwb >> 3, j = blockIdx.x >> 3;
    ti = j / q;
    wb = (blockIdx.x & 7) * q + (j - ti * q);
  } else {
    const int Lid = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    wb = Lid / max_tiles;
    ti = Lid - wb * max_tiles;
  }
  if (wb >= nwb || ti >= *num_tiles) return;
  const int2 tile = tiles[ti];
  const int e = tile.x, t0 = tile.y;
  const int nrows = min(ROWS, counts[e] - t0);
  const int row0 = offsets[e] + t0;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int unit = wb * WAVES + wave;
  const int S = K / kStepK;
  const int row_bytes = F8 ? K : K / 2;

  extern __shared__ __align__(16) uint8_t lds[];
  const uint32_t lbase = (uint32_t)(uintptr_t)lds;

  // DMA sources.  Rows past the tile's end re-read its last row (their
  // results are never stored).  Token scales, and GEMM2's token codes, are
  // K-step planes of sorted rows (hrows rows per plane): one contiguous run
  // per step for the tile.  GEMM1's token codes are gathered by token from the
  // row-major quantized x.
  const uint8_t* wsrc = wc + (G1 ? w1_code_offset(e, unit, 0, H, I) : w2_code_offset(e, unit, 0, H, I)) + lane * 16;
  const uint8_t* ssrc = wsc + (G1 ? w1_scale_offset(e, unit, 0, H, I) : w2_scale_offset(e, unit, 0, H, I)) + lane * 4;
  const size_t code_step = G1 ? TB : (size_t)hrows * TB, scale_step = (size_t)hrows * 4;
  const uint8_t* tsrc[TOK_INSTS];
#pragma unroll
  for (int i = 0; i < TOK_INSTS; ++i) {
    const int slot = (wave * TOK_INSTS + i) * 64 + lane;
    const int n = slot / PPR, r = row0 + min(n, nrows - 1);
    tsrc[i] = act + (G1 ? (size_t)(sorted_rows[r] / k) * row_bytes : (size_t)r * TB) + tok_pos<F8>(n, slot % PPR) * 16;
  }
  const uint8_t* tssrc = act_sf + (size_t)(row0 + min(wave * SC_LANES + min(lane, SC_LANES - 1), nrows - 1)) * 4;

  // DMA i (0 .. DMA_PER_STAGE-1) of stage s: the token scales (the one DMA
  // that not every lane takes part in, first, so that no MFMA of the step is
  // issued before that branch), the unit's four 1 KiB pieces of weight codes,
  // its weight scales, the token-code pieces.
  auto issue_one = [&](int s, int i) {
    const uint32_t sb = lbase + (uint32_t)((s % P) * L::BYTES);
    if (i == 0) {
      if (lane < SC_LANES) dma4_asm(tssrc + s * scale_step, sb + L::T_SCALES + wave * SC_LANES * 4);
    } else if (i <= 4) {
      const int rb = i - 1;
      if constexpr (WNT)
        dma16_nt_asm(wsrc + (size_t)s * kUnitStepStride + rb * 1024, sb + L::W_CODES + wave * kStepCodeBytes + rb * 1024);
      else
        dma16_asm(wsrc + (size_t)s * kUnitStepStride + rb * 1024, sb + L::W_CODES + wave * kStepCodeBytes + rb * 1024);
    } else if (i == 5) {
      if constexpr (WNT)
        dma4_nt_asm(ssrc + (size_t)s * kUnitScaleStride, sb + L::W_SCALES + wave * kStepScaleBytes);
      else
        dma4_asm(ssrc + (size_t)s * kUnitScaleStride, sb + L::W_SCALES + wave * kStepScaleBytes);
    } else {
      dma16_asm(tsrc[i - 6] + s * code_step, sb + L::T_CODES + (wave * TOK_INSTS + i - 6) * 1024);
    }
  };
  auto issue = [&](int s) {
#pragma unroll
    for (int i = 0; i < DMA_PER_STAGE; ++i) issue_one(s, i);
  };

  for (int s = 0; s < P - 1 && s < S; ++s) issue(s);

  v4f acc[NT][4];
  zero_acc<NT>(acc);
  const int tok_lane = lane & 15, kb = lane >> 4;
  // One K step from the stage in LDS; WITH_DMA also issues the DMAs of stage
  // s+P-1.  With MOE_LDS_INTERLEAVE they go between the MFMA groups, one group
  // of four MFMAs per 16 token rows, with scheduling fences so the compiler
  // keeps them there: a wave never sits on a full memory queue with none of
  // its MFMAs issued.  The operand reads come first, all of them.
  auto step = [&](int s, auto with_dma) {
    constexpr bool WITH_DMA = decltype(with_dma)::value;
#if !MOE_LDS_INTERLEAVE
    if constexpr (WITH_DMA) issue(s + P - 1);
#endif
    const uint8_t* st = lds + (s % P) * L::BYTES;
    uint4 a[4], b[NT], b2[F8 ? NT : 1];
    int sbv[NT];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
      a[rb] = *reinterpret_cast<const uint4*>(st + L::W_CODES + wave * kStepCodeBytes + rb * 1024 + lane * 16);
    const int sa = *reinterpret_cast<const int*>(st + L::W_SCALES + wave * kStepScaleBytes + lane * 4);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = nt * 16 + tok_lane;
      if constexpr (F8) {   // pieces kb and kb + 4 (the FP8 operand layout, device_common.h)
        b[nt] = *reinterpret_cast<const uint4*>(st + L::T_CODES + n * TB + tok_pos<true>(n, kb) * 16);
        b2[nt] = *reinterpret_cast<const uint4*>(st + L::T_CODES + n * TB + tok_pos<true>(n, kb + 4) * 16);
      } else {
        b[nt] = *reinterpret_cast<const uint4*>(st + L::T_CODES + n * TB + tok_pos<false>(n, kb) * 16);
      }
      sbv[nt] = (int)(*reinterpret_cast<const uint32_t*>(st + L::T_SCALES + n * 4) >> (8 * kb));
    }
    // Several tiles per expert (the MFMA-bound regime): the wave keeps a
    // raised issue priority over its MFMA block, so the SIMD's other wave
    // (between its own steps) does not interleave its instructions into it.
    if constexpr (!WNT && MOE_LDS_MFMA_PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#if MOE_LDS_INTERLEAVE
      if constexpr (WITH_DMA) {
#pragma unroll
        for (int i = 0; i < DMA_PER_STAGE; ++i)
          if (i * NT / DMA_PER_STAGE == nt) issue_one(s + P - 1, i);
      }
#endif
      if constexpr (F8) {
        acc[nt][0] = mfma_fp4_fp8<0, 0>(a[0], b[nt], b2[nt], acc[nt][0], sa, sbv[nt]);
        acc[nt][1] = mfma_fp4_fp8<1, 0>(a[1], b[nt], b2[nt], acc[nt][1], sa, sbv[nt]);
        acc[nt][2] = mfma_fp4_fp8<2, 0>(a[2], b[nt], b2[nt], acc[nt][2], sa, sbv[nt]);
        acc[nt][3] = mfma_fp4_fp8<3, 0>(a[3], b[nt], b2[nt], acc[nt][3], sa, sbv[nt]);
      } else {
        acc[nt][0] = mfma_fp4<0, 0>(a[0], b[nt], acc[nt][0], sa, sbv[nt]);
        acc[nt][1] = mfma_fp4<1, 0>(a[1], b[nt], acc[nt][1], sa, sbv[nt]);
        acc[nt][2] = mfma_fp4<2, 0>(a[2], b[nt], acc[nt][2], sa, sbv[nt]);
        acc[nt][3] = mfma_fp4<3, 0>(a[3], b[nt], acc[nt][3], sa, sbv[nt]);
      }
#if MOE_LDS_INTERLEAVE
      __builtin_amdgcn_sched_barrier(0);
#endif
    }
    if constexpr (!WNT && MOE_LDS_MFMA_PRIO) __builtin_amdgcn_s_setprio(0);
  };
  // Before step s a wave waits until only the DMAs of the P-2 stages after s
  // that it issued are in flight; the barrier then makes stage s whole and
  // frees the buffer of stage s-1, into which stage s+P-1 goes.
  int s = 0;
  for (; s + P - 1 < S; ++s) {
    wait_vm<DMA_PER_STAGE * (P - 2)>();
    stage_barrier();
    step(s, BoolConst<true>{});
  }
  for (; s < S; ++s) {                      // the last P-1 steps issue nothing
    if (s + P - 2 < S)
      wait_vm<DMA_PER_STAGE * (P - 2)>();
    else
      wait_vm<0>();
    stage_barrier();
    step(s, BoolConst<false>{});
  }

  constexpr int kYStride = 144;
  if constexpr (G1) {
    gemm1_epilogue<NT, F8>(acc, unit, row0, nrows, I, hrows, lane, hq, hsf, acc_out);
  } else if constexpr (WAVES * ROWS * kYStride > P * L::BYTES) {
    gemm2_epilogue<NT>(acc, unit, row0, nrows, H, lane, y);   // (8-wave tiles: the ring is too small)
  } else {
    // y through LDS, so that every store writes whole 128-byte lines: a
    // unit's 64 bf16 columns of a row are one aligned line, and the
    // accumulator layout gives each lane 8 bytes of it (4 pieces, 16 rows
    // apart in the store pattern of gemm2_epilogue).  Each wave puts its
    // ROWS x 64 tile into the ring's bytes (rows kYStride apart: the 16 rows a
    // write touches start on different bank groups), then stores 8 rows per
    // instruction, 16 bytes a lane.  Writing the pieces directly cost GEMM2
    // about 30 % of its time at 4096 tokens.
    __syncthreads();                                   // every wave is done with the ring
    uint8_t* ytile = lds + wave * ROWS * kYStride;
    const int tok_lane = lane & 15, kb = lane >> 4;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
        *reinterpret_cast<uint64_t*>(ytile + (nt * 16 + tok_lane) * kYStride + (16 * rb + 4 * kb) * 2) =
            (uint64_t)(f32_to_bf16(acc[nt][rb][0]) | (f32_to_bf16(acc[nt][rb][1]) << 16)) |
            ((uint64_t)(f32_to_bf16(acc[nt][rb][2]) | (f32_to_bf16(acc[nt][rb][3]) << 16)) << 32);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < ROWS / 8; ++i) {
      const int r = i * 8 + (lane >> 3), c = lane & 7;
      if (r < nrows)
        *reinterpret_cast<uint4*>(y + (size_t)(row0 + r) * H + 64 * unit + 8 * c) =
            *reinterpret_cast<const uint4*>(ytile + r * kYStride + 16 * c);
    }
  }
}

#ifndef MOE_LDS_STAGES
#define MOE_LDS_STAGES 3      // ring stages: two workgroups of 3 x 26 KiB fit a CU's LDS
#endif

constexpr int kLdsNT = 8;     // token tiles of 16 rows per wave: 128-row work tiles

template <bool G1, bool WNT, int WB, bool F8>
static hipError_t launch_prefill_wb(const uint8_t* wc, const uint8_t* wsc, const uint8_t* act,
                                    const uint8_t* act_sf, const int32_t* counts, const int32_t* offsets,
                                    const int32_t* sorted_rows, const int2* tiles, const int32_t* num_tiles,
                                    int max_tiles, int H, int I, int k, int hrows, uint8_t* hq, uint8_t* hsf,
                                    float* acc_out, uint16_t* y, hipStream_t stream) {
  constexpr int P = MOE_LDS_STAGES;
  auto kern = gemm_lds_kernel<G1, kLdsNT, P, WNT, WB, F8>;
  const size_t lds = (size_t)P * LdsStage<kLdsNT, 4 * WB, F8 ? 128 : 64>::BYTES;
  if (lds > 65536) {
    hipError_t err = raise_lds_limit(reinterpret_cast<const void*>(kern), lds);
    if (err != hipSuccess) return err;
  }
  const int nwb = (G1 ? I / 128 : H / 256) / WB;
  const int64_t blocks = WNT && !G1 && MOE_LDS_XCD_TILES ? (int64_t)((max_tiles + 7) / 8) * nwb * 8
                                                  : ((int64_t)max_tiles * nwb + 7) / 8 * 8;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256 * WB), lds, stream, wc, wsc, act, act_sf, counts, offsets,
                     sorted_rows, tiles, num_tiles, max_tiles, H, I, k, hrows, hq, hsf, acc_out, y);
  return hipGetLastError();
}

int lds_tile_rows(int) { return kLdsNT * 16; }

int lds_max_tiles(int R, int E, int tile_rows) { return (R + tile_rows - 1) / tile_rows + E; }

// Mean rows per expert within one tile (the weight stream bounds the GEMM):
// every weight block is read by a single tile, so it streams non-temporal, and
// GEMM1 pairs two weight blocks per workgroup so each staged token piece feeds
// both (half the token traffic; measured 6% faster GEMM1 at 96 rows per
// expert).  More rows: the tiles of an expert share each weight block through
// L2, loads keep the default policy, and single-block workgroups (two per CU,
// each with its own barrier) keep the MFMAs busier.  With E4M3 tokens a stage
// holds twice the token bytes, three stages no longer fit two workgroups per
// CU, and pairing wins everywhere (GEMM2 at 96 rows per expert: 914 -> 897 us
// per layer; Zipf tiles at 16384 tokens: 3066 -> 2748 us).
template <bool G1, bool F8>
static hipError_t launch_prefill(const uint8_t* wc, const uint8_t* wsc, const uint8_t* act, const uint8_t* act_sf,
                                 const int32_t* counts, const int32_t* offsets, const int32_t* sorted_rows,
                                 const int2* tiles, const int32_t* num_tiles, int max_tiles, int rows_hint, int H,
                                 int I, int k, int hrows, uint8_t* hq, uint8_t* hsf, float* acc_out, uint16_t* y,
                                 hipStream_t stream) {
#define MOE_PREFILL_ARGS wc, wsc, act, act_sf, counts, offsets, sorted_rows, tiles, num_tiles, max_tiles, H, I, k, \
                         hrows, hq, hsf, acc_out, y, stream
  const bool single = rows_hint <= kLdsNT * 16;
  const int nwb = G1 ? I / 128 : H / 256;
  const bool pair = nwb % 2 == 0 && (single ? (G1 || (F8 && MOE_LDS_PAIR_G2_F8)) : (F8 && MOE_LDS_PAIR_MULTI_F8));
  if (single && pair) return launch_prefill_wb<G1, true, 2, F8>(MOE_PREFILL_ARGS);
  if (single) return launch_prefill_wb<G1, true, 1, F8>(MOE_PREFILL_ARGS);
  if (pair) return launch_prefill_wb<G1, false, 2, F8>(MOE_PREFILL_ARGS);
  return launch_prefill_wb<G1, false, 1, F8>(MOE_PREFILL_ARGS);
#undef MOE_PREFILL_ARGS
}

// xsf_planes: the token scales of the sorted rows in K-step planes of hrows
// rows (launch_sorted_scales); hq/hsf: GEMM1's output planes (epilogue.h).
hipError_t launch_gemm1_lds(bool fp8, const uint8_t* w1c, const uint8_t* w1s, const uint8_t* xq,
                            const uint8_t* xsf_planes, const int32_t* counts, const int32_t* offsets,
                            const int32_t* sorted_rows, const int2* tiles, const int32_t* num_tiles, int max_tiles,
                            int rows_hint, int H, int I, int k, int hrows, uint8_t* hq, uint8_t* hsf, float* acc_out,
                            hipStream_t stream) {
  auto launch = fp8 ? launch_prefill<true, true> : launch_prefill<true, false>;
  return launch(w1c, w1s, xq, xsf_planes, counts, offsets, sorted_rows, tiles, num_tiles, max_tiles, rows_hint, H, I,
                k, hrows, hq, hsf, acc_out, nullptr, stream);
}

hipError_t launch_gemm2_lds(bool fp8, const uint8_t* w2c, const uint8_t* w2s, const uint8_t* hq, const uint8_t* hsf,
                            const int32_t* counts, const int32_t* offsets, const int2* tiles,
                            const int32_t* num_tiles, int max_tiles, int rows_hint, int H, int I, int hrows,
                            uint16_t* y, hipStream_t stream) {
  auto launch = fp8 ? launch_prefill<false, true> : launch_prefill<false, false>;
  return launch(w2c, w2s, hq, hsf, counts, offsets, nullptr, tiles, num_tiles, max_tiles, rows_hint, H, I, 1, hrows,
                nullptr, nullptr, nullptr, y, stream);
}

}  // namespace moe

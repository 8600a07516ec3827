// Stages S2 / S3 of the NVFP4 type (nvfp4.h) for many routed rows per expert
// (prefill): the tiled GEMMs of gemm_lds.hip with NVFP4 operands.  [P3] prhub
// digest of sglang PR "bump sgl-deep-gemm to 0.1.7, MegaMoE uses the mma_type
// API for MXFP4", "Motivation" (the NVFP4 variant); [P1] sglang PR
// "[deepseek-v4] Bump sgl-deep-gemm for packed FP4xFP4 mega-MoE (W4A4)",
// Appendix A (prefill inputs of 1024 tokens per sequence).
//
// Work item = (tile of up to 128 routed rows of one expert, from the route's
// tile list) x (two weight blocks of 4 units).  The 8 waves of a workgroup
// own one unit each (64 weight rows, the 16-row MFMA A side) and share the
// tile's 128 token rows (the B side).  Both operands go HBM/L2 -> LDS by
// direct-to-LDS loads through a ring of 2 stages, one K step of 128 per stage:
//   weight codes   8 units x 4 KiB (tile order, tiles.h)
//   weight scales  8 units x 512 B (nvfp4.h: lane l's 8 bytes at l * 8)
//   token codes    128 rows x 64 B (16-byte piece c of row n at c ^ (n/4 % 4))
//   token scales   2 dword planes x 128 rows (the sorted scales' dword planes
//                  2s and 2s+1: bytes 2*kb + half of the row's K step)
// 45 KiB per stage, plus a shared fp16 token tile of 32 KiB: 122 KiB per
// workgroup, one workgroup per CU.
//
// Step s: wait for stage s, barrier, issue the DMAs of stage s+1 (they
// overlap the rest of the step), then each wave converts 16 token rows of
// stage s into exact fp16 products e2m1 * e4m3 in the shared tile, a second
// barrier, and each wave turns its unit's four 16-byte weight operands into
// 16 fp16 operands and runs, per 16-row token tile, 16 fp16 MFMAs (4 weight
// blocks x 4 K pieces of 32) on operands read from the fp16 tile.  Converting
// the tokens once per workgroup instead of once per wave measured 10 % faster
// at 96 rows per expert (T = 4096 layer 1793-1801 -> 1630-1634 us).  The
// per-wave form (MOE_NV_LDS_COOP=0: 3 stages, token conversion in every
// wave, the next stage's DMAs between the MFMA groups) is kept for that
// comparison.
//
// Block order as gemm_lds.hip's paired form: XCD x owns weight-block pairs
// [x*q, x*q+q) and runs tile-major over them, so the q workgroups of a tile
// share its token lines in one L2.
#include "epilogue_nv.h"
#include "gemm_common.h"
#include "launch.h"
#include "nvfp4.h"
#include "tiles.h"

namespace moe {
namespace {

#ifndef MOE_NV_LDS_COOP
#define MOE_NV_LDS_COOP 1   // 1: the waves convert the stage's tokens to fp16 once, into a shared LDS tile
#endif

constexpr int kNvLdsWaves = 8;                      // two weight blocks of 4 units
constexpr int kNvLdsNT = 8;                         // 8 token tiles of 16 rows: 128-row work tiles
constexpr int kNvLdsRows = kNvLdsNT * 16;
constexpr int kNvLdsStages = MOE_NV_LDS_COOP ? 2 : 3;
// The shared fp16 token tile: 128 rows x 128 K elements x 2 bytes; 16-byte
// chunk c (K elements 8c..8c+7) of row n at position c ^ (n % 16), so the
// 16 rows one operand read touches fall on distinct banks.
constexpr int kNvF16Tile = MOE_NV_LDS_COOP ? kNvLdsRows * 128 * 2 : 0;

struct NvLdsStage {
  static constexpr int W_CODES = 0;                                           // 8 x 4 KiB
  static constexpr int W_SCALES = kNvLdsWaves * kStepCodeBytes;                // 8 x 512 B
  static constexpr int T_CODES = W_SCALES + kNvLdsWaves * kNvStepScaleBytes;   // 128 x 64 B
  static constexpr int T_SCALES = T_CODES + kNvLdsRows * 64;                   // 2 x 128 dwords
  static constexpr int BYTES = T_SCALES + 2 * kNvLdsRows * 4;
};

// DMAs per wave and stage: token scales (one dword per lane, 32 lanes), four
// 1 KiB pieces of weight codes, two 256 B halves of weight scales, one 1 KiB
// of token codes.
constexpr int kNvDmaPerStage = 8;
static_assert(kNvLdsRows * 64 == kNvLdsWaves * 1024, "one token-code DMA per wave");
static_assert(2 * kNvLdsRows == kNvLdsWaves * 32, "32 token-scale dwords per wave");
static_assert(kNvLdsStages < 3 || kNvDmaPerStage * (kNvLdsStages - 2) <= 63, "vmcnt range");

template <bool B>
struct NvBool {
  static constexpr bool value = B;
};

__device__ __forceinline__ int nv_tok_pos(int n, int c) { return c ^ ((n >> 2) & 3); }

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// Direct global -> LDS copies issued from inline assembly (the compiler would
// otherwise wait for every DMA in flight before each LDS read): M0 carries
// the wave's LDS address, and a DMA that reads M0 right after a scalar write of
// it needs one wait state, which the compiler cannot insert inside the asm.
__device__ __forceinline__ void nv_dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g),
               "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}
__device__ __forceinline__ void nv_dma4(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g),
               "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}
__device__ __forceinline__ void nv_dma16_nt(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(g),
               "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}
__device__ __forceinline__ void nv_dma4_nt(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off nt" ::"v"(g),
               "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void nv_wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void nv_stage_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// The four fp16 operands of a 16-byte FP4 operand with its two scale bytes.
__device__ __forceinline__ void nv_lds_operands(const uint4& c, uint32_t scales, v8h (&o)[4]) {
  const v2h lo = e4m3_scale_f16x2(scales & 0xFFu), hi = e4m3_scale_f16x2((scales >> 8) & 0xFFu);
  o[0] = nv_operand(c.x, lo);
  o[1] = nv_operand(c.y, lo);
  o[2] = nv_operand(c.z, hi);
  o[3] = nv_operand(c.w, hi);
}

}  // namespace

// WNT: weights loaded non-temporal (each expert fits one tile, so each weight
// byte is read by one workgroup only).
template <bool G1, bool WNT>
__global__ void __launch_bounds__(64 * kNvLdsWaves, 1) gemm_lds_nv_kernel(
    const uint8_t* __restrict__ wc, const uint8_t* __restrict__ wsc, const float* __restrict__ gsc,
    const uint8_t* __restrict__ act, const uint8_t* __restrict__ act_sf, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_rows, const int2* __restrict__ tiles,
    const int32_t* __restrict__ num_tiles, int max_tiles, int H, int I, int E, int k, int hrows,
    uint8_t* __restrict__ hq, uint8_t* __restrict__ hsf, float* __restrict__ acc_out, uint16_t* __restrict__ y) {
  using L = NvLdsStage;
  constexpr int P = kNvLdsStages;
  constexpr int ROWS = kNvLdsRows;
  const int K = G1 ? H : I;
  const int nwb = (G1 ? I / 128 : H / 256) / 2;       // weight-block pairs per expert
  const int G = gridDim.x;
  int wb, ti;
  if (nwb % 8 == 0) {
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
  const int unit = wb * kNvLdsWaves + wave;
  const int S = K / kStepK;
  const int row_bytes = K / 2;

  extern __shared__ __align__(16) uint8_t lds[];
  const uint32_t lbase = (uint32_t)(uintptr_t)lds;

  // DMA sources.  Rows past the tile's end re-read its last row (their
  // results are never stored).  GEMM1's token codes are gathered by token
  // from the row-major x-hat; GEMM2's are K-step planes of sorted rows, and
  // the token scales of both are dword planes of sorted rows (two per step).
  const uint8_t* wsrc = wc + (G1 ? w1_code_offset(e, unit, 0, H, I) : w2_code_offset(e, unit, 0, H, I)) + lane * 16;
  const uint8_t* ssrc =
      wsc + (G1 ? nv_w1_scale_offset(e, unit, 0, H, I) : nv_w2_scale_offset(e, unit, 0, H, I)) + lane * 4;
  const size_t code_step = G1 ? 64 : (size_t)hrows * 64, scale_step = (size_t)2 * hrows * 4;
  const uint8_t* tsrc;
  {
    const int slot = wave * 64 + lane;                  // 16-byte piece `slot` of the tile's 8 KiB
    const int n = slot >> 2, r = row0 + min(n, nrows - 1);
    tsrc = act + (G1 ? (size_t)(sorted_rows[r] / k) * row_bytes : (size_t)r * 64) + nv_tok_pos(n, slot & 3) * 16;
  }
  const int sq = wave * 32 + min(lane, 31);             // token-scale dword of the stage: plane sq / 128, row sq % 128
  const uint8_t* tssrc = act_sf + ((size_t)(sq / ROWS) * hrows + row0 + min(sq % ROWS, nrows - 1)) * 4;

  auto issue_one = [&](int s, int i) {
    const uint32_t sb = lbase + (uint32_t)((s % P) * L::BYTES);
    if (i == 0) {
      if (lane < 32) nv_dma4(tssrc + s * scale_step, sb + L::T_SCALES + wave * 32 * 4);
    } else if (i <= 4) {
      const int rb = i - 1;
      const void* g = wsrc + (size_t)s * kUnitStepStride + rb * 1024;
      const uint32_t d = sb + L::W_CODES + wave * kStepCodeBytes + rb * 1024;
      if constexpr (WNT) nv_dma16_nt(g, d); else nv_dma16(g, d);
    } else if (i <= 6) {
      const int h = i - 5;
      const void* g = ssrc + (size_t)s * kNvUnitScaleStride + h * 256;
      const uint32_t d = sb + L::W_SCALES + wave * kNvStepScaleBytes + h * 256;
      if constexpr (WNT) nv_dma4_nt(g, d); else nv_dma4(g, d);
    } else {
      nv_dma16(tsrc + s * code_step, sb + L::T_CODES + wave * 1024);
    }
  };
  auto issue = [&](int s) {
#pragma unroll
    for (int i = 0; i < kNvDmaPerStage; ++i) issue_one(s, i);
  };

  for (int s = 0; s < P - 1 && s < S; ++s) issue(s);

  v4f acc[kNvLdsNT][4];
  zero_acc<kNvLdsNT>(acc);
  const int tok_lane = lane & 15, kb = lane >> 4;
  uint8_t* const f16 = lds + P * L::BYTES;   // the shared fp16 token tile (MOE_NV_LDS_COOP)
  // MOE_NV_LDS_COOP: wave w converts token rows 16w..16w+15 of stage s, lane
  // (row, kb) the 32 K elements of its 16-byte operand, into the fp16 tile.
  auto convert_tokens = [&](int s) {
    const uint8_t* st = lds + (s % P) * L::BYTES;
    const int n = wave * 16 + tok_lane;
    const uint4 b = *reinterpret_cast<const uint4*>(st + L::T_CODES + n * 64 + nv_tok_pos(n, kb) * 16);
    const uint32_t bs =
        *reinterpret_cast<const uint16_t*>(st + L::T_SCALES + ((kb >> 1) * ROWS + n) * 4 + (kb & 1) * 2);
    v8h bo[4];
    nv_lds_operands(b, bs, bo);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<v8h*>(f16 + n * 256 + (((4 * kb + i) ^ (n & 15)) << 4)) = bo[i];
  };
  auto step = [&](int s, auto with_dma) {
    constexpr bool WITH_DMA = decltype(with_dma)::value;
    const uint8_t* st = lds + (s % P) * L::BYTES;
    v8h w[4][4];
    {
      const uint2 sa = *reinterpret_cast<const uint2*>(st + L::W_SCALES + wave * kNvStepScaleBytes + lane * 8);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const uint4 a = *reinterpret_cast<const uint4*>(st + L::W_CODES + wave * kStepCodeBytes + rb * 1024 + lane * 16);
        nv_lds_operands(a, ((rb < 2 ? sa.x : sa.y) >> (16 * (rb & 1))) & 0xFFFFu, w[rb]);
      }
    }
#pragma unroll
    for (int nt = 0; nt < kNvLdsNT; ++nt) {
      if constexpr (WITH_DMA && !MOE_NV_LDS_COOP) {
        if (nt < kNvDmaPerStage) issue_one(s + P - 1, nt);
      }
      const int n = nt * 16 + tok_lane;
      v8h bo[4];
      if constexpr (MOE_NV_LDS_COOP) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          bo[i] = *reinterpret_cast<const v8h*>(f16 + n * 256 + (((4 * kb + i) ^ (n & 15)) << 4));
      } else {
        const uint4 b = *reinterpret_cast<const uint4*>(st + L::T_CODES + n * 64 + nv_tok_pos(n, kb) * 16);
        const uint32_t bs =
            *reinterpret_cast<const uint16_t*>(st + L::T_SCALES + ((kb >> 1) * ROWS + n) * 4 + (kb & 1) * 2);
        nv_lds_operands(b, bs, bo);
      }
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[nt][rb] = mfma_f16(w[rb][i], bo[i], acc[nt][rb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if constexpr (MOE_NV_LDS_COOP) {
    // Two stages.  Step s: wait for stage s, barrier (every wave has left
    // step s-1, so the other ring slot and the fp16 tile are free), issue
    // stage s+1, convert this wave's share of stage s's tokens, barrier, then
    // the MFMAs, which overlap stage s+1's DMA.
    for (int s = 0; s < S; ++s) {
      nv_wait_vm<0>();
      nv_stage_barrier();
      if (s + 1 < S) issue(s + 1);
      convert_tokens(s);
      nv_stage_barrier();
      step(s, NvBool<false>{});
    }
  } else {
    int s = 0;
    for (; s + P - 1 < S; ++s) {
      nv_wait_vm<kNvDmaPerStage * (P - 2)>();
      nv_stage_barrier();
      step(s, NvBool<true>{});
    }
    for (; s < S; ++s) {                      // the last P-1 steps issue nothing
      if (s + P - 2 < S)
        nv_wait_vm<kNvDmaPerStage * (P - 2)>();
      else
        nv_wait_vm<0>();
      nv_stage_barrier();
      step(s, NvBool<false>{});
    }
  }

  if constexpr (G1) {
    const float gg = __fmul_rn(gsc[2 * E], gsc[e]);
    gemm1_epilogue_nv<kNvLdsNT>(acc, unit, row0, nrows, I, hrows, lane, gg, gsc[2 * E + 1], hq, hsf, acc_out);
  } else {
    gemm2_epilogue_nv<kNvLdsNT>(acc, unit, row0, nrows, H, lane, __fmul_rn(gsc[2 * E + 1], gsc[E + e]), y);
  }
}

template <bool G1, bool WNT>
static hipError_t launch_lds_nv(const uint8_t* wc, const uint8_t* wsc, const float* gsc, const uint8_t* act,
                                const uint8_t* act_sf, const int32_t* counts, const int32_t* offsets,
                                const int32_t* sorted_rows, const int2* tiles, const int32_t* num_tiles, int max_tiles,
                                int H, int I, int E, int k, int hrows, uint8_t* hq, uint8_t* hsf, float* acc_out,
                                uint16_t* y, hipStream_t stream) {
  auto kern = gemm_lds_nv_kernel<G1, WNT>;
  const size_t lds = (size_t)kNvLdsStages * NvLdsStage::BYTES + kNvF16Tile;
  hipError_t err = raise_lds_limit(reinterpret_cast<const void*>(kern), lds);
  if (err != hipSuccess) return err;
  const int nwb = (G1 ? I / 128 : H / 256) / 2;
  const int64_t blocks = ((int64_t)max_tiles * nwb + 7) / 8 * 8;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64 * kNvLdsWaves), lds, stream, wc, wsc, gsc, act, act_sf,
                     counts, offsets, sorted_rows, tiles, num_tiles, max_tiles, H, I, E, k, hrows, hq, hsf, acc_out,
                     y);
  return hipGetLastError();
}

hipError_t launch_gemm1_lds_nv(const uint8_t* w1c, const uint8_t* w1s, const float* gsc, const uint8_t* xq,
                               const uint8_t* xsf_planes, const int32_t* counts, const int32_t* offsets,
                               const int32_t* sorted_rows, const int2* tiles, const int32_t* num_tiles,
                               int max_tiles, int rows_hint, int H, int I, int E, int k, int hrows, uint8_t* hq,
                               uint8_t* hsf, float* acc_out, hipStream_t stream) {
  auto launch = rows_hint <= kNvLdsRows ? launch_lds_nv<true, true> : launch_lds_nv<true, false>;
  return launch(w1c, w1s, gsc, xq, xsf_planes, counts, offsets, sorted_rows, tiles, num_tiles, max_tiles, H, I, E, k,
                hrows, hq, hsf, acc_out, nullptr, stream);
}

hipError_t launch_gemm2_lds_nv(const uint8_t* w2c, const uint8_t* w2s, const float* gsc, const uint8_t* hq,
                               const uint8_t* hsf, const int32_t* counts, const int32_t* offsets, const int2* tiles,
                               const int32_t* num_tiles, int max_tiles, int rows_hint, int H, int I, int E,
                               int hrows, uint16_t* y, hipStream_t stream) {
  auto launch = rows_hint <= kNvLdsRows ? launch_lds_nv<false, true> : launch_lds_nv<false, false>;
  return launch(w2c, w2s, gsc, hq, hsf, counts, offsets, nullptr, tiles, num_tiles, max_tiles, H, I, E, 1, hrows,
                nullptr, nullptr, nullptr, y, stream);
}

}  // namespace moe

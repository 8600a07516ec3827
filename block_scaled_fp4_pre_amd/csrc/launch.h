// Host-side launchers of the gfx950 kernels (one translation unit per stage).
// Every launcher only enqueues on `stream`; shapes were validated by the caller.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#ifndef MOE_STREAM_ROWS2
#define MOE_STREAM_ROWS2 24   // token rows per pass of the streaming GEMMs' two-tile form (17..32)
#endif

namespace moe {

constexpr size_t kCuLdsBytes = 160 * 1024;   // LDS of one gfx950 CU

// LDS of a streaming GEMM's token tile, which spans all of K (H for GEMM1, I
// for GEMM2): 16 rows, or MOE_STREAM_ROWS2 with two tiles (mean rows per
// expert above 8), each K/2 code bytes (E4M3: K) plus K/32 scale bytes.
inline size_t stream_tile_lds(bool fp8, int K, int rows_hint) {
  const size_t rows = rows_hint > 8 ? MOE_STREAM_ROWS2 : 16;
  return rows * ((size_t)(fp8 ? K : K / 2) + (size_t)K / 32);
}

// MOE_OK if the current HIP device is a gfx950, else MOE_ENODEVICE (cached per device).
int check_device();

// Stage S1a: MXFP4 quantization of rows of bf16 (src_is_bf16) or fp32 values;
// fp8: MXFP8 E4M3 codes instead (the fp8xfp4 MMA type's activations, bf16 only).
hipError_t launch_quantize(bool src_is_bf16, bool fp8, const void* src, int64_t ngroups,
                           uint8_t* codes, uint8_t* scales, hipStream_t stream);
// NVFP4 under tensor scale gs (or *gsp, a device address, when gsp is not
// null): per 32-element group 16 code bytes and 2 scale bytes.
hipError_t launch_quantize_nv(bool src_is_bf16, const void* src, int64_t ngroups, float gs, const float* gsp,
                              uint8_t* codes, uint8_t* scales, hipStream_t stream);

// Stage S1b: stable counting sort of R routed rows over E experts.  With
// tile_rows > 0 it also lists the (expert, first row) tiles of tile_rows rows
// that the tiled GEMMs work on.
hipError_t launch_route(const int32_t* ids, int R, int E, int32_t* hist, int32_t* counts,
                        int32_t* offsets, int32_t* sorted_rows, int32_t* pos, int tile_rows, int2* tiles,
                        int32_t* num_tiles, hipStream_t stream);

// Stages S1a + S1b in one launch: block 0 routes all R <= kPredispatchMaxRows
// rows, the other blocks quantize the bf16 tokens (act: 0 MXFP4, 1 MXFP8
// E4M3, 2 NVFP4 under the tensor scale at device address gx).
constexpr int kPredispatchMaxRows = 8192;
hipError_t launch_predispatch(int act, const uint16_t* x, int64_t ngroups, const float* gx, uint8_t* xq,
                              uint8_t* xsf, const int32_t* ids, int R, int E, int32_t* counts, int32_t* offsets,
                              int32_t* sorted_rows, int32_t* pos, int tile_rows, int2* tiles, int32_t* num_tiles,
                              hipStream_t stream);

// The whole forward in one launch (mega.hip) for at most kMegaMaxRows routed
// rows, H and I each 512, 1024, 2048 or 4096: route, quantization, both GEMMs
// and the combine; MXFP4 tokens and h, or E4M3 (f8, the fp8xfp4 MMA type).
// state: the workspace's `mega` region (zero at the launch, left zero);
// xq/xsf, counts, offsets, sorted_rows, pos, hq/hsf and y receive what the
// stages write.  poll_limit bounds every wait.
hipError_t launch_mega(const uint8_t* w1c, const uint8_t* w1s, const uint8_t* w2c, const uint8_t* w2s,
                       const uint16_t* x, const int32_t* ids, const float* tw, uint16_t* out, int T, int H, int I,
                       int E, int k, int hrows, uint8_t* xq, uint8_t* xsf, uint8_t* hq, uint8_t* hsf, uint16_t* y,
                       uint64_t* state, int32_t* counts, int32_t* offsets, int32_t* sorted_rows, int32_t* pos,
                       bool f8, uint32_t poll_limit, hipStream_t stream);

// Prefill GEMMs with both operands staged in LDS (gemm_lds.hip): tiles of
// lds_tile_rows(mean rows per expert) routed rows; rows_hint (the mean) also
// picks the weight load policy and the work order.
// hrows: rows of one K-step plane of the sorted-row activations (hq/hsf and
// the sorted token scales; epilogue.h), the workspace's routed-row capacity.
int lds_tile_rows(int rows_hint);
int lds_max_tiles(int R, int E, int tile_rows);
// fp8: the activations are E4M3 (the fp8xfp4 MMA type) instead of E2M1.
hipError_t launch_gemm1_lds(bool fp8, const uint8_t* w1c, const uint8_t* w1s, const uint8_t* xq,
                            const uint8_t* xsf_planes, const int32_t* counts, const int32_t* offsets,
                            const int32_t* sorted_rows, const int2* tiles, const int32_t* num_tiles, int max_tiles,
                            int rows_hint, int H, int I, int k, int hrows, uint8_t* hq, uint8_t* hsf, float* acc_out,
                            hipStream_t stream);
hipError_t launch_gemm2_lds(bool fp8, const uint8_t* w2c, const uint8_t* w2s, const uint8_t* hq, const uint8_t* hsf,
                            const int32_t* counts, const int32_t* offsets, const int2* tiles,
                            const int32_t* num_tiles, int max_tiles, int rows_hint, int H, int I, int hrows,
                            uint16_t* y, hipStream_t stream);

// The token scales of the sorted rows [0, offsets[E]) in dword planes: plane
// d, row q = scale dword d of token sorted_rows[q] / k (sc_dwords per token:
// H/128, one per K step, for MXFP4; H/64, two per K step, for NVFP4).  Read
// by the LDS-staged GEMM1, whose per-step token-scale loads then cover
// consecutive addresses.  rows_bound >= offsets[E] sizes the grid.
hipError_t launch_sorted_scales(const uint8_t* xsf, const int32_t* sorted_rows, const int32_t* offsets, int E,
                                int rows_bound, int sc_dwords, int k, int hrows, uint8_t* xsf_planes,
                                hipStream_t stream);

// Stage S2: grouped GEMM1 over the prepared W1 tiles + SwiGLU + MXFP4 requant
// (fp8: E4M3 activations and requant, the fp8xfp4 MMA type).
hipError_t launch_gemm1(bool fp8, const uint8_t* w1_codes, const uint8_t* w1_scales, const uint8_t* xq,
                        const uint8_t* xsf, const int32_t* counts, const int32_t* offsets,
                        const int32_t* sorted_rows, int H, int I, int E, int k, int rows_hint, int hrows,
                        uint8_t* hq, uint8_t* hsf, float* acc_out, hipStream_t stream);

// Stage S3: grouped GEMM2 over the prepared W2 tiles -> bf16 y in sorted order
// (fp8: E4M3 activations).
hipError_t launch_gemm2(bool fp8, const uint8_t* w2_codes, const uint8_t* w2_scales, const uint8_t* hq,
                        const uint8_t* hsf, const int32_t* counts, const int32_t* offsets, int H,
                        int I, int E, int rows_hint, int hrows, uint16_t* y, hipStream_t stream);

// Stages S2 and S3 of the NVFP4 type for many rows per expert
// (gemm_lds_nv.hip): LDS-staged tiles of lds_tile_rows rows from the route's
// tile list, token scales from the sorted dword planes (launch_sorted_scales).
hipError_t launch_gemm1_lds_nv(const uint8_t* w1c, const uint8_t* w1s, const float* gsc, const uint8_t* xq,
                               const uint8_t* xsf_planes, const int32_t* counts, const int32_t* offsets,
                               const int32_t* sorted_rows, const int2* tiles, const int32_t* num_tiles,
                               int max_tiles, int rows_hint, int H, int I, int E, int k, int hrows, uint8_t* hq,
                               uint8_t* hsf, float* acc_out, hipStream_t stream);
hipError_t launch_gemm2_lds_nv(const uint8_t* w2c, const uint8_t* w2s, const float* gsc, const uint8_t* hq,
                               const uint8_t* hsf, const int32_t* counts, const int32_t* offsets, const int2* tiles,
                               const int32_t* num_tiles, int max_tiles, int rows_hint, int H, int I, int E,
                               int hrows, uint16_t* y, hipStream_t stream);

// Stages S2 and S3 of the NVFP4 type (gemm_nv.hip): the weight-streaming
// GEMMs on the dense bf16 MFMA, any rows per expert (passes of 16 rows, or of
// kNvStreamRows with two token tiles).  gsc: the prepared tensor scales
// [g_w1[E], g_w2[E], g_x, g_h] on the device.  hsf holds the scale bytes of h
// in dword planes: unit u's two bytes of sorted row p at ((u/2) * hrows + p)
// * 4 + (u%2) * 2.
hipError_t launch_gemm1_nv(const uint8_t* w1_codes, const uint8_t* w1_scales, const float* gsc, const uint8_t* xq,
                           const uint8_t* xsf, const int32_t* counts, const int32_t* offsets,
                           const int32_t* sorted_rows, int H, int I, int E, int k, int rows_hint, int hrows,
                           uint8_t* hq, uint8_t* hsf, float* acc_out, hipStream_t stream);
hipError_t launch_gemm2_nv(const uint8_t* w2_codes, const uint8_t* w2_scales, const float* gsc, const uint8_t* hq,
                           const uint8_t* hsf, const int32_t* counts, const int32_t* offsets, int H, int I, int E,
                           int rows_hint, int hrows, uint16_t* y, hipStream_t stream);

// Stage S4: top-k weighted combine back to token order, bf16 output.
hipError_t launch_combine(const uint16_t* y, const int32_t* pos, const float* w, int T, int H, int k,
                          uint16_t* out, hipStream_t stream);

// Stage S0: canonical MXFP4 weights -> device tile order.
hipError_t launch_prepare(const uint8_t* w1c, const uint8_t* w1s, const uint8_t* w2c,
                          const uint8_t* w2s, int H, int I, int E, uint8_t* p_w1c, uint8_t* p_w1s,
                          uint8_t* p_w2c, uint8_t* p_w2s, hipStream_t stream);
// The same for NVFP4 weights (scale bytes per 16, nvfp4.h), and the tensor
// scales into gsc = [g_w1[E], g_w2[E], g_x, g_h].
hipError_t launch_prepare_nv(const uint8_t* w1c, const uint8_t* w1s, const float* gw1, const uint8_t* w2c,
                             const uint8_t* w2s, const float* gw2, float gx, float gh, int H, int I, int E,
                             uint8_t* p_w1c, uint8_t* p_w1s, uint8_t* p_w2c, uint8_t* p_w2s, float* gsc,
                             hipStream_t stream);

}  // namespace moe

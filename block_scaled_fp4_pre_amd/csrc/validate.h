// Host-side argument checks and buffer layouts of the C ABI (moe_w4a4.h).
//
// Plain C++ with no HIP dependency: abi.cpp runs these checks before it makes
// any HIP call, and the CPU tests build this file on its own with the host
// address and undefined-behaviour sanitizers and drive every error path
// through it.  Each check returns MOE_OK or the status code the ABI returns.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "moe_w4a4.h"

namespace moe {

constexpr int kMaxExperts = 512;
constexpr int kMaxTopk = 16;
constexpr int kRouteRowsPerBlock = 1024;   // rows per block of the multi-block route (per-block histograms)

// NVFP4 (MOE_MMA_NVF4_X_NVF4): token rows per pass of its streaming GEMMs
// with two token tiles, and the longest K (hidden or inter) whose token tile
// (rows * (K/2 code bytes + K/16 scale bytes)) fits a CU's 160 KiB of LDS.
constexpr int kNvStreamRows = 24;
constexpr int kNvMaxK = 12032;
// Range of an NVFP4 tensor scale: every fp32 step of the encoding stays finite.
constexpr float kNvScaleMin = 0x1p-100f;
constexpr float kNvScaleMax = 0x1p100f;

// The single-launch forward (mega.hip): MXFP4 x MXFP4 or fp8xfp4, at most
// kMegaMaxRows routed rows (num_tokens * topk; one thread each in the
// workgroup's own route), hidden and inter each 512, 1024, 2048 or kMegaMaxK
// (each of a work item's 4 waves takes a quarter of K: 1, 2, 4 or 8 steps of
// 128, the slice lengths the kernel is built for).
constexpr int kMegaMaxRows = MOE_MEGA_MAX_ROWS;
constexpr int kMegaMaxK = 4096;
// Ticket counters per work phase of the single-launch forward.
constexpr int kMegaQueues = 16;
// Its state region, the first region of every workspace whatever the
// configuration (so that it stays put in the allocation-free forward's
// scratch): queue, done and error words, one h counter per expert, and one
// combine counter per (token, 64 hidden columns).
constexpr uint64_t kMegaStateBytes = MOE_MEGA_STATE_BYTES;
bool mega_shape_ok(const moe_w4a4_cfg* c);     // c must pass check_cfg
// MOE_OK when the single-launch forward supports cfg and num_tokens (c must
// pass check_cfg), else MOE_EUNSUPPORTED.
int check_mega_args(const moe_w4a4_cfg* c, int32_t num_tokens);

// Bytes after the last region of the prepared weights.  The streaming GEMMs
// keep a ring of up to 4 K steps of weight loads in flight per wave and issue
// the ring's refills past a unit's last step without a branch; for the last
// unit of the last expert those loads (never consumed) read up to 4 steps of
// 16 KiB past the end of the codes, into the following regions and this tail.
constexpr uint64_t kPreparedTailBytes = 64 * 1024;

// Region offsets of the prepared weights (256-byte aligned), tail included in
// total.  gsc: the NVFP4 tensor scales, fp32 [g_w1[E], g_w2[E], g_x, g_h]
// (empty for the MX types).
struct PreparedLayout {
  uint64_t w1c, w1s, w2c, w2s, gsc, total;
};

// Elements per scale byte of cfg's MMA type: 16 for NVFP4, else 32.
inline int scale_group(const moe_w4a4_cfg* c) { return c->mma_type == MOE_MMA_NVF4_X_NVF4 ? 16 : 32; }

int check_cfg(const moe_w4a4_cfg* c);
PreparedLayout prepared_layout(const moe_w4a4_cfg* c);      // c must pass check_cfg
moe_w4a4_ws_layout ws_layout(const moe_w4a4_cfg* c);        // c must pass check_cfg

// Arguments of moe_w4a4_quantize.  *noop is set when there is nothing to
// enqueue (rows == 0) and the call returns MOE_OK.
int check_quantize_args(int32_t src_dtype, const void* src, int64_t rows, int32_t cols, const void* codes,
                        const void* scales, bool* noop);

// An NVFP4 tensor scale passed by value: finite and in [kNvScaleMin, kNvScaleMax].
bool nv_scale_ok(float g);

// Arguments of moe_w4a4_prepare_weights (MX types only).
int check_prepare_args(const moe_w4a4_cfg* cfg, const void* w1_codes, const void* w1_scales,
                       const void* w2_codes, const void* w2_scales, const void* prepared, size_t prepared_bytes);

// Arguments of moe_w4a4_prepare_weights_nvfp4 (NVFP4 configurations only).
int check_prepare_nv_args(const moe_w4a4_cfg* cfg, const void* w1_codes, const void* w1_scales,
                          const void* w1_tensor_scales, const void* w2_codes, const void* w2_scales,
                          const void* w2_tensor_scales, float x_tensor_scale, float h_tensor_scale,
                          const void* prepared, size_t prepared_bytes);

// Arguments of moe_w4a4_run_stages (and so of moe_w4a4_forward, which runs
// every stage).  *noop is set when there is nothing to enqueue (no tokens or
// no stages) and the call returns MOE_OK without looking at any pointer.
int check_stage_args(const moe_w4a4_cfg* cfg, const void* prepared, int32_t num_tokens, const void* x,
                     const void* topk_ids, const void* topk_weights, const void* out, const void* workspace,
                     size_t workspace_bytes, uint32_t stages, const void* gemm1_acc, bool* noop);

}  // namespace moe

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

// Bytes after the last region of the prepared weights.  The streaming GEMMs
// keep a ring of up to 4 K steps of weight loads in flight per wave and issue
// the ring's refills past a unit's last step without a branch; for the last
// unit of the last expert those loads (never consumed) read up to 4 steps of
// 16 KiB past the end of the codes, into the following regions and this tail.
constexpr uint64_t kPreparedTailBytes = 64 * 1024;

// Region offsets of the prepared weights (256-byte aligned), tail included in total.
struct PreparedLayout {
  uint64_t w1c, w1s, w2c, w2s, total;
};

int check_cfg(const moe_w4a4_cfg* c);
PreparedLayout prepared_layout(const moe_w4a4_cfg* c);      // c must pass check_cfg
moe_w4a4_ws_layout ws_layout(const moe_w4a4_cfg* c);        // c must pass check_cfg

// Arguments of moe_w4a4_quantize.  *noop is set when there is nothing to
// enqueue (rows == 0) and the call returns MOE_OK.
int check_quantize_args(int32_t src_dtype, const void* src, int64_t rows, int32_t cols, const void* codes,
                        const void* scales, bool* noop);

// Arguments of moe_w4a4_prepare_weights.
int check_prepare_args(const moe_w4a4_cfg* cfg, const void* w1_codes, const void* w1_scales,
                       const void* w2_codes, const void* w2_scales, const void* prepared, size_t prepared_bytes);

// Arguments of moe_w4a4_run_stages (and so of moe_w4a4_forward, which runs
// every stage).  *noop is set when there is nothing to enqueue (no tokens or
// no stages) and the call returns MOE_OK without looking at any pointer.
int check_stage_args(const moe_w4a4_cfg* cfg, const void* prepared, int32_t num_tokens, const void* x,
                     const void* topk_ids, const void* topk_weights, const void* out, const void* workspace,
                     size_t workspace_bytes, uint32_t stages, const void* gemm1_acc, bool* noop);

}  // namespace moe

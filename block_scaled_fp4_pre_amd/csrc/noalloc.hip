// moe_w4a4_forward_noalloc: the forward for callers that cannot allocate
// device memory (code under HIP graph capture, serving loops, harnesses that
// forbid hipMalloc).  Its workspace is `scratch`, a file-scope device array of
// MOE_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds until the
// process ends.
//
// In host code `scratch` names a host-side stand-in, not the device array, so
// it is never passed to a kernel or a copy.  On the first call on a device
// (with that device current) its device address is looked up once with
// hipGetSymbolAddress and kept per device; each GPU has its own copy of the
// array at its own address.
//
// Nothing in the workspace has to start at zero: every stage writes the
// regions it reads later in the same forward (counts, offsets, the tile list
// and the histograms included), so the array keeps whatever the previous call
// left.  Calls that overlap on one GPU share the array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"
#include "moe_w4a4.h"
#include "validate.h"

static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];   // device address of `scratch` on each device, once looked up

// The current device's copy of `scratch`, looked up on first use.
int device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ENODEVICE;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MOE_EHIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

extern "C" int moe_w4a4_forward_noalloc(const moe_w4a4_cfg* cfg, const void* prepared, int32_t num_tokens,
                                        const uint16_t* x, const int32_t* topk_ids, const float* topk_weights,
                                        uint16_t* out, void* stream) {
  int st = moe::check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (num_tokens < 0) return MOE_EINVAL;
  if (num_tokens > cfg->max_tokens) return MOE_ECAPACITY;
  if (num_tokens == 0) return MOE_OK;
  // The workspace is laid out for the live token count only.
  moe_w4a4_cfg live = *cfg;
  live.max_tokens = num_tokens;
  const size_t need = (size_t)moe::ws_layout(&live).total;
  if (need > kScratchBytes) return MOE_ESCRATCH;
  bool noop = false;
  // Pointer checks with a stand-in workspace address (aligned, never used).
  st = moe::check_stage_args(&live, prepared, num_tokens, x, topk_ids, topk_weights, out,
                             reinterpret_cast<const void*>(uintptr_t(256)), need, MOE_STAGE_ALL, nullptr, &noop);
  if (st != MOE_OK || noop) return st;
  st = moe::check_device();
  if (st != MOE_OK) return st;
  void* ws = nullptr;
  st = device_scratch(&ws);
  if (st != MOE_OK) return st;
  return moe_w4a4_forward(&live, prepared, num_tokens, x, topk_ids, topk_weights, out, ws, need, stream);
}

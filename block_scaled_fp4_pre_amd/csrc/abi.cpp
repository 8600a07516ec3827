// C ABI of the W4A4 MoE layer (declared in include/moe_w4a4.h): argument
// validation on the host, workspace/prepared layouts, and the stage sequence.
// The pages' interface ([P3] prhub digest of sglang PR "bump sgl-deep-gemm to
// 0.1.7, MegaMoE uses the mma_type API for MXFP4", "Key source snippets") is a
// Python one: a buffer factory keyed by (tokens capacity, experts, topk,
// hidden, inter, mma_type) with activation="swiglu", a pre_dispatch call that
// takes the live num_tokens and group_size=32, and a weight transform.  Here
// the buffer is a caller-owned workspace sized by moe_w4a4_query and the types
// are explicit integers; nothing is cached across calls except whether a device
// is a gfx950.
#include <hip/hip_runtime.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "moe_w4a4.h"
#include "launch.h"
#include "validate.h"

namespace {

constexpr int kMaxDevices = 64;
#ifndef MOE_STREAM_MAX_ROWS
#define MOE_STREAM_MAX_ROWS 16   // mean routed rows per expert up to which the VGPR-streaming GEMMs run
#endif
constexpr int kStreamMaxRows = MOE_STREAM_MAX_ROWS;
// Polls of a wait in the single-launch forward before it gives up: about a
// microsecond each (a sleep of 64 cycles and a load from memory), so about
// 0.1 s, against waits of a few to a few hundred microseconds.
constexpr uint32_t kMegaPollLimit = 1u << 16;

std::atomic<int> g_is_gfx950[kMaxDevices];  // 0 unknown, 1 yes, 2 no

inline int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

}  // namespace

namespace moe {

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MOE_ENODEVICE;
  if (dev < kMaxDevices) {
    const int known = g_is_gfx950[dev].load(std::memory_order_relaxed);
    if (known != 0) return known == 1 ? MOE_OK : MOE_ENODEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_ENODEVICE;
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_is_gfx950[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? MOE_OK : MOE_ENODEVICE;
}

hipError_t raise_lds_limit(const void* kernel, size_t bytes) {
  struct Entry { const void* kernel; int device; size_t bytes; };
  static std::mutex mu;
  static Entry done[64];
  static int ndone = 0;
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < ndone; ++i)
    if (done[i].kernel == kernel && done[i].device == dev && done[i].bytes >= bytes) return hipSuccess;
  err = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (err == hipSuccess && ndone < 64) done[ndone++] = Entry{kernel, dev, bytes};
  return err;
}

}  // namespace moe

extern "C" {

const char* moe_w4a4_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument (null or misaligned pointer, or negative size)";
    case MOE_EUNSUPPORTED: return "unsupported configuration (shape, group size, mma_type or activation)";
    case MOE_ECAPACITY: return "num_tokens exceeds the configured max_tokens";
    case MOE_EWORKSPACE: return "buffer smaller than moe_w4a4_query requires";
    case MOE_ENODEVICE: return "current HIP device is not a gfx950";
    case MOE_EHIP: return "HIP runtime call or kernel launch failed";
    case MOE_ESCRATCH:
      return "the forward needs more workspace than the library's static scratch; "
             "use moe_w4a4_forward with a caller-owned workspace";
    default: return "unknown status";
  }
}

int moe_w4a4_query(const moe_w4a4_cfg* cfg, size_t* prepared_bytes, size_t* workspace_bytes) {
  const int st = moe::check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (prepared_bytes) *prepared_bytes = (size_t)moe::prepared_layout(cfg).total;
  if (workspace_bytes) *workspace_bytes = (size_t)moe::ws_layout(cfg).total;
  return MOE_OK;
}

int moe_w4a4_workspace_layout(const moe_w4a4_cfg* cfg, moe_w4a4_ws_layout* out) {
  const int st = moe::check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (out == nullptr) return MOE_EINVAL;
  *out = moe::ws_layout(cfg);
  return MOE_OK;
}

int moe_w4a4_quantize(int32_t src_dtype, const void* src, int64_t rows, int32_t cols, uint8_t* codes,
                      uint8_t* scales, void* stream) {
  bool noop = false;
  const int st = moe::check_quantize_args(src_dtype, src, rows, cols, codes, scales, &noop);
  if (st != MOE_OK || noop) return st;
  const int dv = moe::check_device();
  if (dv != MOE_OK) return dv;
  return hip_status(moe::launch_quantize(src_dtype == 0, false, src, rows * (int64_t)(cols / 32), codes, scales,
                                         static_cast<hipStream_t>(stream)));
}

int moe_w4a4_quantize_nvfp4(int32_t src_dtype, const void* src, int64_t rows, int32_t cols, float g,
                            uint8_t* codes, uint8_t* scales, void* stream) {
  bool noop = false;
  const int st = moe::check_quantize_args(src_dtype, src, rows, cols, codes, scales, &noop);
  if (st != MOE_OK) return st;
  if (!moe::nv_scale_ok(g)) return MOE_EINVAL;
  if (noop) return MOE_OK;
  const int dv = moe::check_device();
  if (dv != MOE_OK) return dv;
  return hip_status(moe::launch_quantize_nv(src_dtype == 0, src, rows * (int64_t)(cols / 32), g, nullptr, codes,
                                            scales, static_cast<hipStream_t>(stream)));
}

int moe_w4a4_prepare_weights_nvfp4(const moe_w4a4_cfg* cfg, const uint8_t* w1_codes, const uint8_t* w1_scales,
                                   const float* w1_tensor_scales, const uint8_t* w2_codes, const uint8_t* w2_scales,
                                   const float* w2_tensor_scales, float x_tensor_scale, float h_tensor_scale,
                                   void* prepared, size_t prepared_bytes, void* stream) {
  int st = moe::check_prepare_nv_args(cfg, w1_codes, w1_scales, w1_tensor_scales, w2_codes, w2_scales,
                                      w2_tensor_scales, x_tensor_scale, h_tensor_scale, prepared, prepared_bytes);
  if (st != MOE_OK) return st;
  st = moe::check_device();
  if (st != MOE_OK) return st;
  const moe::PreparedLayout P = moe::prepared_layout(cfg);
  uint8_t* base = static_cast<uint8_t*>(prepared);
  return hip_status(moe::launch_prepare_nv(w1_codes, w1_scales, w1_tensor_scales, w2_codes, w2_scales,
                                           w2_tensor_scales, x_tensor_scale, h_tensor_scale, cfg->hidden, cfg->inter,
                                           cfg->num_experts, base + P.w1c, base + P.w1s, base + P.w2c, base + P.w2s,
                                           reinterpret_cast<float*>(base + P.gsc), static_cast<hipStream_t>(stream)));
}

int moe_w4a4_prepare_weights(const moe_w4a4_cfg* cfg, const uint8_t* w1_codes, const uint8_t* w1_scales,
                             const uint8_t* w2_codes, const uint8_t* w2_scales, void* prepared,
                             size_t prepared_bytes, void* stream) {
  int st = moe::check_prepare_args(cfg, w1_codes, w1_scales, w2_codes, w2_scales, prepared, prepared_bytes);
  if (st != MOE_OK) return st;
  st = moe::check_device();
  if (st != MOE_OK) return st;
  const moe::PreparedLayout P = moe::prepared_layout(cfg);
  uint8_t* base = static_cast<uint8_t*>(prepared);
  return hip_status(moe::launch_prepare(w1_codes, w1_scales, w2_codes, w2_scales, cfg->hidden, cfg->inter,
                                        cfg->num_experts, base + P.w1c, base + P.w1s, base + P.w2c,
                                        base + P.w2s, static_cast<hipStream_t>(stream)));
}

int moe_w4a4_run_stages(const moe_w4a4_cfg* cfg, const void* prepared, int32_t num_tokens, const uint16_t* x,
                        const int32_t* topk_ids, const float* topk_weights, uint16_t* out, void* workspace,
                        size_t workspace_bytes, uint32_t stages, float* gemm1_acc, void* stream) {
  bool noop = false;
  int st = moe::check_stage_args(cfg, prepared, num_tokens, x, topk_ids, topk_weights, out, workspace,
                                 workspace_bytes, stages, gemm1_acc, &noop);
  if (st != MOE_OK || noop) return st;
  st = moe::check_device();
  if (st != MOE_OK) return st;
  const moe_w4a4_ws_layout L = moe::ws_layout(cfg);

  const int H = cfg->hidden, I = cfg->inter, E = cfg->num_experts, k = cfg->topk;
  const bool fp8 = cfg->mma_type == MOE_MMA_FP8_X_MXF4;   // E4M3 activations
  const bool nv = cfg->mma_type == MOE_MMA_NVF4_X_NVF4;   // NVFP4 activations and weights
  const int act = nv ? 2 : fp8 ? 1 : 0;
  const int T = num_tokens, R = T * k;
  const int rows_hint = (int)(((int64_t)R + E - 1) / E);
  // Few rows per expert: stream each expert's weights once with the whole
  // token tile in LDS.  Many rows, or a K too long for that tile to fit a
  // CU's LDS: tiled GEMMs over a device-built tile list, both operands staged
  // through LDS one K step at a time.  NVFP4's tiled GEMMs pair weight
  // blocks, so they need an even number of blocks (H % 512, I % 256); other
  // NVFP4 shapes stream the weights once per pass of rows (check_cfg bounds K
  // so that the streaming tile fits).
  const bool tiled = nv ? rows_hint > kStreamMaxRows && H % 512 == 0 && I % 256 == 0
                        : rows_hint > kStreamMaxRows || moe::stream_tile_lds(fp8, H, rows_hint) > moe::kCuLdsBytes ||
                              moe::stream_tile_lds(fp8, I, rows_hint) > moe::kCuLdsBytes;
  const int tile_rows = tiled ? moe::lds_tile_rows(rows_hint) : 0;
  const int max_tiles = tiled ? moe::lds_max_tiles(R, E, tile_rows) : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint8_t* xq = ws + L.xq;
  uint8_t* xsf = ws + L.xsf;
  int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  int32_t* sorted_rows = reinterpret_cast<int32_t*>(ws + L.sorted_rows);
  int32_t* pos = reinterpret_cast<int32_t*>(ws + L.pos);
  int32_t* hist = reinterpret_cast<int32_t*>(ws + L.hist);
  int2* tiles = reinterpret_cast<int2*>(ws + L.tiles);
  int32_t* num_tiles = reinterpret_cast<int32_t*>(ws + L.num_tiles);
  uint8_t* xsf_planes = ws + L.xsf_planes;
  const int hrows = cfg->max_tokens * k;   // rows of one K-step plane (routed-row capacity)
  uint8_t* hq = ws + L.hq;
  uint8_t* hsf = ws + L.hsf;
  uint16_t* y = reinterpret_cast<uint16_t*>(ws + L.y);
  const moe::PreparedLayout P = moe::prepared_layout(cfg);
  const uint8_t* pw = static_cast<const uint8_t*>(prepared);
  // NVFP4 tensor scales [g_w1[E], g_w2[E], g_x, g_h] (check_stage_args: prepared
  // is given whenever a stage that reads them runs)
  const float* gsc = nv && pw != nullptr ? reinterpret_cast<const float*>(pw + P.gsc) : nullptr;
  const float* gx = gsc != nullptr ? gsc + 2 * E : nullptr;

  if ((stages & MOE_STAGE_QUANT) && (stages & MOE_STAGE_ROUTE) && R <= moe::kPredispatchMaxRows) {
    // pre-dispatch in one launch: one block routes, the others quantize
    st = hip_status(moe::launch_predispatch(act, x, (int64_t)T * (H / 32), gx, xq, xsf, topk_ids, R, E, counts,
                                            offsets, sorted_rows, pos, tile_rows, tiles, num_tiles, s));
    if (st != MOE_OK) return st;
  } else {
    if (stages & MOE_STAGE_QUANT) {
      st = hip_status(nv ? moe::launch_quantize_nv(true, x, (int64_t)T * (H / 32), 0.0f, gx, xq, xsf, s)
                         : moe::launch_quantize(true, fp8, x, (int64_t)T * (H / 32), xq, xsf, s));
      if (st != MOE_OK) return st;
    }
    if (stages & MOE_STAGE_ROUTE) {
      st = hip_status(
          moe::launch_route(topk_ids, R, E, hist, counts, offsets, sorted_rows, pos, tile_rows, tiles, num_tiles, s));
      if (st != MOE_OK) return st;
    }
  }
  if ((stages & MOE_STAGE_ROUTE) && tiled) {
    // the tiled GEMM1's token scales, in the sorted order the route just fixed
    st = hip_status(moe::launch_sorted_scales(xsf, sorted_rows, offsets, E, R, H / (nv ? 64 : 128), k, hrows,
                                              xsf_planes, s));
    if (st != MOE_OK) return st;
  }
  if ((stages & MOE_STAGE_GEMM1) && nv) {
    st = hip_status(tiled ? moe::launch_gemm1_lds_nv(pw + P.w1c, pw + P.w1s, gsc, xq, xsf_planes, counts, offsets,
                                                     sorted_rows, tiles, num_tiles, max_tiles, rows_hint, H, I, E, k,
                                                     hrows, hq, hsf, gemm1_acc, s)
                          : moe::launch_gemm1_nv(pw + P.w1c, pw + P.w1s, gsc, xq, xsf, counts, offsets, sorted_rows,
                                                 H, I, E, k, rows_hint, hrows, hq, hsf, gemm1_acc, s));
    if (st != MOE_OK) return st;
  } else if (stages & MOE_STAGE_GEMM1) {
    st = hip_status(tiled ? moe::launch_gemm1_lds(fp8, pw + P.w1c, pw + P.w1s, xq, xsf_planes, counts, offsets,
                                                  sorted_rows, tiles, num_tiles, max_tiles, rows_hint, H, I, k,
                                                  hrows, hq, hsf, gemm1_acc, s)
                          : moe::launch_gemm1(fp8, pw + P.w1c, pw + P.w1s, xq, xsf, counts, offsets, sorted_rows,
                                              H, I, E, k, rows_hint, hrows, hq, hsf, gemm1_acc, s));
    if (st != MOE_OK) return st;
  }
  if ((stages & MOE_STAGE_GEMM2) && nv) {
    st = hip_status(tiled ? moe::launch_gemm2_lds_nv(pw + P.w2c, pw + P.w2s, gsc, hq, hsf, counts, offsets, tiles,
                                                     num_tiles, max_tiles, rows_hint, H, I, E, hrows, y, s)
                          : moe::launch_gemm2_nv(pw + P.w2c, pw + P.w2s, gsc, hq, hsf, counts, offsets, H, I, E,
                                                 rows_hint, hrows, y, s));
    if (st != MOE_OK) return st;
  } else if (stages & MOE_STAGE_GEMM2) {
    st = hip_status(tiled ? moe::launch_gemm2_lds(fp8, pw + P.w2c, pw + P.w2s, hq, hsf, counts, offsets, tiles,
                                                  num_tiles, max_tiles, rows_hint, H, I, hrows, y, s)
                          : moe::launch_gemm2(fp8, pw + P.w2c, pw + P.w2s, hq, hsf, counts, offsets, H, I, E,
                                              rows_hint, hrows, y, s));
    if (st != MOE_OK) return st;
  }
  if (stages & MOE_STAGE_COMBINE) {
    st = hip_status(moe::launch_combine(y, pos, topk_weights, T, H, k, out, s));
    if (st != MOE_OK) return st;
  }
  return MOE_OK;
}

int moe_w4a4_forward_mega(const moe_w4a4_cfg* cfg, const void* prepared, int32_t num_tokens, const uint16_t* x,
                          const int32_t* topk_ids, const float* topk_weights, uint16_t* out, void* workspace,
                          size_t workspace_bytes, void* stream) {
  bool noop = false;
  int st = moe::check_stage_args(cfg, prepared, num_tokens, x, topk_ids, topk_weights, out, workspace,
                                 workspace_bytes, MOE_STAGE_ALL, nullptr, &noop);
  if (st != MOE_OK) return st;
  st = moe::check_mega_args(cfg, num_tokens);
  if (st != MOE_OK || noop) return st;
  st = moe::check_device();
  if (st != MOE_OK) return st;
  const moe_w4a4_ws_layout L = moe::ws_layout(cfg);
  const moe::PreparedLayout P = moe::prepared_layout(cfg);
  const uint8_t* pw = static_cast<const uint8_t*>(prepared);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  return hip_status(moe::launch_mega(
      pw + P.w1c, pw + P.w1s, pw + P.w2c, pw + P.w2s, x, topk_ids, topk_weights, out, num_tokens, cfg->hidden,
      cfg->inter, cfg->num_experts, cfg->topk, cfg->max_tokens * cfg->topk, ws + L.xq, ws + L.xsf, ws + L.hq,
      ws + L.hsf, reinterpret_cast<uint16_t*>(ws + L.y), reinterpret_cast<uint64_t*>(ws + L.mega),
      reinterpret_cast<int32_t*>(ws + L.counts), reinterpret_cast<int32_t*>(ws + L.offsets),
      reinterpret_cast<int32_t*>(ws + L.sorted_rows), reinterpret_cast<int32_t*>(ws + L.pos),
      cfg->mma_type == MOE_MMA_FP8_X_MXF4, kMegaPollLimit, static_cast<hipStream_t>(stream)));
}

int moe_w4a4_forward(const moe_w4a4_cfg* cfg, const void* prepared, int32_t num_tokens, const uint16_t* x,
                     const int32_t* topk_ids, const float* topk_weights, uint16_t* out, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (cfg != nullptr && moe::check_cfg(cfg) == MOE_OK && moe::check_mega_args(cfg, num_tokens) == MOE_OK &&
      (int64_t)num_tokens * cfg->topk <=
          (cfg->mma_type == MOE_MMA_FP8_X_MXF4 ? MOE_MEGA_AUTO_ROWS_FP8 : MOE_MEGA_AUTO_ROWS))
    return moe_w4a4_forward_mega(cfg, prepared, num_tokens, x, topk_ids, topk_weights, out, workspace,
                                 workspace_bytes, stream);
  return moe_w4a4_run_stages(cfg, prepared, num_tokens, x, topk_ids, topk_weights, out, workspace,
                             workspace_bytes, MOE_STAGE_ALL, nullptr, stream);
}

}  // extern "C"

// Host-side argument checks and buffer layouts of the C ABI (validate.h).
// The supported configurations, status codes and pointer rules are the ones
// include/moe_w4a4.h documents: the pages' buffer factory ([P3] prhub digest
// of sglang PR "bump sgl-deep-gemm to 0.1.7, MegaMoE uses the mma_type API for
// MXFP4", "Key source snippets": capacity, experts, topk, hidden, inter,
// mma_type, activation="swiglu", group_size=32) made into explicit integers.
#include "validate.h"

namespace moe {
namespace {

inline uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }
inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace

int check_cfg(const moe_w4a4_cfg* c) {
  if (c == nullptr) return MOE_EINVAL;
  if (c->hidden <= 0 || c->inter <= 0 || c->num_experts <= 0 || c->topk <= 0 || c->max_tokens < 0)
    return MOE_EINVAL;
  if (c->hidden % 256 != 0 || c->inter % 128 != 0) return MOE_EUNSUPPORTED;
  if (c->hidden > (1 << 16) || c->inter > (1 << 16)) return MOE_EUNSUPPORTED;
  if (c->num_experts > kMaxExperts || c->topk > kMaxTopk) return MOE_EUNSUPPORTED;
  const bool mx = c->mma_type == MOE_MMA_MXF4_X_MXF4 || c->mma_type == MOE_MMA_FP8_X_MXF4;
  const bool nv = c->mma_type == MOE_MMA_NVF4_X_NVF4;
  if (!(mx && c->group_size == 32) && !(nv && c->group_size == 16)) return MOE_EUNSUPPORTED;
  if (c->activation != MOE_ACT_SWIGLU) return MOE_EUNSUPPORTED;
  if (nv && (c->hidden > kNvMaxK || c->inter > kNvMaxK)) return MOE_EUNSUPPORTED;
  if ((int64_t)c->max_tokens * c->topk >= (int64_t)1 << 31) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

PreparedLayout prepared_layout(const moe_w4a4_cfg* c) {
  const uint64_t H = c->hidden, I = c->inter, E = c->num_experts, G = scale_group(c);
  PreparedLayout p{};
  uint64_t off = 0;
  p.w1c = off; off = align256(off + E * 2 * I * H / 2);
  p.w1s = off; off = align256(off + E * 2 * I * H / G);
  p.w2c = off; off = align256(off + E * H * I / 2);
  p.w2s = off; off = align256(off + E * H * I / G);
  p.gsc = off; off = align256(off + (c->mma_type == MOE_MMA_NVF4_X_NVF4 ? (2 * E + 2) * 4 : 0));
  p.total = off + kPreparedTailBytes;
  return p;
}

// Hidden and inter of 512, 1024, 2048 or 4096: K splits into 4 slices of 1,
// 2, 4 or 8 steps of 128, the slice lengths the kernel is built for.
static bool mega_k_ok(int64_t K) { return K >= 512 && K <= kMegaMaxK && (K & (K - 1)) == 0; }

bool mega_shape_ok(const moe_w4a4_cfg* c) {
  return (c->mma_type == MOE_MMA_MXF4_X_MXF4 || c->mma_type == MOE_MMA_FP8_X_MXF4) && mega_k_ok(c->hidden) &&
         mega_k_ok(c->inter);
}

int check_mega_args(const moe_w4a4_cfg* c, int32_t num_tokens) {
  if (!mega_shape_ok(c) || (int64_t)num_tokens * c->topk > kMegaMaxRows) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

moe_w4a4_ws_layout ws_layout(const moe_w4a4_cfg* c) {
  const uint64_t H = c->hidden, I = c->inter, E = c->num_experts, M = c->max_tokens, G = scale_group(c);
  const uint64_t R = M * c->topk;
  const uint64_t nb = (R + kRouteRowsPerBlock - 1) / kRouteRowsPerBlock;
  moe_w4a4_ws_layout L{};
  uint64_t off = 0;
  // First and of one size for every configuration, so that it stays put in
  // the allocation-free forward's scratch, which is laid out per call.
  L.mega = off; off = align256(off + kMegaStateBytes);
  const uint64_t ab = c->mma_type == MOE_MMA_FP8_X_MXF4 ? 2 : 1;   // activation bytes per 2 elements
  L.xq = off; off = align256(off + M * H / 2 * ab);
  L.xsf = off; off = align256(off + M * H / G);
  L.counts = off; off = align256(off + E * 4);
  L.offsets = off; off = align256(off + (E + 1) * 4);
  L.sorted_rows = off; off = align256(off + R * 4);
  L.pos = off; off = align256(off + R * 4);
  L.hist = off; off = align256(off + nb * E * 4);
  L.hq = off; off = align256(off + R * I / 2 * ab);
  L.hsf = off; off = align256(off + R * I / G);
  L.y = off; off = align256(off + R * H * 2);
  L.tiles = off; off = align256(off + (R / 16 + E + 1) * 8);
  L.num_tiles = off; off = align256(off + 4);
  L.xsf_planes = off; off = align256(off + R * H / G);
  L.total = off;
  return L;
}

int check_quantize_args(int32_t src_dtype, const void* src, int64_t rows, int32_t cols, const void* codes,
                        const void* scales, bool* noop) {
  *noop = false;
  if (src_dtype != 0 && src_dtype != 1) return MOE_EUNSUPPORTED;
  if (rows < 0 || cols <= 0) return MOE_EINVAL;
  if (cols % 32 != 0) return MOE_EUNSUPPORTED;
  if (rows == 0) {
    *noop = true;
    return MOE_OK;
  }
  if (src == nullptr || codes == nullptr || scales == nullptr) return MOE_EINVAL;
  if (!aligned(src, 16) || !aligned(codes, 16)) return MOE_EINVAL;
  // one thread per 32-group: the group count must fit the launch's index range
  if (rows > (int64_t)1 << 40 || rows * (int64_t)(cols / 32) >= (int64_t)1 << 40) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

bool nv_scale_ok(float g) { return g >= kNvScaleMin && g <= kNvScaleMax; }   // false for NaN

int check_prepare_args(const moe_w4a4_cfg* cfg, const void* w1_codes, const void* w1_scales,
                       const void* w2_codes, const void* w2_scales, const void* prepared, size_t prepared_bytes) {
  const int st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (cfg->mma_type == MOE_MMA_NVF4_X_NVF4) return MOE_EUNSUPPORTED;   // moe_w4a4_prepare_weights_nvfp4
  if (!w1_codes || !w1_scales || !w2_codes || !w2_scales || !prepared) return MOE_EINVAL;
  if (!aligned(w1_codes, 16) || !aligned(w2_codes, 16) || !aligned(prepared, 256)) return MOE_EINVAL;
  if (prepared_bytes < prepared_layout(cfg).total) return MOE_EWORKSPACE;
  return MOE_OK;
}

int check_prepare_nv_args(const moe_w4a4_cfg* cfg, const void* w1_codes, const void* w1_scales,
                          const void* w1_tensor_scales, const void* w2_codes, const void* w2_scales,
                          const void* w2_tensor_scales, float x_tensor_scale, float h_tensor_scale,
                          const void* prepared, size_t prepared_bytes) {
  const int st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (cfg->mma_type != MOE_MMA_NVF4_X_NVF4) return MOE_EUNSUPPORTED;   // moe_w4a4_prepare_weights
  if (!w1_codes || !w1_scales || !w1_tensor_scales || !w2_codes || !w2_scales || !w2_tensor_scales || !prepared)
    return MOE_EINVAL;
  if (!aligned(w1_codes, 16) || !aligned(w2_codes, 16) || !aligned(prepared, 256) ||
      !aligned(w1_tensor_scales, 4) || !aligned(w2_tensor_scales, 4))
    return MOE_EINVAL;
  if (!nv_scale_ok(x_tensor_scale) || !nv_scale_ok(h_tensor_scale)) return MOE_EINVAL;
  if (prepared_bytes < prepared_layout(cfg).total) return MOE_EWORKSPACE;
  return MOE_OK;
}

int check_stage_args(const moe_w4a4_cfg* cfg, const void* prepared, int32_t num_tokens, const void* x,
                     const void* topk_ids, const void* topk_weights, const void* out, const void* workspace,
                     size_t workspace_bytes, uint32_t stages, const void* gemm1_acc, bool* noop) {
  *noop = false;
  const int st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (num_tokens < 0) return MOE_EINVAL;
  if (num_tokens > cfg->max_tokens) return MOE_ECAPACITY;
  if ((stages & ~uint32_t(MOE_STAGE_ALL)) != 0) return MOE_EINVAL;
  if (num_tokens == 0 || stages == 0) {     // nothing to do; empty tensors may be NULL
    *noop = true;
    return MOE_OK;
  }
  if (workspace == nullptr || !aligned(workspace, 256)) return MOE_EINVAL;
  if (workspace_bytes < ws_layout(cfg).total) return MOE_EWORKSPACE;
  if ((stages & MOE_STAGE_QUANT) && (x == nullptr || !aligned(x, 16))) return MOE_EINVAL;
  if ((stages & MOE_STAGE_ROUTE) && (topk_ids == nullptr || !aligned(topk_ids, 4))) return MOE_EINVAL;
  // the GEMMs read the prepared weights; NVFP4's quantization reads its g_x there too
  const uint32_t need_prepared = MOE_STAGE_GEMM1 | MOE_STAGE_GEMM2 |
                                 (cfg->mma_type == MOE_MMA_NVF4_X_NVF4 ? uint32_t(MOE_STAGE_QUANT) : 0u);
  if ((stages & need_prepared) && (prepared == nullptr || !aligned(prepared, 256))) return MOE_EINVAL;
  if ((stages & MOE_STAGE_COMBINE) &&
      (topk_weights == nullptr || out == nullptr || !aligned(topk_weights, 4) || !aligned(out, 16)))
    return MOE_EINVAL;
  if (gemm1_acc != nullptr && !aligned(gemm1_acc, 16)) return MOE_EINVAL;
  return MOE_OK;
}

}  // namespace moe

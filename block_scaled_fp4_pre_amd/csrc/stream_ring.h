// Weight ring of the streaming GEMMs (gemm1.hip, gemm2.hip): each wave keeps
// its next D K steps of weights in VGPRs, one step being four 1 KiB code loads
// (16 bytes per lane each) and one scale dword per lane.
#pragma once
#include "gemm_common.h"
#include "tiles.h"
#include "validate.h"

namespace moe {

// Dynamic LDS of a streaming launch at least this much, so that at most two
// of its 4-wave workgroups share a CU.  At decode sizes most workgroups
// belong to experts without rows and exit at once; the few live ones were
// placed up to four to a CU when their registers and a small token tile
// allowed it, and streamed their weights more slowly than two to a CU: at 8
// tokens (DeepSeek-V4-Flash shape, top-6, MXFP4) the two GEMMs took 99 us
// instead of 132 per layer, at 64 tokens 397 instead of 403; at 512 tokens
// (two token tiles, three to a CU before) the layer took 534 instead of 538.
constexpr size_t kStreamMinLds = 56u << 10;

// Fill the ring with the wave's first D K steps.
// The ring's refills run up to D steps past a wave's last one (gemm1.hip,
// gemm2.hip); the prepared buffer's tail covers them after its last region.
template <int D>
__device__ __forceinline__ void fill_weight_ring(uint4 (&a)[D][4], uint32_t (&sa)[D], __amdgpu_buffer_rsrc_t wr,
                                                 __amdgpu_buffer_rsrc_t sr, int voff, int svoff, int step_stride,
                                                 int scale_stride) {
  static_assert(D * kUnitStepStride <= kPreparedTailBytes, "weight read-ahead past the prepared tail");
#pragma unroll
  for (int d = 0; d < D; ++d) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) a[d][rb] = buf_load16(wr, voff + rb * 1024, d * step_stride);
    sa[d] = buf_load4(sr, svoff, d * scale_stride);
  }
}

}  // namespace moe

// Building blocks shared by the two grouped GEMM kernels (gemm1.hip, gemm2.hip).
//
// Weight stream: each wave walks its unit's tiles (tiles.h) through a buffer
// resource -- lane offset in a VGPR, step offset in an SGPR, block offset as
// the instruction immediate -- into a ring of D register slots, so D steps of
// loads are in flight while the MFMAs consume the oldest slot.  Out-of-range
// buffer reads return zero instead of faulting.
//
// Token tile: the B operand (up to NT*16 token rows of packed codes and their
// scale bytes) is copied into LDS with gfx950 direct-to-LDS loads; each wave
// instruction fills 1 KiB (codes) or 256 B (scales) of contiguous LDS.  Code
// rows are unpadded; the 16-byte chunk c of row n sits at position
// c ^ (n % SWZ) so that the 16 rows read by one MFMA operand load spread over
// the LDS banks.
#pragma once
#include "device_common.h"

namespace moe {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kBufferFlags = 0x00020000;  // raw buffer, 32-bit dwords (gfx9 descriptor word 3)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferFlags);
}

// Cache policy of a weight stream.  The streaming GEMMs read every weight byte
// once per forward and load it non-temporal (NT bit), which measured ~9% more
// sustained read bandwidth on gfx950 than the default policy.
constexpr int kPolicyStream = 2;

template <int CP = kPolicyStream>
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, CP);
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int CP = kPolicyStream>
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, CP);
}

// Direct global -> LDS copy: lane l's 16 (or 4) bytes land at wave_dst + l*16 (l*4).
__device__ __forceinline__ void lds_dma16(const void* src, void* wave_dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)wave_dst, 16, 0, 0);
}
__device__ __forceinline__ void lds_dma4(const void* src, void* wave_dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)wave_dst, 4, 0, 0);
}

// Lets `kernel` use `bytes` (> 64 KiB) of dynamic LDS.  The attribute is per
// kernel and process-wide, so it is set once per (kernel, device) and cached.
hipError_t raise_lds_limit(const void* kernel, size_t bytes);

// Largest power of two <= want that divides units (the units of one expert
// handled by each wave of a 4-wave workgroup).
inline int units_per_wave(int units, int want) {
  int u = 1;
  while (u * 2 <= want && units % (u * 2) == 0) u *= 2;
  return u;
}

__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Swizzle width of the scale rows in LDS: the largest power of two (at most
// 32) dividing the dwords per row.  Row n keeps its step-s dword at position
// s ^ (n % width), so the 16 token rows read by one MFMA scale load hit
// different banks instead of two.
__device__ __forceinline__ int scale_swizzle(int sc_bytes) {
  const int dws = sc_bytes >> 2;
  const int low = dws & (-dws);
  return low > 32 ? 32 : low;
}

// Copy ROWS token rows into LDS.  Row n (n < nrows) is global row
// row_index(n) of `codes` and `scales`: row-major (row_bytes and sc_bytes per
// row) when PLANES is false; in K-step planes of hrows rows when it is true
// (PB code bytes -- 64 for E2M1, 128 for E4M3 -- and one scale dword per row
// and plane; epilogue.h).  sc_bytes is a multiple of 4.  Lanes whose slot lies
// past the last row are masked off, so ROWS * row_bytes need not be a
// multiple of 1024.
template <int ROWS, int SWZ, bool PLANES = false, int PB = 64, class RowIndex>
__device__ __forceinline__ void gather_tile(uint8_t* lds_codes, uint8_t* lds_scales, const uint8_t* codes,
                                            const uint8_t* scales, int row_bytes, int sc_bytes, int nrows,
                                            RowIndex row_index, int wave, int lane, int nwaves, int hrows = 0) {
  const int chunks = row_bytes >> 4;
  const int code_insts = (ROWS * row_bytes + 1023) >> 10;
  for (int j = wave; j < code_insts; j += nwaves) {
    const int slot = j * 64 + lane;
    const int n = slot / chunks, pos = slot - n * chunks;
    const int src = row_index(n);            // evaluated by every lane (it may shuffle)
    if (n < nrows) {
      const int c = pos ^ (n & (SWZ - 1));
      constexpr int CPP = PB / 16;           // 16-byte chunks per plane row
      const size_t off = PLANES ? ((size_t)(c / CPP) * hrows + src) * PB + (c % CPP) * 16
                                : (size_t)src * row_bytes + c * 16;
      lds_dma16(codes + off, lds_codes + j * 1024);
    }
  }
  // Scale dword d of row n sits at position d ^ (n % scale_swizzle(sc_bytes)).
  const int dws = sc_bytes >> 2;
  const int scm = scale_swizzle(sc_bytes) - 1;
  const int sc_total = ROWS * dws;
  for (int j = wave; j * 64 < sc_total; j += nwaves) {
    const int slot = j * 64 + lane;
    const int n = min(slot / dws, ROWS - 1), dpos = slot - (slot / dws) * dws;
    const int src = row_index(n);
    if (slot < sc_total && n < nrows) {
      const int d = dpos ^ (n & scm);
      const size_t off = PLANES ? ((size_t)d * hrows + src) * 4 : (size_t)src * sc_bytes + d * 4;
      lds_dma4(scales + off, lds_scales + j * 256);
    }
  }
}

// Scale byte of step s for token column n and K block kb.
__device__ __forceinline__ int tile_scale(const uint8_t* lds_scales, int sc_bytes, int n, int s, int kb) {
  const int scm = scale_swizzle(sc_bytes) - 1;
  return lds_scales[n * sc_bytes + (s ^ (n & scm)) * 4 + kb];
}

// B operand of step s for token column n (row of the LDS tile) and K block kb.
template <int SWZ>
__device__ __forceinline__ uint4 tile_operand(const uint8_t* lds_codes, int row_bytes, int n, int s, int kb) {
  const int pos = (s * 4 + kb) ^ (n & (SWZ - 1));
  return *reinterpret_cast<const uint4*>(lds_codes + n * row_bytes + pos * 16);
}

// The same for E4M3 codes (one byte per element): lane group kb takes the
// 16-element chunks kb and kb + 4 of step s (the FP8 operand layout,
// device_common.h).
template <int SWZ>
__device__ __forceinline__ void tile_operand8(const uint8_t* lds_codes, int row_bytes, int n, int s, int kb,
                                              uint4& lo, uint4& hi) {
  const int c = s * 8 + kb;
  lo = *reinterpret_cast<const uint4*>(lds_codes + n * row_bytes + (c ^ (n & (SWZ - 1))) * 16);
  hi = *reinterpret_cast<const uint4*>(lds_codes + n * row_bytes + ((c + 4) ^ (n & (SWZ - 1))) * 16);
}

}  // namespace moe

// Device tile order of the prepared expert weights (written by prepare.hip,
// read by gemm1.hip / gemm2.hip).  The GEMMs run "swap-AB": weight rows are the
// 16-row MFMA A operand and token rows the 16-column B operand, so a weight
// tile is read exactly once per pass and needs no LDS.
//
// One wave owns a UNIT of 64 weight rows (four 16-row blocks rb = 0..3) over the
// whole K range, walked in steps of 128.  For each (unit, step):
//   codes : 4 x 1 KiB, block rb at rb * 1024, lane l's 16 bytes at l * 16 --
//           row (l % 16) of block rb, K elements [step*128 + 32*(l/16), +32).
//           One global_load_dwordx4 per block per wave, fully contiguous.
//   scales: 256 B, lane l's dword at l * 4; byte rb = UE8M0 scale of that
//           lane's row of block rb and its 32-element K block (MFMA op_sel rb).
// GEMM1 unit u covers inter columns [32u, 32u+32): blocks 0,1 are gate rows
// 32u..32u+15, 32u+16..32u+31 and blocks 2,3 the up rows with the same
// columns, so gate and up of a column land in the same lane and register.
// GEMM2 unit v covers hidden rows [64v, 64v+64), block rb = rows 64v+16rb...
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kUnitRows = 64;
constexpr int kStepK = 128;
constexpr int kStepCodeBytes = 4 * 1024;
constexpr int kStepScaleBytes = 256;

// GEMM1: units per expert = I / 32, steps = H / 128.
__host__ __device__ inline size_t w1_code_offset(int e, int u, int s, int H, int I) {
  return (((size_t)e * (I / 32) + u) * (H / kStepK) + s) * kStepCodeBytes;
}
__host__ __device__ inline size_t w1_scale_offset(int e, int u, int s, int H, int I) {
  return (((size_t)e * (I / 32) + u) * (H / kStepK) + s) * kStepScaleBytes;
}
// GEMM2: units per expert = H / 64, steps = I / 128.
__host__ __device__ inline size_t w2_code_offset(int e, int v, int s, int H, int I) {
  return (((size_t)e * (H / kUnitRows) + v) * (I / kStepK) + s) * kStepCodeBytes;
}
__host__ __device__ inline size_t w2_scale_offset(int e, int v, int s, int H, int I) {
  return (((size_t)e * (H / kUnitRows) + v) * (I / kStepK) + s) * kStepScaleBytes;
}

}  // namespace moe

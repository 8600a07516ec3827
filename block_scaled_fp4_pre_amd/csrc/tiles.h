// Device tile order of the prepared expert weights (written by prepare.hip,
// read by gemm1.hip / gemm2.hip).  The GEMMs run "swap-AB": weight rows are the
// 16-row MFMA A operand and token rows the 16-column B operand, so a weight
// tile is read exactly once per pass and needs no LDS.
//
// One wave owns a UNIT of 64 weight rows (four 16-row blocks rb = 0..3) over the
// whole K range, walked in steps of 128.  For each (unit, step), one 4 KiB chunk
// of codes and one 256 B chunk of scales:
//   codes : 4 x 1 KiB, block rb at rb * 1024, lane l's 16 bytes at l * 16 --
//           row (l % 16) of block rb, K elements [step*128 + 32*(l/16), +32).
//           One global_load_dwordx4 per block per wave, fully contiguous.
//   scales: 256 B, lane l's dword at l * 4; byte rb = UE8M0 scale of that
//           lane's row of block rb and its 32-element K block (MFMA op_sel rb).
// Chunk order: experts, then groups of 4 consecutive units, then steps, then the
// unit within its group.  The 4 waves of a workgroup own the 4 units of a group,
// so per K step the workgroup reads one contiguous 16 KiB of codes and 1 KiB of
// scales, and each unit's chunks follow each other at a stride of 16 KiB (1 KiB).
// (Contiguous per-workgroup steps measured about 1 % faster for the weight
// streams of the layer at 64 and 512 tokens than one 128 KiB run per unit.)
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
constexpr int kGroupUnits = 4;                                  // units per contiguous group
constexpr int kUnitStepStride = kGroupUnits * kStepCodeBytes;   // one unit, step s -> s + 1
constexpr int kUnitScaleStride = kGroupUnits * kStepScaleBytes;

// Chunk index of (expert e, unit u, step s) for U units per expert and S steps.
__host__ __device__ inline size_t unit_chunk(int e, int u, int s, int U, int S) {
  return (((size_t)e * (U / kGroupUnits) + u / kGroupUnits) * S + s) * kGroupUnits + u % kGroupUnits;
}
// GEMM1: units per expert = I / 32, steps = H / 128.
__host__ __device__ inline size_t w1_code_offset(int e, int u, int s, int H, int I) {
  return unit_chunk(e, u, s, I / 32, H / kStepK) * kStepCodeBytes;
}
__host__ __device__ inline size_t w1_scale_offset(int e, int u, int s, int H, int I) {
  return unit_chunk(e, u, s, I / 32, H / kStepK) * kStepScaleBytes;
}
// GEMM2: units per expert = H / 64, steps = I / 128.
__host__ __device__ inline size_t w2_code_offset(int e, int v, int s, int H, int I) {
  return unit_chunk(e, v, s, H / kUnitRows, I / kStepK) * kStepCodeBytes;
}
__host__ __device__ inline size_t w2_scale_offset(int e, int v, int s, int H, int I) {
  return unit_chunk(e, v, s, H / kUnitRows, I / kStepK) * kStepScaleBytes;
}

}  // namespace moe

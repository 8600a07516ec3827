/* Measurement probes for the MoE layer's rooflines on MI355X (gfx950).
 *
 * Not part of the layer's path.  They measure the two ceilings its kernels are
 * compared against, next to the published peaks (8 TB/s HBM3E, 10.1 PFLOP/s
 * dense FP4):
 *   - moe_ceiling_stream_read: the practical HBM read rate of a plain streaming
 *     read, with the access pattern of the layer's weight streams (each
 *     workgroup reads one contiguous chunk with 16-byte buffer loads, several
 *     in flight per lane);
 *   - moe_ceiling_mfma_fp4 / moe_ceiling_mfma_fp8xfp4: the practical rate of
 *     the block-scaled MFMA (V_MFMA_SCALE_F32_16X16X128_F8F6F4) with both
 *     operands E2M1, or with E2M1 weights and E4M3 tokens (the layer's two MMA
 *     types), issued back to back from register operands;
 *   - moe_ceiling_mfma_bf16: the practical dense bf16 MFMA rate
 *     (V_MFMA_F32_16X16X32_BF16), the rate a block-scaled format whose scales
 *     the f8f6f4 MFMA cannot take (E4M3 block scales, NVFP4) would run at.
 * Each probe writes a result the caller can check exactly, so that a probe
 * that skipped work would be caught.
 *
 * Built as block_scaled_fp4_pre_amd/libmoe_ceiling.so.  Pointers are device
 * pointers owned by the caller; the calls only enqueue on `stream` (no
 * allocation, no synchronization).  Arguments are checked on the host before
 * any HIP call.
 */
#ifndef MOE_CEILING_H
#define MOE_CEILING_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MOE_CEILING_OK = 0,
  MOE_CEILING_EINVAL = 1, /* null pointer, zero count, or sizes that do not divide as stated */
  MOE_CEILING_EHIP = 2    /* the launch failed */
};

/* Read `bytes` bytes at `src` once.  Workgroup g (of `workgroups`, 256 threads
 * each) reads the contiguous chunk [g*c, (g+1)*c), c = bytes / workgroups, and
 * writes to digest[g] the XOR of the chunk's 32-bit little-endian words.
 * non_temporal != 0 sets the non-temporal cache policy on the loads (as the
 * layer's weight streams do).  Requires bytes % (16 * workgroups) == 0 and
 * c < 2^31; src 16-byte aligned; digest holds `workgroups` words. */
int moe_ceiling_stream_read(const void* src, uint64_t bytes, uint32_t workgroups, int non_temporal,
                            uint32_t* digest, hipStream_t stream);

/* `workgroups` workgroups of 4 waves; each wave runs `iterations` rounds of 8
 * independent 16x16x128 FP4 MFMAs (2*16*16*128 flops each) on operands whose
 * every element is 1.0 with unit scales, then writes to out[wave] the sum of
 * element 0 of its 8 accumulators: exactly 8 * 128 * iterations.  Requires
 * 1 <= iterations <= 16384 (the sums stay exact in fp32); out holds
 * 4 * workgroups floats. */
int moe_ceiling_mfma_fp4(uint32_t workgroups, int32_t iterations, float* out, hipStream_t stream);

/* The same with E4M3 B operands (every element 1.0): the fp8xfp4 MMA type's
 * instruction form.  Same result, requirements and flops per MFMA. */
int moe_ceiling_mfma_fp8xfp4(uint32_t workgroups, int32_t iterations, float* out, hipStream_t stream);

/* `workgroups` workgroups of 4 waves; each wave runs `iterations` rounds of 8
 * independent 16x16x32 bf16 MFMAs (2*16*16*32 flops each) on operands whose
 * every element is 1.0, then writes to out[wave] the sum of element 0 of its
 * 8 accumulators: exactly 8 * 32 * iterations.  Requires 1 <= iterations <=
 * 16384; out holds 4 * workgroups floats. */
int moe_ceiling_mfma_bf16(uint32_t workgroups, int32_t iterations, float* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_CEILING_H */

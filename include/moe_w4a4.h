/*
 * moe_w4a4.h -- C ABI of the MI355X (gfx950) W4A4 routed-expert MoE layer.
 *
 * The layer is the fused "mega-MoE" W4A4 layer of a DeepSeek-V4-Flash-shaped
 * model (hidden 4096, inter 2048, 256 experts, top-6): tokens and expert
 * weights are both MXFP4 (E2M1 codes, one UE8M0 scale per 32 elements), or,
 * with the fp8xfp4 mma_type below, the tokens are MXFP8 E4M3; the expert MLP
 * is SwiGLU.  Sources:
 *   [P1] sglang PR "[deepseek-v4] Bump sgl-deep-gemm for packed FP4xFP4
 *        mega-MoE (W4A4)": title (packed FP4 x FP4 operands), Appendix
 *        "measured data" (the layer shape).
 *   [P3] prhub digest of sglang PR "bump sgl-deep-gemm to 0.1.7, MegaMoE uses
 *        the mma_type API for MXFP4": "Key source snippets" (the symmetric
 *        buffer factory with mma_type and activation="swiglu"; the mxf4xmxf4
 *        pre_dispatch call with group_size=32 and a live num_tokens below the
 *        buffer capacity; the gate/up split of the L1 weights), and
 *        "Implementation breakdown" item 4 (weights are transformed once at
 *        load time for the chosen mma_type).
 *   [OCP-MX] OCP Microscaling Formats (MX) v1.0: E2M1 element and E8M0 scale
 *        encodings.
 *   [P3] "Motivation" names an NVFP4 mega-MoE as well; MOE_MMA_NVF4_X_NVF4
 *        below is that variant in the public NVFP4 format (E2M1 elements, an
 *        E4M3 scale per 16 elements, an fp32 scale per tensor).
 *
 * Conventions for every entry point
 *   - Device pointers are allocated and owned by the caller; the library never
 *     allocates, frees or synchronizes, and reads no environment variables.
 *     A call only enqueues work on `stream` (a hipStream_t; NULL = the null
 *     stream), so it can be captured into a HIP graph.
 *   - Arguments are validated on the host before any HIP call; a failed check
 *     returns a status code and enqueues nothing.
 *   - Faults while kernels execute surface at the caller's next synchronization.
 *   - The library keeps only per-device caches (whether the device is a
 *     gfx950, the dynamic-LDS limits it raised for its large-tile kernels,
 *     the address of moe_w4a4_forward_noalloc's static scratch), each behind
 *     a lock or an atomic; calls on different streams with distinct
 *     workspaces may run concurrently (moe_w4a4_forward_noalloc calls share
 *     their GPU's scratch and may not).
 *
 * MXFP4 encoding used throughout ([OCP-MX]; the scale rule is the reading
 * taken where the pages are silent):
 *   code (4 bits): bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa;
 *                  magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
 *   packing:       two codes per byte, the even element in the low nibble.
 *   scale byte b:  value 2^(b-127); for a block with absolute maximum a the
 *                  scale is 2^e with e the smallest integer such that
 *                  a <= 6*2^e, clamped to [-127, 127] (a == 0 gives b = 0).
 *   rounding:      nearest code to v/2^e, ties to the even mantissa; the sign
 *                  bit is copied from v (so -0 encodes as 0x8).
 */
#ifndef MOE_W4A4_H
#define MOE_W4A4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,        /* null or misaligned pointer, negative size            */
  MOE_EUNSUPPORTED = 2,  /* shape, group size, mma_type or activation not built   */
  MOE_ECAPACITY = 3,     /* num_tokens > cfg->max_tokens                          */
  MOE_EWORKSPACE = 4,    /* a buffer is smaller than moe_w4a4_query() requires    */
  MOE_ENODEVICE = 5,     /* the current HIP device is not a gfx950                */
  MOE_EHIP = 6,          /* a HIP runtime call or kernel launch failed            */
  MOE_ESCRATCH = 7       /* moe_w4a4_forward_noalloc: more than its static scratch */
};

/* mma_type: the pairing of activation and weight formats ([P3] "Implementation
 * breakdown" items 1-3: the mma_type that replaced the env-var switches).
 *   MOE_MMA_MXF4_X_MXF4 ("mxf4xmxf4"): x and h are MXFP4 E2M1, two codes a byte.
 *   MOE_MMA_FP8_X_MXF4  ("fp8xfp4"):  x and h are MXFP8 E4M3 ([OCP-MX]), one
 *     code a byte, with the same UE8M0 scale per 32 (scale 2^e: the smallest
 *     with amax <= 448 * 2^e); ties to the even mantissa, sign kept.
 * The weights are MXFP4 in both.
 *   MOE_MMA_NVF4_X_NVF4 ("nvf4xnvf4", group_size 16): x, h and the weights are
 *     NVFP4: E2M1 codes (two a byte, as above), one E4M3 scale byte per 16
 *     elements along K (sign bit clear) and one fp32 tensor scale g per
 *     tensor (x and h per layer, W1 and W2 per expert), value = e2m1 * e4m3
 *     * g.  A block with absolute maximum a gets the E4M3 code nearest to
 *     min(f32(a / f32(6*g)), 448) (ties to even); its codes are the E2M1
 *     codes nearest to f32(v * inv) clamped to [-6, 6], inv = 0 for a zero
 *     scale, else f32(1 / f32(e4m3 * g)) (ties to even, sign kept).  The
 *     GEMMs run the 16-bit MFMA on the exact products e2m1 * e4m3 in
 *     bfloat16 and apply the tensor scales to the fp32 sums.  hidden and
 *     inter are limited to 12032 (the token tile of the weight-streaming
 *     GEMMs, the only ones built for this type, must fit a CU's LDS). */
enum { MOE_MMA_MXF4_X_MXF4 = 0, MOE_MMA_FP8_X_MXF4 = 1, MOE_MMA_NVF4_X_NVF4 = 2 };
/* activation: SwiGLU, silu(gate) * up, with no clamp or bias ([P3]). */
enum { MOE_ACT_SWIGLU = 0 };

/* Layer configuration.  Supported: hidden % 256 == 0, inter % 128 == 0,
 * 1 <= num_experts <= 512, 1 <= topk <= 16, 0 <= max_tokens and
 * max_tokens * topk < 2^31, group_size == 32 for the two MX types and 16 for
 * NVFP4, mma_type one of the three above, activation == MOE_ACT_SWIGLU.  max_tokens is the capacity the workspace is
 * sized for (num_max_tokens_per_rank in [P3]); each forward passes the live
 * token count. */
typedef struct moe_w4a4_cfg {
  int32_t hidden;       /* H */
  int32_t inter;        /* I */
  int32_t num_experts;  /* E */
  int32_t topk;         /* k */
  int32_t max_tokens;   /* capacity */
  int32_t group_size;   /* 32 (MX types) or 16 (NVFP4) */
  int32_t mma_type;     /* MOE_MMA_MXF4_X_MXF4, MOE_MMA_FP8_X_MXF4 or MOE_MMA_NVF4_X_NVF4 */
  int32_t activation;   /* MOE_ACT_SWIGLU */
} moe_w4a4_cfg;

/* Sizes in bytes of the prepared-weights buffer and of the forward workspace
 * for `cfg`.  This is the sizing half of the pages' buffer factory ([P3]
 * "Key source snippets", _get_mega_moe_symm_buffer: one buffer per
 * (num_max_tokens_per_rank, experts, topk, hidden, intermediate_hidden,
 * mma_type, activation), reused by every forward); here the caller allocates
 * what these sizes say.  The prepared size is the four weight regions (with
 * NVFP4 also its tensor scales) plus a 64 KiB tail that the weight streams'
 * read-ahead may touch.  Either output
 * pointer may be NULL.  Pure host function: returns MOE_EINVAL or
 * MOE_EUNSUPPORTED for a configuration moe_w4a4_cfg does not allow, with the
 * outputs untouched. */
int moe_w4a4_query(const moe_w4a4_cfg* cfg, size_t* prepared_bytes, size_t* workspace_bytes);

/* Quantize `rows` rows of `cols` values to MXFP4 along each row.
 * src_dtype: 0 = bfloat16 (uint16 bit patterns), 1 = float32.  Values must be
 * finite.  src: device [rows, cols], 16-byte aligned.  codes: device uint8
 * [rows, cols/2] (packed, 16-byte aligned); scales: device uint8 [rows, cols/32].
 * cols % 32 == 0, rows >= 0.  This is the activation quantizer of the
 * pre-dispatch step ([P3] "Key source snippets": pre_dispatch packs E2M1 with
 * group_size=32) and the load-time quantizer for fp32 expert weights. */
int moe_w4a4_quantize(int32_t src_dtype, const void* src, int64_t rows, int32_t cols,
                      uint8_t* codes, uint8_t* scales, void* stream);

/* NVFP4 quantization of `rows` rows of `cols` values along each row with the
 * tensor scale g (the rule under MOE_MMA_NVF4_X_NVF4 above): codes uint8
 * [rows, cols/2] (packed, 16-byte aligned), scales uint8 [rows, cols/16] (E4M3
 * bytes).  src_dtype, src, rows and cols as for moe_w4a4_quantize (cols % 32
 * == 0).  g must be finite and in [2^-100, 2^100] (else MOE_EINVAL).  The
 * pre-dispatch step of the NVFP4 type uses the same rule for x with the
 * layer's g_x; callers use it to quantize fp32 expert weights at load time.
 * Source: [P3] "Motivation" (the NVFP4 variant) and "Key source snippets"
 * (pre_dispatch quantizes the tokens once, group by group). */
int moe_w4a4_quantize_nvfp4(int32_t src_dtype, const void* src, int64_t rows, int32_t cols, float g,
                            uint8_t* codes, uint8_t* scales, void* stream);

/* Re-lay canonical MXFP4 expert weights into the device tile order used by the
 * forward ([P3] "Implementation breakdown" item 4: a one-off weight transform at
 * load time).  A pure byte permutation.
 *   w1_codes  [E, 2I, H/2], w1_scales [E, 2I, H/32]: rows [0, I) are gate and
 *             rows [I, 2I) are up ([P3] gate/up split of the L1 weights);
 *   w2_codes  [E, H, I/2],  w2_scales [E, H, I/32].
 * All device pointers; codes 16-byte aligned.  prepared: device buffer of at
 * least moe_w4a4_query()'s prepared_bytes, 256-byte aligned; owned by the
 * caller and read by every later forward.  An NVFP4 cfg returns
 * MOE_EUNSUPPORTED (it takes moe_w4a4_prepare_weights_nvfp4). */
int moe_w4a4_prepare_weights(const moe_w4a4_cfg* cfg,
                             const uint8_t* w1_codes, const uint8_t* w1_scales,
                             const uint8_t* w2_codes, const uint8_t* w2_scales,
                             void* prepared, size_t prepared_bytes, void* stream);

/* The same for NVFP4 weights ([P3] "Motivation"; the one-off weight transform
 * of "Implementation breakdown" item 4), for a cfg with MOE_MMA_NVF4_X_NVF4
 * (else MOE_EUNSUPPORTED):
 *   w1_codes [E, 2I, H/2], w1_scales [E, 2I, H/16] (E4M3 bytes),
 *   w1_tensor_scales fp32 [E]; w2_codes [E, H, I/2], w2_scales [E, H, I/16],
 *   w2_tensor_scales fp32 [E] -- device pointers; each tensor scale in
 *   [2^-100, 2^100] (the library cannot read device values on the host: out
 *   of range gives unspecified numbers, never a fault);
 *   x_tensor_scale, h_tensor_scale: g of the layer's activations x and of the
 *   intermediate h (calibration constants: every forward quantizes x and
 *   requantizes h with them), by value, in [2^-100, 2^100] (else MOE_EINVAL).
 * All tensor scales are copied into `prepared`, which the forward then reads
 * on the device. */
int moe_w4a4_prepare_weights_nvfp4(const moe_w4a4_cfg* cfg,
                                   const uint8_t* w1_codes, const uint8_t* w1_scales, const float* w1_tensor_scales,
                                   const uint8_t* w2_codes, const uint8_t* w2_scales, const float* w2_tensor_scales,
                                   float x_tensor_scale, float h_tensor_scale,
                                   void* prepared, size_t prepared_bytes, void* stream);

/* One forward of the layer for num_tokens (0 <= num_tokens <= cfg->max_tokens).
 * It is the routed branch of the pages' MoE runner ([P3] "Key source snippets",
 * _run_mega_routed: pre_dispatch of the bf16 hidden states with topk_ids and
 * topk_weights into the buffer for the live num_tokens, group_size=32, then
 * the fused mega-MoE kernel over the prepared L1/L2 weights), as one call:
 *   1. pre-dispatch: each token row of x quantized once to MXFP4 (MXFP8 E4M3
 *      for MOE_MMA_FP8_X_MXF4, NVFP4 with g_x for MOE_MMA_NVF4_X_NVF4; so is
 *      h in step 3, NVFP4 with g_h);
 *   2. route: stable counting sort of the routed rows r = t*k + j by expert
 *      (ids outside [0, E) are skipped; duplicates are separate rows);
 *   3. GEMM1 per expert with fp32 accumulation, SwiGLU, requantization of h to
 *      MXFP4 along I (NVFP4: the sums times g_x * g_w1[e] before SwiGLU);
 *   4. GEMM2 per expert with fp32 accumulation, the result per routed row
 *      rounded to bfloat16 (NVFP4: the sums times g_h * g_w2[e] first);
 *   5. combine: out[t] = sum over valid slots j (in slot order, fp32, from +0)
 *      of topk_weights[t, j] * y[row (t, j)], rounded to bfloat16.
 * x:            device bfloat16 [num_tokens, H], 16-byte aligned
 * topk_ids:     device int32 [num_tokens, k]
 * topk_weights: device float32 [num_tokens, k], used as given
 * out:          device bfloat16 [num_tokens, H], 16-byte aligned
 * workspace:    device buffer of at least query()'s workspace_bytes, 256-byte
 *               aligned; holds the intermediates (layout: moe_w4a4_workspace_layout)
 * num_tokens == 0 returns MOE_OK and enqueues nothing, without looking at
 * any pointer (empty tensors may have NULL data).  Errors, before anything is
 * enqueued: MOE_EINVAL (a null or misaligned pointer, num_tokens < 0),
 * MOE_ECAPACITY (num_tokens > max_tokens), MOE_EWORKSPACE (workspace_bytes
 * too small), MOE_EUNSUPPORTED (cfg), MOE_ENODEVICE (current device not a
 * gfx950); MOE_EHIP if a launch fails.  The shapes behind the pointers are
 * the caller's promise: the library cannot see them.
 * The result is deterministic: no floating-point atomics, stable sort. */
int moe_w4a4_forward(const moe_w4a4_cfg* cfg, const void* prepared, int32_t num_tokens,
                     const uint16_t* x, const int32_t* topk_ids, const float* topk_weights,
                     uint16_t* out, void* workspace, size_t workspace_bytes, void* stream);

/* The same forward as ONE kernel launch, for decode-sized batches: the pages'
 * single fused mega-MoE kernel ([P1] sglang PR "[deepseek-v4] Bump
 * sgl-deep-gemm for packed FP4xFP4 mega-MoE (W4A4)", title and section B; [P3]
 * "Key source snippets", _run_mega_routed, which runs one fused kernel per
 * forward after pre_dispatch).  Every workgroup routes the top-k ids itself;
 * work items (a 64-row unit of W1 for one expert, which quantizes the token
 * rows it needs; a 64-row unit of W2 for one expert) come from device-side
 * ticket counters, all W1 units before any W2 unit; a W2 item waits for its
 * expert's h through a counter in the workspace; the W2 item that completes a
 * token's 64 hidden columns combines them.
 * Supported: MOE_MMA_MXF4_X_MXF4 and MOE_MMA_FP8_X_MXF4,
 * num_tokens * topk <= MOE_MEGA_MAX_ROWS,
 * hidden and inter each 512, 1024, 2048 or 4096; otherwise MOE_EUNSUPPORTED
 * and nothing is enqueued.  Arguments, other errors and the workspace as for
 * moe_w4a4_forward, plus: the workspace's `mega` region (its first
 * MOE_MEGA_STATE_BYTES) must be zero before the first call on it, and every
 * call leaves it zero (so zero it once after allocating the workspace); calls
 * that share a workspace must not overlap.  A wait inside the kernel that runs
 * out of polls (about 0.1 s; none does unless the state was not zero) sets the
 * error word, uint64 number MOE_MEGA_ERR_WORD of the region, which the kernel
 * never clears; that call's results are then unspecified, and the rest of the
 * region is still left zero.  Words MOE_MEGA_HCOUNT_WORD + e (e < num_experts)
 * hold the per-expert counts that the W2 items wait for (tests force a wait
 * to give up by setting them beforehand).  Afterwards the workspace holds the same
 * intermediates as after moe_w4a4_forward (xq, xsf, counts, offsets,
 * sorted_rows, pos, hq, hsf, y).  Numerics as moe_w4a4_forward except the
 * order of the fp32 sums of both GEMMs (each sum is four partial sums over
 * quarters of K, added in order), so the two paths agree to the parity bar
 * rather than bit for bit; the result is deterministic.
 * moe_w4a4_forward takes this path by itself when it is supported and
 * num_tokens * topk <= MOE_MEGA_AUTO_ROWS (MXFP4) or MOE_MEGA_AUTO_ROWS_FP8
 * (fp8xfp4), the sizes up to which it measured faster than the stage
 * sequence at the DeepSeek-V4-Flash shape. */
#define MOE_MEGA_MAX_ROWS 256
#define MOE_MEGA_AUTO_ROWS 48
#define MOE_MEGA_AUTO_ROWS_FP8 24
#define MOE_MEGA_STATE_BYTES (144u << 10)
#define MOE_MEGA_ERR_WORD 800
#define MOE_MEGA_HCOUNT_WORD 816
int moe_w4a4_forward_mega(const moe_w4a4_cfg* cfg, const void* prepared, int32_t num_tokens,
                          const uint16_t* x, const int32_t* topk_ids, const float* topk_weights,
                          uint16_t* out, void* workspace, size_t workspace_bytes, void* stream);

/* The same forward with no workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The intermediates live in a static
 * device array of the library, MOE_NOALLOC_SCRATCH_BYTES per GPU, which each
 * GPU the library runs on holds until the process ends; its layout is
 * moe_w4a4_workspace_layout of cfg with max_tokens = num_tokens.  Nothing is
 * allocated or freed.  Returns MOE_ESCRATCH, enqueuing nothing, when that
 * layout exceeds the scratch (about 1,100 tokens at hidden 4096, inter 2048,
 * top-6).  Every call on a GPU uses that GPU's one array: calls that overlap on
 * one GPU (other streams, other threads) race and must be serialized by the
 * caller.  Other arguments, results and errors as for moe_w4a4_forward. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int moe_w4a4_forward_noalloc(const moe_w4a4_cfg* cfg, const void* prepared, int32_t num_tokens,
                             const uint16_t* x, const int32_t* topk_ids, const float* topk_weights,
                             uint16_t* out, void* stream);

/* Human-readable text of a status code (static storage). */
const char* moe_w4a4_status_string(int status);

/* ---- inspection and stage-by-stage execution (tests, profiling) -------- */

/* Byte offsets of each intermediate inside the forward workspace; every region
 * is 256-byte aligned and sized for cfg->max_tokens.  R = max_tokens*k.  The
 * sorted-row activations of the GEMMs are stored as K-step planes, plane c
 * holding K step c (128 elements) of every sorted row: 64 code bytes at
 * (c*R + row)*64 and one dword of 4 scale bytes at (c*R + row)*4, so that a
 * tile of consecutive rows reads one contiguous run per K step.  With NVFP4
 * every scale region holds one byte per 16 elements: xsf [max_tokens, H/16],
 * hsf planes of 8 bytes per row ([I/128, R, 8]), xsf_planes unused. */
typedef struct moe_w4a4_ws_layout {
  uint64_t xq;           /* uint8  [max_tokens, H/2]   quantized tokens (packed E2M1;
                                                        E4M3: [max_tokens, H])      */
  uint64_t xsf;          /* uint8  [max_tokens, H/32]  their scale bytes            */
  uint64_t counts;       /* int32  [E]                 routed rows per expert       */
  uint64_t offsets;      /* int32  [E+1]               exclusive prefix of counts   */
  uint64_t sorted_rows;  /* int32  [max_tokens*k]      r = t*k+j in (expert, r) order */
  uint64_t pos;          /* int32  [max_tokens*k]      index of r in sorted_rows or -1 */
  uint64_t hist;         /* int32  [ceil(max_tokens*k/1024), E] per-block counts   */
  uint64_t hq;           /* uint8  [I/128, R, 64]      requantized h (sorted rows, planes;
                                                        E4M3: [I/128, R, 128])      */
  uint64_t hsf;          /* uint8  [I/128, R, 4]       its scale bytes (planes)     */
  uint64_t y;            /* bf16   [max_tokens*k, H]   GEMM2 result (sorted order)  */
  uint64_t tiles;        /* int32  [max_tokens*k/16 + E, 2] (expert, first row) work tiles */
  uint64_t num_tiles;    /* int32  [1]                 number of valid tiles        */
  uint64_t xsf_planes;   /* uint8  [H/128, R, 4]       token scales of the sorted rows
                                                        (planes; the tiled GEMM1's input) */
  uint64_t mega;         /* MOE_MEGA_STATE_BYTES at offset 0: the single-launch forward's
                                                        work queues and counters; must be zero
                                                        before its first call, left zero by each */
  uint64_t total;        /* == workspace_bytes                                      */
} moe_w4a4_ws_layout;

int moe_w4a4_workspace_layout(const moe_w4a4_cfg* cfg, moe_w4a4_ws_layout* out);

/* Stage bits for moe_w4a4_run_stages. */
enum {
  MOE_STAGE_QUANT = 1,    /* x -> xq, xsf                                  */
  MOE_STAGE_ROUTE = 2,    /* topk_ids -> counts, offsets, sorted_rows, pos;
                             with more than 16 routed rows per expert on
                             average also the tile list, and xsf ->
                             xsf_planes (the token scales in sorted order) */
  MOE_STAGE_GEMM1 = 4,    /* xq, xsf (or xsf_planes), route -> hq, hsf     */
  MOE_STAGE_GEMM2 = 8,    /* hq, route -> y                                */
  MOE_STAGE_COMBINE = 16, /* y, pos, topk_weights -> out                   */
  MOE_STAGE_ALL = 31
};

/* Run the selected stages of a forward on the workspace, reading whatever the
 * skipped stages would have written from the workspace as the caller left it
 * (a test can fill an intermediate and run a single stage).  Arguments as for
 * moe_w4a4_forward; a pointer only some stages read may be NULL when those
 * stages are not selected.  gemm1_acc: NULL, or a device float buffer
 * [max_tokens*k, 2I] into which GEMM1 also writes its raw fp32 accumulators
 * (gate in columns [0, I), up in [I, 2I)), in sorted-row order; with NVFP4
 * after the tensor scales g_x * g_w1[e] are applied. */
int moe_w4a4_run_stages(const moe_w4a4_cfg* cfg, const void* prepared, int32_t num_tokens,
                        const uint16_t* x, const int32_t* topk_ids, const float* topk_weights,
                        uint16_t* out, void* workspace, size_t workspace_bytes,
                        uint32_t stages, float* gemm1_acc, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_W4A4_H */

/*
 * nvfp4_w4a16.h -- C ABI of the NVFP4 W4A16 lm_head library for MI355X (gfx950).
 *
 * Three calls: quantize a bf16 lm_head weight to NVFP4, re-quantize it in
 * place into the same buffers, and compute logits from the quantized weight
 * with bf16 activations.  Two more adopt a pre-quantized NVFP4 checkpoint
 * (ModelOpt or compressed-tensors) for the same GEMM.  Everything runs in
 * hand-written HIP kernels.
 *
 * The method is the one the vLLM API docs describe for
 * vllm.model_executor.layers.quantization.online.lm_head (function
 * _quantize_nvfp4, class _LMHeadNvfp4Method, refresh_quantized_lm_heads).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every pointer is a DEVICE pointer on the current HIP device, except where
 *    stated.  bf16 tensors are passed as raw 16-bit words (bfloat16 bits).
 *  - All matrices are row-major and dense (row pitch = number of columns).
 *  - The caller owns every buffer; the library allocates nothing and keeps no
 *    state between calls, so calls are reentrant and can be captured into a
 *    HIP graph.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Each
 *    call only enqueues work on it: no host<->device synchronisation.
 *  - Arguments are validated on the host before any HIP API call.  A non-zero
 *    status means nothing was enqueued, except NVFP4_ERR_LAUNCH, which reports
 *    a HIP error raised while enqueueing (see nvfp4_last_hip_error()).
 *  - Device faults surface as HIP errors at the caller's next synchronisation.
 *  - Alignment: W, x and y must be 16-byte aligned; packed 16-byte aligned;
 *    scales 4-byte aligned (16-byte for the two checkpoint calls);
 *    global_scale, flags and partition scales 4-byte aligned; bias 2-byte
 *    aligned.
 *  - Outputs may not overlap inputs or each other (NVFP4_ERR_ALIAS).
 *  - Non-finite weights are outside the contract (results unspecified).
 */
#ifndef NVFP4_W4A16_H_
#define NVFP4_W4A16_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = 1,   /* a required pointer is NULL                                   */
  NVFP4_ERR_SHAPE = 2,  /* N < 1, K < 16, K % 16 != 0, M < 0, or a size too large       */
  NVFP4_ERR_ALIGN = 3,  /* a pointer breaks the alignment rules above                   */
  NVFP4_ERR_ALIAS = 4,  /* an output byte range overlaps an input or another output     */
  NVFP4_ERR_LAUNCH = 5, /* HIP reported an error while enqueueing                        */
  NVFP4_ERR_ARG = 6,    /* an enumerated argument (e.g. a scale convention) is out of range */
  NVFP4_ERR_SCRATCH = 7 /* the call needs more scratch than the library's static array holds */
} nvfp4_status;

/* Group size along K: one E4M3 scale per 16 consecutive weights of a row
 * (vLLM modelopt.py, ModelOptNvFp4Config default group size; vLLM API docs,
 * compressed_tensors.schemes, CompressedTensorsW4A16Fp4). */
#define NVFP4_GROUP 16

/*
 * nvfp4_quantize -- online NVFP4 quantization of a bf16 weight.
 * (vLLM API docs, quantization.online.lm_head, _quantize_nvfp4.)
 *
 *   W            in   bf16 [N, K]                the weight (e.g. a vocab shard of lm_head)
 *   N, K         in   N >= 1 rows, K >= 16 columns, K % 16 == 0 (vLLM modelopt.py,
 *                     KNvfp4Static rejects other K)
 *   packed       out  uint8 [N, K/2]            E2M1 codes, two per byte, the even-k code
 *                                               in the low nibble; bit 3 of a code = sign
 *   scales       out  float8_e4m3fn bytes [N, K/16]   block scale of W[n, 16j : 16j+16]
 *   global_scale out  1 float                   max(amax(|W|) / (6 * 448), 1e-12): the
 *                                               dequantization-direction global scale
 *                                               (ModelOpt's amax/2688, per modelopt.py
 *                                               KNvfp4Static.process)
 *
 * Dequantization: w[n,k] ~= E2M1(code[n,k]) * e4m3(scales[n,k/16]) * global_scale.
 * Per block: u = min((max|w| / 6) * (1/global_scale), 448) rounded to E4M3
 * (nearest-even); each weight is multiplied by (1/global_scale)/scale and
 * rounded to the E2M1 grid {0,.5,1,1.5,2,3,4,6} (nearest, ties to the even
 * code, saturating at 6).  A zero block has scale 0 and codes 0; zero never
 * carries a sign.  The global_scale word also serves as the amax accumulator
 * while the call runs, so the outputs are only valid once the stream reaches
 * the end of the call.
 */
nvfp4_status nvfp4_quantize(const void* W, int64_t N, int64_t K,
                            uint8_t* packed, uint8_t* scales, float* global_scale,
                            void* stream);

/*
 * nvfp4_refresh_inplace -- re-derive the quantized copy from an updated weight.
 * (vLLM API docs, quantization.online.lm_head, refresh_quantized_lm_heads: the
 * copy is rewritten in place so that captured graphs keep valid pointers.)
 *
 * Same arguments, computation and result as nvfp4_quantize, into buffers that
 * already hold a quantization of a weight of the same (N, K).  It writes only
 * the bytes of packed, scales and global_scale, allocates nothing and uses no
 * memset nodes, so a HIP graph that captured nvfp4_w4a16_gemm on these
 * pointers reads the new values on its next replay.  A refresh that overlaps
 * a GEMM reading the same buffers on another stream is the caller's race.
 */
nvfp4_status nvfp4_refresh_inplace(const void* W, int64_t N, int64_t K,
                                   uint8_t* packed, uint8_t* scales, float* global_scale,
                                   void* stream);

/*
 * nvfp4_w4a16_gemm -- logits from bf16 activations and the NVFP4 weight.
 * (vLLM API docs, quantization.online.lm_head, _LMHeadNvfp4Method.apply:
 * weight-only NVFP4, activations stay in the model dtype.)
 *
 *   x            in   bf16 [M, K]     activations; M >= 0 (M == 0 enqueues nothing, and
 *                                    x and y may then be NULL)
 *   packed, scales, global_scale in  as produced by nvfp4_quantize for [N, K]
 *   N            in   N >= 1
 *   bias         in   bf16 [N] or NULL
 *   y            out  bf16 [M, N]
 *
 *   y[m, n] = bf16_rne( global_scale * sum_k x[m,k] * E2M1(code[n,k]) * e4m3(scale[n,k/16])
 *                       + bias[n] )
 * with fp32 accumulation; summation order is unspecified but deterministic.
 * The dequantized weight E2M1 * e4m3 is exact (at most 6 significant bits).
 * M <= 64 runs the streaming decode kernels, larger M the MFMA prefill kernel.
 *
 * Products: the prefill kernel and most decode kernels multiply the bf16
 * activations as given, so every product is exact in fp32.  The decode
 * kernels for 3 <= M <= 16 that hold the activation in LDS, whole (K a
 * multiple of 256 and M * (2K + 16) bytes small enough) or one range of K/2,
 * K/4 or K/8 columns (a multiple of 1024) at a time, stage each activation
 * row m in f16 as x * 2^-p_m, with the power of two chosen from the whole
 * row's largest magnitude so that it lands in [2^14, 2^15), and multiply the
 * f16 results by 2^p_m in fp32.  An activation with |x| >= 2^-28 * max_k |x[m,k]| converts
 * exactly (bf16's 8 significant bits fit f16's 11); a smaller one may move by
 * at most max(2^-39 * max_k |x[m,k]|, 2^-151), half the f16 subnormal spacing
 * at that scale.  Each y[m, n] may therefore differ from the exact-product
 * sum by at most that bound times sum_k |w[n,k]| before the fp32 summation
 * and bf16 rounding errors; no other rounding enters.
 */
nvfp4_status nvfp4_w4a16_gemm(const void* x, int64_t M, int64_t K,
                              const uint8_t* packed, const uint8_t* scales,
                              const float* global_scale, int64_t N,
                              const void* bias, void* y, void* stream);

/*
 * Pre-quantized checkpoints.
 * (vLLM modelopt.py, class KNvfp4Static, create_weights and process; vLLM API
 * docs, compressed_tensors.schemes, class CompressedTensorsW4A16Fp4,
 * create_weights and process_weights_after_loading.)
 *
 * Both formats store the packed codes as uint8 [N, K/2] and the block scales
 * as float8_e4m3fn [N, K/16] exactly as nvfp4_quantize writes them, so
 * nvfp4_w4a16_gemm reads them as loaded.  They differ in the per-partition
 * global scale (one float per fused output partition, e.g. 1 for lm_head):
 */
typedef enum {
  /* weight_scale_2 = amax / 2688 (the dequantization direction); the global
   * scale is the largest of them, used as is */
  NVFP4_SCALE2_MODELOPT = 0,
  /* weight_global_scale = 2688 / amax, stored inverted; the global scale is
   * 1 / (the largest of them), one IEEE float32 division */
  NVFP4_SCALE2_COMPRESSED_TENSORS = 1
} nvfp4_scale2_convention;

/* Bits of the flags word nvfp4_import_checkpoint writes. */
#define NVFP4_IMPORT_SCALES_NOT_LOADED 1u   /* a block scale is an e4m3fn NaN (0x7F or 0xFF)      */
#define NVFP4_IMPORT_PARTITIONS_DIFFER 2u   /* the partition scales are not all equal (IEEE ==),   */
                                            /* which costs accuracy: one global scale serves all   */
#define NVFP4_IMPORT_BAD_GLOBAL_SCALE  4u   /* the global scale is not a finite number > 0         */

/*
 * nvfp4_fill_scale_sentinel -- mark a block-scale buffer as not loaded.
 *
 *   scales  out  float8_e4m3fn bytes [N, K/16], 16-byte aligned; every byte is
 *                set to 0x7F (an e4m3fn NaN), the sentinel KNvfp4Static
 *                creates its weight_scale with
 *   N, K    in   the weight's shape (rules of nvfp4_quantize)
 *
 * Call it on a freshly allocated buffer before the checkpoint loader fills
 * it, so that nvfp4_import_checkpoint can tell which scales were never loaded.
 */
nvfp4_status nvfp4_fill_scale_sentinel(uint8_t* scales, int64_t N, int64_t K, void* stream);

/*
 * nvfp4_import_checkpoint -- the GEMM's global scale from a checkpoint, and a
 * check of its block scales.
 *
 *   partition_scales in  float [num_partitions], 4-byte aligned: the stored
 *                        per-partition global scales, in `convention`
 *   num_partitions   in  1 .. 2^20
 *   convention       in  an nvfp4_scale2_convention (else NVFP4_ERR_ARG)
 *   scales           in  float8_e4m3fn bytes [N, K/16] as loaded, 16-byte aligned
 *   N, K             in  the weight's shape (rules of nvfp4_quantize)
 *   global_scale     out 1 float: what nvfp4_w4a16_gemm takes as global_scale
 *                        (a NaN result is written as the quiet NaN 0x7FC00000)
 *   flags            out 1 uint32: NVFP4_IMPORT_* bits
 *
 * The library only reports: a caller that follows KNvfp4Static rejects the
 * tensor when NVFP4_IMPORT_SCALES_NOT_LOADED is set and warns on
 * NVFP4_IMPORT_PARTITIONS_DIFFER.  Both outputs are valid once the stream
 * reaches the end of the call; no output may overlap an input or the other
 * output.  The partition scales are read once, the block scales once
 * (N*K/16 bytes).
 */
nvfp4_status nvfp4_import_checkpoint(const float* partition_scales, int64_t num_partitions, int convention,
                                     const uint8_t* scales, int64_t N, int64_t K, float* global_scale,
                                     uint32_t* flags, void* stream);

/*
 * The FP8 lm_head copy.
 * (vLLM API docs, quantization.online.lm_head, quantized_lm_head_copy: the
 * "fp8" copy uses per-row weight scales and per-token activation scales on
 * an FP8 linear kernel; vLLM modelopt.py, KFp8StaticChannel and the
 * FP8_PER_CHANNEL_PER_TOKEN recipe; vLLM API docs, compressed_tensors.schemes,
 * the W8A8 FP8 apply_weights path.)
 *
 * nvfp4_fp8_quantize_rows -- row-wise E4M3 quantization of a bf16 matrix;
 * quantizes the weight once (one scale per output row) and the activations
 * at every call (one scale per token).
 *
 *   A           in   bf16 [R, K], 16-byte aligned (R >= 1, K >= 16, K % 16 == 0)
 *   q           out  float8_e4m3fn bytes [R, K], 16-byte aligned
 *   row_scales  out  float [R]
 *
 *   s[r] = max(max_k |A[r,k]| / 448, 1e-12)     (float32, one IEEE division)
 *   q[r,k] = e4m3_rne(clamp(A[r,k] * (1 / s[r]), -448, 448)), sign kept
 *
 * The pages do not show the quantizer's arithmetic; this is the plainest
 * reading (the clamp mirrors the NVFP4 global scale's).
 */
nvfp4_status nvfp4_fp8_quantize_rows(const void* A, int64_t R, int64_t K, uint8_t* q, float* row_scales,
                                     void* stream);

/*
 * nvfp4_fp8_gemm -- logits from the FP8 copy.
 *
 *   xq, x_scales in  float8_e4m3fn [M, K] and float [M] from nvfp4_fp8_quantize_rows (M >= 0;
 *                    M == 0 enqueues nothing, and xq, x_scales and y may then be NULL)
 *   wq, w_scales in  float8_e4m3fn [N, K] and float [N], likewise
 *   bias         in  bf16 [N] or NULL
 *   y            out bf16 [M, N], 16-byte aligned
 *
 *   y[m, n] = bf16_rne(x_scales[m] * w_scales[n] * sum_k e4m3(xq[m,k]) * e4m3(wq[n,k]) + bias[n])
 * with float32 accumulation of exact float32 products.
 */
nvfp4_status nvfp4_fp8_gemm(const uint8_t* xq, const float* x_scales, int64_t M, int64_t K, const uint8_t* wq,
                            const float* w_scales, int64_t N, const void* bias, void* y, void* stream);

/*
 * NVFP4 W4A4: activations quantized to NVFP4 at run time with a static global
 * input scale, and the GEMM of the two NVFP4 operands.
 * (vLLM modelopt.py, KNvfp4Dynamic, maybe_fuse_global_scales and the NVFP4
 * recipe: static FP4 weight, dynamic FP4 activation, alpha =
 * input_global_scale * weight_global_scale.)
 *
 * nvfp4_quantize_activations -- x bf16 [M, K] (16-byte aligned) -> packed
 * uint8 [M, K/2] and float8_e4m3fn scales [M, K/16], with the rules of
 * nvfp4_quantize but the given input_global_scale (1 float on the device, the
 * dequantization direction, e.g. the max of a checkpoint's input_scale; it
 * must be a finite number > 0) in place of amax/2688.  Nothing is written to
 * input_global_scale.
 */
nvfp4_status nvfp4_quantize_activations(const void* x, int64_t M, int64_t K, const float* input_global_scale,
                                        uint8_t* packed, uint8_t* scales, void* stream);

/*
 * nvfp4_w4a4_workspace_bytes -- size of nvfp4_w4a4_gemm's workspace: 2*M*K + 16
 * (host helper, no device work; 0 for negative sizes).
 */
int64_t nvfp4_w4a4_workspace_bytes(int64_t M, int64_t K);

/*
 * nvfp4_w4a4_gemm -- logits from NVFP4 activations and the NVFP4 weight.
 *
 *   x_packed, x_scales   in  from nvfp4_quantize_activations, [M, K/2] / [M, K/16]
 *   input_global_scale   in  the global scale they were quantized with (1 float)
 *   packed, scales, global_scale, N, bias   in  as for nvfp4_w4a16_gemm
 *   workspace            tmp device buffer of nvfp4_w4a4_workspace_bytes(M, K) bytes,
 *                            16-byte aligned, overlapping nothing else; it holds the
 *                            activations' exact bf16 values code * block scale, then
 *                            alpha, and may be reused once the stream is past the call
 *   y                    out bf16 [M, N]
 *
 *   y[m, n] = bf16_rne( alpha * sum_k (E2M1(cx) * e4m3(sx)) * (E2M1(cw) * e4m3(sw)) + bias[n] ),
 *   alpha = fl32(input_global_scale * global_scale), float32 accumulation of exact products.
 * M == 0 enqueues nothing (the activation pointers, workspace and y may then be NULL).
 */
nvfp4_status nvfp4_w4a4_gemm(const uint8_t* x_packed, const uint8_t* x_scales, const float* input_global_scale,
                             int64_t M, int64_t K, const uint8_t* packed, const uint8_t* scales,
                             const float* global_scale, int64_t N, const void* bias, void* workspace, void* y,
                             void* stream);

/*
 * nvfp4_w4a4_gemm_noalloc -- nvfp4_w4a4_gemm without a workspace argument and
 * without any allocation, for callers that cannot allocate device memory
 * (code being captured into a HIP graph, tight serving loops, harnesses that
 * forbid hipMalloc).
 *
 * Same arguments (minus `workspace`), computation, result and errors as
 * nvfp4_w4a4_gemm.  The workspace lives in a static device array of
 * NVFP4_W4A4_SCRATCH_BYTES bytes that the library holds on each GPU it runs
 * on until the process ends; calls whose workspace
 * (nvfp4_w4a4_workspace_bytes(M, K) = 2*M*K + 16 bytes, i.e. M*K <= 2097144)
 * would not fit return NVFP4_ERR_SCRATCH and enqueue nothing.  All calls on
 * one GPU share that array: calls that may overlap on one GPU (other streams,
 * other host threads) race and must be serialised by the caller.  The first
 * call on a device looks up the array's address on that device (no
 * allocation); every call writes the whole region it reads before reading it.
 */
#define NVFP4_W4A4_SCRATCH_BYTES (4 << 20)
nvfp4_status nvfp4_w4a4_gemm_noalloc(const uint8_t* x_packed, const uint8_t* x_scales,
                                     const float* input_global_scale, int64_t M, int64_t K,
                                     const uint8_t* packed, const uint8_t* scales, const float* global_scale,
                                     int64_t N, const void* bias, void* y, void* stream);

/*
 * Mixture of experts, W4A16 NVFP4 (vLLM modelopt.py, ModelOptNvFp4FusedMoE with
 * use_a16: per-expert NVFP4 weights w13 [E, 2I, H/2] / scales [E, 2I, H/16] and
 * w2 [E, H, I/2] / scales [E, H, I/16], one float32 global scale per expert and
 * matrix -- for w13 the w1 column of w13_weight_scale_2 -- and routing by
 * topk_ids / topk_weights as apply() receives them).
 *
 * Pair p = t * topk + j is token t's j-th routed expert topk_ids[t * topk + j].
 * A pair whose id lies outside [0, E) is outside the contract: it is counted
 * into *invalid_pairs (when non-NULL) and its GEMM output row is zero.
 *
 * nvfp4_moe_gemm_workspace_bytes -- workspace of nvfp4_moe_w4a16_gemm: the
 * routing table, 4 * (round_up(E + 2, 4) + round_up(P, 4)) bytes (host helper;
 * 0 for P < 0 or E < 1).
 */
int64_t nvfp4_moe_gemm_workspace_bytes(int64_t P, int64_t E);

/*
 * nvfp4_moe_w4a16_gemm -- the grouped expert GEMM:
 *   y[p, n] = bf16_rne( gs[e] * sum_k x[p / row_div, k] * E2M1(code_e[n, k]) * e4m3(scale_e[n, k/16]) ),
 *   e = topk_ids[p], float32 accumulation of exact products.
 *
 *   x              in  bf16 [x_rows, K]; row_div = topk reads token rows (the first
 *                      GEMM), row_div = 1 reads one row per pair (the second);
 *                      x_rows >= ceil(P / row_div)
 *   topk_ids       in  int32 [P]
 *   packed, scales in  [E, N, K/2] uint8 / [E, N, K/16] e4m3fn, the per-expert layout
 *                      of the pages (packed 16-byte aligned)
 *   global_scales  in  float32 [E]
 *   workspace      tmp nvfp4_moe_gemm_workspace_bytes(P, E) bytes, 16-byte aligned
 *   y              out bf16 [P, N]
 *   invalid_pairs  out optional uint32 (NULL = not reported)
 * An expert with no pair reads none of its weights.  P == 0 enqueues nothing.
 */
nvfp4_status nvfp4_moe_w4a16_gemm(const void* x, int64_t x_rows, int64_t K, const int32_t* topk_ids, int64_t P,
                                  int64_t row_div, const uint8_t* packed, const uint8_t* scales,
                                  const float* global_scales, int64_t E, int64_t N, void* workspace, void* y,
                                  uint32_t* invalid_pairs, void* stream);

/*
 * nvfp4_moe_silu_and_mul -- a[p, i] = bf16_rne( silu(h[p, i]) * h[p, I + i] ),
 * silu(g) = g / (1 + exp(-g)) in float32: the act-and-mul layout [w1; w3] of
 * w13.  h bf16 [P, 2I], a bf16 [P, I], I % 8 == 0, both 16-byte aligned.
 */
nvfp4_status nvfp4_moe_silu_and_mul(const void* h, int64_t P, int64_t I, void* a, void* stream);

/*
 * nvfp4_moe_combine -- out[t, n] = bf16_rne( sum_j topk_weights[t, j] * o[t * topk + j, n] ),
 * float32 in slot order j = 0, 1, ...  o bf16 [T * topk, H], topk_weights float32
 * [T, topk], out bf16 [T, H], H % 8 == 0, o and out 16-byte aligned.
 */
nvfp4_status nvfp4_moe_combine(const void* o, const float* topk_weights, int64_t T, int64_t topk, int64_t H,
                               void* out, void* stream);

/*
 * nvfp4_moe_workspace_bytes -- workspace of nvfp4_moe_w4a16_forward: the routing
 * table, then h [P, 2I], a [P, I] and o [P, H] in bf16, each rounded up to 256 bytes
 * (host helper; 0 for invalid sizes).
 *
 * nvfp4_moe_w4a16_forward -- the whole W4A16 expert layer on bf16 x [T, H]:
 * routing, h = grouped GEMM with w13, a = silu_and_mul(h), o = grouped GEMM
 * with w2, out = combine(o, topk_weights); each stage as the calls above, h, a
 * and o rounded to bf16.  out bf16 [T, H].  T == 0 enqueues nothing.
 */
int64_t nvfp4_moe_workspace_bytes(int64_t T, int64_t topk, int64_t E, int64_t H, int64_t I);
nvfp4_status nvfp4_moe_w4a16_forward(const void* x, int64_t T, int64_t H, const int32_t* topk_ids,
                                     const float* topk_weights, int64_t topk, const uint8_t* w13_packed,
                                     const uint8_t* w13_scales, const float* w13_global_scales,
                                     const uint8_t* w2_packed, const uint8_t* w2_scales,
                                     const float* w2_global_scales, int64_t E, int64_t I, void* workspace,
                                     void* out, uint32_t* invalid_pairs, void* stream);

/* Host-side helpers (no device work). */
const char* nvfp4_status_string(int status);   /* static string for a status code        */
const char* nvfp4_last_hip_error(void);        /* last HIP error text of this thread, or "" */
int nvfp4_abi_version(void);                   /* bumps when a signature above changes   */

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_W4A16_H_ */

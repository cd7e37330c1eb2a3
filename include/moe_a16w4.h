/*
 * moe_a16w4 -- fused mixture-of-experts layer with bf16 activations and
 * 4-bit expert weights (A16W4) for AMD Instinct MI355X (gfx950).
 *
 * The layer, per token t with router logits l[t, :] and activation x[t, :]:
 *   1. route: the topk experts with the largest logits, weighted by their
 *      softmax probabilities renormalised over the chosen k;
 *   2. align/sort: the (token, slot) pairs grouped by expert;
 *   3. per pair (t, j) with expert e: gate/up = W13[e] . x[t]
 *      (rows [0, I) gate, rows [I, 2I) up), h = silu(gate) * up,
 *      y = W2[e] . h;
 *   4. out[t] = sum_j weight[t, j] * y(t, j).
 *
 * Sources: the vLLM API page of the mxfp4 quantization module, class
 * Mxfp4MoEMethod (create_weights: the weight and scale tensor shapes;
 * apply / apply_monolithic: forward with precomputed or in-kernel routing;
 * _setup_kernel_k3_situ_gfx942: the MXFP4 -> int4 requantization), and the
 * vLLM pull request "[ROCm][Kimi-K3] Add opt-in gfx942 MXFP4-to-int4
 * conversion" (Summary, Changes: the int4_per_group_32 format, conversion
 * eight experts at a time, fail-closed activation check).
 *
 * Conventions for every call:
 *   - Pointers are caller-owned device memory unless stated otherwise; the
 *     library never allocates device memory.
 *   - `stream` is a hipStream_t (NULL = the default stream). Work is
 *     enqueued asynchronously; no call synchronises the host, so a sequence
 *     of calls may be captured into a HIP graph.
 *   - Arguments are validated before anything is enqueued; on any error
 *     nothing is launched and moe_last_error() describes the problem.
 *   - bf16 values travel as uint16_t bit patterns.
 *   - Data held in device memory is not validated (it cannot be read without
 *     a host synchronisation); out-of-contract device data gives unspecified
 *     results but never out-of-bounds accesses, except where noted.
 */
#ifndef MOE_A16W4_H
#define MOE_A16W4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1, /* a size, pointer or range is invalid */
    MOE_ERR_UNSUPPORTED = 2, /* valid request outside what is implemented */
    MOE_ERR_HIP = 3          /* the HIP runtime reported an error at launch */
} moe_status;

/* Weight formats. MXFP4 is the checkpoint format (create_weights on the
 * mxfp4 API page): e2m1 nibbles packed two per byte along K (even k in the
 * low nibble) with one e8m0 byte per 32 elements along K. INT4G32 is the
 * opt-in int4_per_group_32 format of the MXFP4-to-int4 pull request:
 * two's-complement int4 nibbles with the same packing and one bf16 scale per
 * 32 elements along K. */
typedef enum { MOE_W_MXFP4 = 0, MOE_W_INT4G32 = 1 } moe_wfmt;

/* Gated activations. Only SwiGLU, silu(gate) * up, is implemented; any other
 * value fails closed with MOE_ERR_UNSUPPORTED rather than silently computing
 * SwiGLU (the pull request's Changes: fail closed unless the kernel honours
 * the requested activation). */
typedef enum { MOE_ACT_SWIGLU = 0 } moe_act;

/* Message for the last non-OK status returned on the calling thread
 * (a static, thread-local string; never NULL). */
const char* moe_last_error(void);

/* Softmax top-k routing (the routing inside apply_monolithic on the mxfp4
 * API page; the pages do not print the rule, this is plain softmax top-k).
 *   logits        fp32 [T, E], row-major.
 *   topk_ids      out int32 [T, topk]: expert indices in descending logit
 *                 order; equal logits rank the lower index first.
 *   topk_weights  out fp32 [T, topk]: softmax probabilities of the chosen
 *                 experts, renormalised to sum 1 when renormalize != 0.
 * Limits: T >= 0 (T == 0 is a no-op), 1 <= E <= 1024, 1 <= topk <= min(E, 64).
 * NaN logits give unspecified (in-range) ids. */
moe_status moe_route_topk(const float* logits, int T, int E, int topk, int renormalize,
                          int32_t* topk_ids, float* topk_weights, void* stream);

/* Rows of sorted_ids needed for T*topk pairs over E experts when every
 * expert segment is padded to a multiple of block_m:
 * roundup(P + min(E, P) * (block_m - 1), block_m), P = T*topk.
 * Returns -1 for invalid arguments. */
int64_t moe_align_sort_capacity(int T, int topk, int E, int block_m);

/* Block size the forward works best with for this token count
 * (16 up to 48 tokens, else 32). */
int moe_default_block_m(int T, int topk, int E);

/* Group the P = T*topk (token, slot) pairs by expert for the grouped GEMMs
 * of the two-stage MoE. Pair p = t*topk + j.
 *   topk_ids        int32 [T, topk]; ids within a token must be distinct
 *                   and in [0, E) -- pairs with an id outside [0, E) are
 *                   dropped (not listed).
 *   block_m         16, 32, 64, 128 or 256.
 *   sorted_ids      out int32 [cap] (cap = moe_align_sort_capacity): for
 *                   each expert in ascending order, its pairs in ascending p,
 *                   padded to a multiple of block_m with the sentinel P;
 *                   rows past the last segment are P as well.
 *   block_expert    out int32 [cap / block_m]: expert of each block, -1 for
 *                   blocks past the last segment.
 *   expert_offsets  out int32 [E + 1]: start row of each expert's padded
 *                   segment; expert_offsets[E] == *num_post_pad.
 *   num_post_pad    out int32 [1]: rows in use.
 * The result is deterministic (no dependence on atomic ordering).
 * Limits: E <= 1024, T*topk < 2^31 - cap. */
moe_status moe_align_sort(const int32_t* topk_ids, int T, int topk, int E, int block_m,
                          int32_t* sorted_ids, int32_t* block_expert, int32_t* expert_offsets,
                          int32_t* num_post_pad, void* stream);

/* moe_route_topk followed by moe_align_sort for the same arguments, with
 * identical outputs; up to 64 tokens run as one launch that keeps the ids on
 * chip between the two steps (the in-kernel routing of apply_monolithic on
 * the mxfp4 API page). Limits and errors are those of the two calls; all
 * output buffers are required (topk_ids/topk_weights [T, topk] included). */
moe_status moe_route_align(const float* logits, int T, int E, int topk, int renormalize,
                           int block_m, int32_t* topk_ids, float* topk_weights,
                           int32_t* sorted_ids, int32_t* block_expert, int32_t* expert_offsets,
                           int32_t* num_post_pad, void* stream);

/* Bytes of device workspace moe_a16w4_forward needs (256-byte aligned
 * start required). Returns -1 for invalid arguments. */
int64_t moe_a16w4_workspace_size(int T, int H, int I, int E, int topk, int block_m);

/* Fused MoE forward with precomputed routing (apply() on the mxfp4 API
 * page): grouped gate_up GEMM with the weights dequantized in registers,
 * SwiGLU, grouped down GEMM, top-k weighted combine.
 *   x             bf16 [T, H].
 *   w13           uint8 [E, 2I, H/2] packed 4-bit weights (gate rows [0, I),
 *                 up rows [I, 2I)); w13_scale [E, 2I, H/32]: uint8 e8m0 for
 *                 MXFP4, uint16 bf16 for INT4G32.
 *   w2            uint8 [E, H, I/2]; w2_scale [E, H, I/32] (same typing).
 *   topk_ids, topk_weights   int32 / fp32 [T, topk] (router weights are
 *                 applied at the combine).
 *   sorted_ids, block_expert, num_post_pad   moe_align_sort's output for
 *                 the same topk_ids and block_m.
 *   out           bf16 [T, H].
 *   workspace     device memory of moe_a16w4_workspace_size bytes.
 * Requirements: H % 32 == 0, I % 32 == 0, H >= 32, I >= 32, E >= 1,
 *   1 <= topk <= E, block_m in {16, 32, 64} (128 and 256 are valid sort
 *   sizes but give MOE_ERR_UNSUPPORTED here); all pointers 16-byte aligned
 *   (workspace 256-byte aligned).
 * Size limits (MOE_ERR_UNSUPPORTED, nothing launched): x [T, H] and the
 *   workspace's bf16 h [cap, I] (cap = moe_align_sort_capacity) must each
 *   stay below 2^31 - 2^16 bytes, and with block_m == 64 cap / 64 <= 65535.
 *   At H = 3584, I = 3072, E = 112, topk = 15, block_m = 32 that allows up
 *   to about 23,000 tokens per call; larger batches are split by the caller.
 * MXFP4 e8m0 bytes must be in [0, 254]; weights whose value overflows bf16
 * give unspecified results. */
moe_status moe_a16w4_forward(const uint16_t* x, const uint8_t* w13, const void* w13_scale,
                             const uint8_t* w2, const void* w2_scale, moe_wfmt fmt, moe_act act,
                             const int32_t* topk_ids, const float* topk_weights,
                             const int32_t* sorted_ids, const int32_t* block_expert,
                             const int32_t* num_post_pad, int T, int H, int I, int E, int topk,
                             int block_m, uint16_t* out, void* workspace, size_t workspace_bytes,
                             void* stream);

/* The forward split into its launches, for callers that schedule or time
 * them separately (the modular-kernel stages of the pages). Bits of
 * `stages`: MOE_STAGE_GATE_UP (grouped gate_up GEMM + SwiGLU into the
 * workspace), MOE_STAGE_DOWN (grouped down GEMM from the workspace into the
 * workspace), MOE_STAGE_COMBINE (weighted combine from the workspace into
 * out). Enabled stages run in that order on `stream`; a stage reads what
 * the previous stage wrote into the same workspace for the same arguments.
 * moe_a16w4_forward == moe_a16w4_forward_stages with MOE_STAGE_ALL. Same
 * arguments, requirements and errors as moe_a16w4_forward; stages == 0 or
 * unknown bits give MOE_ERR_INVALID_ARG. */
#define MOE_STAGE_GATE_UP 1u
#define MOE_STAGE_DOWN 2u
#define MOE_STAGE_COMBINE 4u
#define MOE_STAGE_ALL 7u
moe_status moe_a16w4_forward_stages(const uint16_t* x, const uint8_t* w13, const void* w13_scale,
                                    const uint8_t* w2, const void* w2_scale, moe_wfmt fmt,
                                    moe_act act, const int32_t* topk_ids,
                                    const float* topk_weights, const int32_t* sorted_ids,
                                    const int32_t* block_expert, const int32_t* num_post_pad, int T,
                                    int H, int I, int E, int topk, int block_m, uint16_t* out,
                                    void* workspace, size_t workspace_bytes, unsigned stages,
                                    void* stream);

/* moe_a16w4_forward_stages with the optional expert biases and GEMM1 clamp
 * of the mxfp4 API page (create_weights under has_bias makes w13_bias and
 * w2_bias in bf16; get_fused_moe_quant_config passes them to the kernel with
 * the layer's swiglu_limit as the GEMM1 clamp limit):
 *   gate/up = W13[e] . x + w13_bias[e]   (w13_bias bf16 [E, 2I]: gate biases
 *                                          in [0, I), up biases in [I, 2I))
 *   gate, up clamped to [-swiglu_limit, swiglu_limit] when swiglu_limit > 0
 *   h = silu(gate) * up;  y = W2[e] . h + w2_bias[e]  (w2_bias bf16 [E, H])
 *   out[t] = sum_j weight[t, j] * y(t, j).
 * The pages name these terms but print no formula; this placement (each
 * bias on its GEMM's output, the clamp on both GEMM1 outputs before the
 * activation) is the reading taken. Either bias may be NULL (no term);
 * swiglu_limit == 0 means no clamp, a negative or NaN limit is
 * MOE_ERR_INVALID_ARG. Bias pointers 16-byte aligned. Everything else as
 * moe_a16w4_forward_stages; the w2 bias is applied by the combine stage. */
moe_status moe_a16w4_forward_ex(const uint16_t* x, const uint8_t* w13, const void* w13_scale,
                                const uint16_t* w13_bias, const uint8_t* w2, const void* w2_scale,
                                const uint16_t* w2_bias, moe_wfmt fmt, moe_act act,
                                float swiglu_limit, const int32_t* topk_ids,
                                const float* topk_weights, const int32_t* sorted_ids,
                                const int32_t* block_expert, const int32_t* num_post_pad, int T,
                                int H, int I, int E, int topk, int block_m, uint16_t* out,
                                void* workspace, size_t workspace_bytes, unsigned stages,
                                void* stream);

/* The whole layer from router logits (apply_monolithic on the mxfp4 API
 * page: routing inside the kernels): moe_route_align for
 * (router_logits, renormalize, block_m) into topk_ids, topk_weights,
 * sorted_ids, block_expert, expert_offsets and num_post_pad (all outputs,
 * sized as for moe_route_align), then moe_a16w4_forward_ex. Results equal
 * those two calls (routing and align/sort outputs bit for bit, out bit for
 * bit as well), with fewer launches where the shape allows: one token with
 * MXFP4 weights, E <= 128, H a multiple of 256 and I of 128 (both up to
 * 4096) routes inside the gate_up kernel (no separate routing launch).
 *   router_logits  fp32 [T, E] (16-byte aligned).
 *   stages         MOE_STAGE_ALL, MOE_STAGE_GATE_UP (routing, align/sort and
 *                  gate_up) or MOE_STAGE_DOWN | MOE_STAGE_COMBINE (the rest);
 *                  other masks give MOE_ERR_INVALID_ARG.
 * Requirements and limits: those of moe_route_align and moe_a16w4_forward_ex;
 * the workspace is moe_a16w4_workspace_size bytes. */
moe_status moe_a16w4_forward_monolithic(const uint16_t* x, const float* router_logits,
                                        const uint8_t* w13, const void* w13_scale,
                                        const uint16_t* w13_bias, const uint8_t* w2,
                                        const void* w2_scale, const uint16_t* w2_bias,
                                        moe_wfmt fmt, moe_act act, float swiglu_limit,
                                        int renormalize, int T, int H, int I, int E, int topk,
                                        int block_m, int32_t* topk_ids, float* topk_weights,
                                        int32_t* sorted_ids, int32_t* block_expert,
                                        int32_t* expert_offsets, int32_t* num_post_pad,
                                        uint16_t* out, void* workspace, size_t workspace_bytes,
                                        unsigned stages, void* stream);

/* moe_a16w4_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc). The workspace is the library's
 * own scratch array of MOE_NOALLOC_SCRATCH_BYTES on each GPU, reserved
 * when the library's code is loaded on that GPU and held until the process
 * ends; its device address is looked up on the first call on each device.
 * The call allocates nothing (no hipMalloc/hipFree, no allocating library
 * routine); the caller passes inputs and `out` as for moe_a16w4_forward.
 *   - Same arguments, requirements and results as moe_a16w4_forward minus
 *     workspace/workspace_bytes.
 *   - A batch whose moe_a16w4_workspace_size exceeds the scratch returns
 *     MOE_ERR_UNSUPPORTED before anything is enqueued (64 MiB holds the
 *     workspace of up to about 128 tokens at H = 3584, I = 3072, E = 112,
 *     topk = 15).
 *   - Every call on one GPU shares that GPU's scratch and leaves its
 *     contents behind; nothing in it needs to start at zero (each call
 *     writes what it reads). Calls that overlap in time on one GPU (on
 *     different streams, or from different threads) race on it and give
 *     wrong results: order them on one stream. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status moe_a16w4_forward_noalloc(const uint16_t* x, const uint8_t* w13, const void* w13_scale,
                                     const uint8_t* w2, const void* w2_scale, moe_wfmt fmt,
                                     moe_act act, const int32_t* topk_ids,
                                     const float* topk_weights, const int32_t* sorted_ids,
                                     const int32_t* block_expert, const int32_t* num_post_pad,
                                     int T, int H, int I, int E, int topk, int block_m,
                                     uint16_t* out, void* stream);

/* MXFP4 -> int4 per-group-32 requantization of experts [expert_lo,
 * expert_hi) of a [E, N, K] weight (convert() in
 * Mxfp4MoEMethod._setup_kernel_k3_situ_gfx942; the pull request converts
 * eight experts per call into preallocated outputs). Per 32-group along K:
 * v = bf16(e2m1 * 2^(e8m0 - 127)); scale = bf16(amax(|v|) / 7) computed in
 * fp32; code = clamp(round_half_even(v / scale), -8, 7) with an IEEE fp32
 * divide (an all-zero group gives scale 0 and codes 0); codes packed two per
 * byte, even k in the low nibble.
 *   w, scale_e8m0   uint8 [E, N, K/2] and [E, N, K/32] (MXFP4).
 *   w_int4          out uint8 [E, N, K/2]; scale_bf16 out uint16 [E, N, K/32].
 *                   Only experts in [expert_lo, expert_hi) are written; the
 *                   library uses no scratch memory beyond these outputs.
 * Requirements: K % 32 == 0, N >= 1, 0 <= expert_lo <= expert_hi <= E;
 * pointers 16-byte aligned. Lossy by construction.
 * Domain: e8m0 bytes 0..252. Bytes 253..255 (decoded values that overflow
 * bf16, or a NaN scale) give unspecified codes and scales, computed without
 * faulting. */
moe_status mxfp4_to_int4g32_requant(const uint8_t* w, const uint8_t* scale_e8m0, int E, int N,
                                    int K, int expert_lo, int expert_hi, uint8_t* w_int4,
                                    uint16_t* scale_bf16, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_A16W4_H */

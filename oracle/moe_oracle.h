/*
 * CPU oracle for the A16W4 mixture-of-experts layer.
 *
 * TEST INFRASTRUCTURE ONLY. This library is the slow, plain reference that
 * the GPU path is checked against. Only the test suite, the package smoke
 * check and the benchmark's CPU-baseline leg may load it; the product path
 * never calls it and shares no code, header or table with it.
 *
 * Sources (the pages):
 *   [P1] vLLM pull request "[ROCm][Kimi-K3] Add opt-in gfx942 MXFP4-to-int4
 *        conversion" -- sections Summary, Changes, Validation and the
 *        squashed commit messages.
 *   [P2] vLLM API page for the mxfp4 quantization module, class
 *        Mxfp4MoEMethod -- methods create_weights, apply, apply_monolithic,
 *        get_fused_moe_quant_config and the per-chunk convert() inside
 *        _setup_kernel_k3_situ_gfx942.
 *
 * Arithmetic: float64 wherever the pages leave the precision open. The
 * requantization takes its integer decisions in float32 (scale = bf16 of the
 * float32 quotient amax/7, codes = round-half-even of the float32 quotient),
 * the precision of the kernel it is compared with.
 *
 * Parity status per function is listed in the .c file header.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weight storage formats. */
#define ORACLE_FMT_MXFP4   0  /* e2m1 nibbles + one e8m0 byte per 32 along K */
#define ORACLE_FMT_INT4G32 1  /* signed int4 nibbles + one bf16 scale per 32 along K */

double oracle_e2m1_value(int code);          /* 4-bit e2m1 code -> value */
double oracle_e8m0_value(int byte);          /* e8m0 byte -> 2^(byte-127); 255 -> NaN */
int    oracle_nibble(const uint8_t* row, int k); /* k-th 4-bit field of a packed row */
double oracle_bf16_value(uint16_t bits);     /* bf16 bit pattern -> value */
uint16_t oracle_f32_to_bf16_rne(float v);    /* float32 -> bf16, round half to even */

/* Dequantize rows [0, rows) of a [rows, K] weight (packed [rows, K/2] bytes,
 * scales [rows, K/32]) into float64 out[rows*K]. */
void oracle_dequant(const uint8_t* w, const void* scale, int fmt,
                    int rows, int K, double* out);

/* Softmax top-k routing of fp32 logits [T, E]. ids[T, topk] in descending
 * logit order (ties: lower expert index first); weights[T, topk] are the
 * softmax probabilities of the chosen experts, renormalised over the chosen
 * k when renormalize != 0. */
void oracle_route_topk(const float* logits, int T, int E, int topk, int renormalize,
                       int32_t* ids, float* weights);

/* Capacity of the sorted pair list for block size bm. */
int64_t oracle_align_capacity(int T, int topk, int E, int bm);

/* Stable grouping of the P = T*topk (token, slot) pairs by expert; every
 * expert segment padded to a multiple of bm with the sentinel P.
 * sorted_ids[cap], block_expert[cap/bm] (-1 past the end), expert_offsets[E+1]
 * (padded segment starts), num_post_pad[1]. */
void oracle_align_sort(const int32_t* ids, int T, int topk, int E, int bm,
                       int32_t* sorted_ids, int32_t* block_expert,
                       int32_t* expert_offsets, int32_t* num_post_pad);

/* Fused MoE forward for the listed tokens (tokens[n_tokens], or all tokens
 * 0..T-1 when tokens == NULL): out[n_tokens, H] in float64.
 * x: bf16 bits [T, H]; w13: [E, 2I, H/2] with scales [E, 2I, H/32];
 * w2: [E, H, I/2] with scales [E, H, I/32]; ids / weights: [T, topk]. */
void oracle_moe_forward(const uint16_t* x, const uint8_t* w13, const void* w13_scale,
                        const uint8_t* w2, const void* w2_scale, int fmt,
                        const int32_t* ids, const float* weights,
                        int T, int H, int I, int E, int topk,
                        const int32_t* tokens, int n_tokens, double* out);

/* The same with the optional expert biases and GEMM1 clamp:
 * w13_bias bf16 [E, 2I] (gate biases, then up biases) and w2_bias bf16
 * [E, H], each NULL for none; swiglu_limit > 0 clamps gate and up (after
 * their bias) to [-limit, limit] before SwiGLU, <= 0 leaves them. */
void oracle_moe_forward_ex(const uint16_t* x, const uint8_t* w13, const void* w13_scale,
                           const uint16_t* w13_bias, const uint8_t* w2, const void* w2_scale,
                           const uint16_t* w2_bias, double swiglu_limit, int fmt,
                           const int32_t* ids, const float* weights,
                           int T, int H, int I, int E, int topk,
                           const int32_t* tokens, int n_tokens, double* out);

/* MXFP4 -> int4 per-group-32 requantisation of experts [lo, hi) of a
 * [E, N, K] weight. Outputs are full-size [E, N, K/2] codes and
 * [E, N, K/32] bf16 scales; only the experts in [lo, hi) are written. */
void oracle_requant_int4g32(const uint8_t* w, const uint8_t* scale_e8m0,
                            int E, int N, int K, int lo, int hi,
                            uint8_t* w_int4, uint16_t* scale_bf16);

/* Number of OpenMP threads the forward uses (1 when built without OpenMP). */
int oracle_num_threads(void);
void oracle_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif

/*
 * CPU oracle for the A16W4 mixture-of-experts layer -- TEST INFRASTRUCTURE.
 *
 * Plain, slow and written to be checked by eye against the pages. Only the
 * test suite, the package smoke check and the benchmark's CPU-baseline leg
 * load this library; the GPU product path never calls it and shares no code
 * with it.
 *
 * Pages cited below:
 *   [P1] vLLM pull request "[ROCm][Kimi-K3] Add opt-in gfx942 MXFP4-to-int4
 *        conversion" (sections Summary, Changes, Validation; commit messages).
 *   [P2] vLLM API page of the mxfp4 quantization module, class Mxfp4MoEMethod
 *        (create_weights, apply, apply_monolithic, get_fused_moe_quant_config,
 *        and convert() inside _setup_kernel_k3_situ_gfx942).
 *
 * Pins (what each function is checked against, besides itself):
 *   oracle_e2m1_value     closed-form e2m1 minifloat decode, all 16 codes
 *   oracle_e8m0_value     torch's float8_e8m0fnu cast and ldexp, all 256 bytes
 *   oracle_nibble         pack/unpack round trip of all 256 bytes
 *   oracle_f32_to_bf16_rne torch's float32 -> bfloat16 cast on edge values
 *   oracle_dequant        closed-form decode + torch e8m0 cast, random rows
 *   oracle_route_topk     brute force by full stable sort; scipy softmax at
 *                         topk == E; topk == 1 gives weight exactly 1
 *   oracle_align_sort     Python sorted() brute force and segment invariants
 *   oracle_moe_forward    numpy float64 dense SwiGLU MLP with torch's bf16
 *                         cast of the SwiGLU output (E = 1, topk = 1);
 *                         per-token dense reconstruction on tiny shapes;
 *                         routing independence with identical experts
 *   oracle_requant_int4g32 hand-derived closed-form code table (the e8m0
 *                         factor cancels); reconstruction error <= s/2
 *   SiTUv2 and other activations: not implemented (formula not on the pages).
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- decode -- */

/* e2m1 (OCP MX FP4): 1 sign bit, 2 exponent bits, 1 mantissa bit. The pages
 * decode packed fp4 through a 16-entry float table (mxfp4_to_f32 in [P2]
 * convert(); [P1] commit message on the 8x unpack). The table below holds the
 * sixteen values of that format; code 8 is negative zero. */
static const double kE2M1[16] = {
    0.0,  0.5,  1.0,  1.5,  2.0,  3.0,  4.0,  6.0,
    -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0,
};

double oracle_e2m1_value(int code) { return kE2M1[code & 0xF]; }

/* e8m0 block scale: a biased power of two, 2^(byte-127); 255 encodes NaN
 * ([P2] e8m0_to_f32 in convert(); scale dtype float8_e8m0fnu). */
double oracle_e8m0_value(int byte) {
    if (byte == 255) return NAN;
    return ldexp(1.0, byte - 127);
}

/* Two fields per byte along K; the even k sits in the low nibble (reading of
 * the packed float4_e2m1fn_x2 view in [P2] convert()). */
int oracle_nibble(const uint8_t* row, int k) {
    return (row[k >> 1] >> (4 * (k & 1))) & 0xF;
}

double oracle_bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

uint16_t oracle_f32_to_bf16_rne(float v) {
    uint32_t u;
    memcpy(&u, &v, sizeof u);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u); /* quiet NaN, sign kept */
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb; /* round half to even on the dropped 16 bits */
    return (uint16_t)(u >> 16);
}

/* Row `row` of a [rows, K] weight in either format, into out[K].
 * MXFP4: e2m1(nibble) * 2^(e8m0 - 127), one scale per 32 along K
 *        ([P2] create_weights: mxfp4_block = 32; convert(): the f32 weight
 *        viewed as [.., K/32, 32] times the scale viewed as [.., K/32, 1]).
 * INT4G32: two's-complement nibble times its group's bf16 scale ([P1]
 *        Summary: int4 with groupwise bf16 scales, group 32). */
static void dequant_row(const uint8_t* w, const void* scale, int fmt, int K, int64_t row,
                        double* out) {
    const uint8_t* wrow = w + row * (int64_t)(K / 2);
    for (int g = 0; g < K / 32; ++g) {
        int64_t si = row * (int64_t)(K / 32) + g;
        double s = fmt == ORACLE_FMT_MXFP4 ? oracle_e8m0_value(((const uint8_t*)scale)[si])
                                           : oracle_bf16_value(((const uint16_t*)scale)[si]);
        for (int i = 0; i < 32; ++i) {
            int k = g * 32 + i;
            int code = oracle_nibble(wrow, k);
            double v = fmt == ORACLE_FMT_MXFP4 ? oracle_e2m1_value(code)
                                               : (double)(code >= 8 ? code - 16 : code);
            out[k] = v * s;
        }
    }
}

void oracle_dequant(const uint8_t* w, const void* scale, int fmt,
                    int rows, int K, double* out) {
    for (int64_t r = 0; r < rows; ++r) dequant_row(w, scale, fmt, K, r, out + r * K);
}

/* --------------------------------------------------------------- routing -- */

/* Plain softmax top-k: rank experts by logit (the order of the softmax
 * probabilities), keep the first topk, and take their softmax probabilities,
 * renormalised over the kept experts when asked. The pages route inside
 * apply_monolithic ([P2]) without printing the rule; this is the plain
 * reading. Equal logits rank the lower expert index first. */
void oracle_route_topk(const float* logits, int T, int E, int topk, int renormalize,
                       int32_t* ids, float* weights) {
    char* taken = (char*)malloc((size_t)E);
    double* prob = (double*)malloc(sizeof(double) * (size_t)E);
    for (int t = 0; t < T; ++t) {
        const float* l = logits + (int64_t)t * E;
        /* softmax over all E experts */
        double lmax = -INFINITY;
        for (int e = 0; e < E; ++e)
            if ((double)l[e] > lmax) lmax = l[e];
        double denom = 0.0;
        for (int e = 0; e < E; ++e) {
            prob[e] = exp((double)l[e] - lmax);
            denom += prob[e];
        }
        for (int e = 0; e < E; ++e) prob[e] /= denom;
        /* top-k by logit, ties to the lower index */
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < topk; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e;
            }
            taken[best] = 1;
            ids[(int64_t)t * topk + j] = best;
        }
        double kept = 0.0;
        for (int j = 0; j < topk; ++j) kept += prob[ids[(int64_t)t * topk + j]];
        for (int j = 0; j < topk; ++j) {
            double p = prob[ids[(int64_t)t * topk + j]];
            weights[(int64_t)t * topk + j] = (float)(renormalize ? p / kept : p);
        }
    }
    free(prob);
    free(taken);
}

/* ------------------------------------------------------------ align/sort -- */

int64_t oracle_align_capacity(int T, int topk, int E, int bm) {
    int64_t P = (int64_t)T * topk;
    int64_t groups = P < E ? P : E;
    int64_t cap = P + groups * (bm - 1);
    return (cap + bm - 1) / bm * bm;
}

/* The grouped GEMMs of the two-stage MoE ([P1] Test plan: the two-stage MoE
 * GEMM pipeline) need the (token, slot) pairs grouped by expert. Pairs are
 * listed per expert in ascending pair index p = t*topk + j; each segment is
 * padded to a multiple of bm with the sentinel P. */
void oracle_align_sort(const int32_t* ids, int T, int topk, int E, int bm,
                       int32_t* sorted_ids, int32_t* block_expert,
                       int32_t* expert_offsets, int32_t* num_post_pad) {
    int64_t P = (int64_t)T * topk;
    int64_t cap = oracle_align_capacity(T, topk, E, bm);
    for (int64_t i = 0; i < cap; ++i) sorted_ids[i] = (int32_t)P;
    for (int64_t b = 0; b < cap / bm; ++b) block_expert[b] = -1;
    int64_t pos = 0;
    for (int e = 0; e < E; ++e) {
        expert_offsets[e] = (int32_t)pos;
        int64_t start = pos;
        for (int64_t p = 0; p < P; ++p)
            if (ids[p] == e) sorted_ids[pos++] = (int32_t)p;
        int64_t n = pos - start;
        int64_t padded = (n + bm - 1) / bm * bm;
        pos = start + padded;
        for (int64_t b = start / bm; b < pos / bm; ++b) block_expert[b] = e;
    }
    expert_offsets[E] = (int32_t)pos;
    num_post_pad[0] = (int32_t)pos;
}

/* --------------------------------------------------------------- forward -- */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* One pair (token t, expert e): gate/up projection against w13 (rows [0, I)
 * gate, rows [I, 2I) up -- the fused gate_up_proj of [P2] create_weights),
 * plus the expert's w13 bias when given, each of gate and up clamped to
 * [-limit, limit] when limit > 0, SwiGLU silu(gate) * up rounded to bf16,
 * then the down projection against w2 plus the expert's w2 bias when given.
 * y[H] out.
 * [P2] create_weights: under has_bias, w13_bias [E, 2I] and w2_bias [E, H]
 * in bf16; get_fused_moe_quant_config hands them to the kernel with the
 * layer's swiglu_limit as the GEMM1 clamp limit. The pages do not spell out
 * where the terms enter; the reading here: each bias is added to its GEMM's
 * output, the clamp applies to both GEMM1 outputs after the bias and before
 * the activation.
 * Every dot product is summed in ascending k. */
static void expert_mlp(const uint16_t* xt, const uint8_t* w13, const void* w13_scale,
                       const uint8_t* w2, const void* w2_scale, int fmt,
                       const uint16_t* w13_bias, const uint16_t* w2_bias, double limit,
                       int e, int H, int I, double* hbuf, double* y) {
    int64_t r13 = (int64_t)e * 2 * I; /* first w13 row of expert e */
    int64_t r2 = (int64_t)e * H;      /* first w2 row of expert e */
    double* xv = (double*)malloc(sizeof(double) * (size_t)H);
    for (int k = 0; k < H; ++k) xv[k] = oracle_bf16_value(xt[k]);
#pragma omp parallel
    {
        double* wg = (double*)malloc(sizeof(double) * (size_t)H);
        double* wu = (double*)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(static)
        for (int i = 0; i < I; ++i) {
            dequant_row(w13, w13_scale, fmt, H, r13 + i, wg);
            dequant_row(w13, w13_scale, fmt, H, r13 + I + i, wu);
            double g = 0.0, u = 0.0;
            for (int k = 0; k < H; ++k) {
                g += wg[k] * xv[k];
                u += wu[k] * xv[k];
            }
            if (w13_bias) {
                g += oracle_bf16_value(w13_bias[(int64_t)e * 2 * I + i]);
                u += oracle_bf16_value(w13_bias[(int64_t)e * 2 * I + I + i]);
            }
            if (limit > 0.0) {
                g = g > limit ? limit : (g < -limit ? -limit : g);
                u = u > limit ? limit : (u < -limit ? -limit : u);
            }
            /* A16W4: both grouped GEMMs take bf16 activations, so the
             * SwiGLU output enters the down projection as bf16 ([P1]
             * Summary: the BF16 x packed-int4 path; [P2] EMULATION comment:
             * bf16 activations, only the weights dequantized). */
            hbuf[i] = oracle_bf16_value(oracle_f32_to_bf16_rne((float)(silu(g) * u)));
        }
        free(wu);
        free(wg);
    }
#pragma omp parallel
    {
        double* wd = (double*)malloc(sizeof(double) * (size_t)I);
#pragma omp for schedule(static)
        for (int n = 0; n < H; ++n) {
            dequant_row(w2, w2_scale, fmt, I, r2 + n, wd);
            double acc = 0.0;
            for (int i = 0; i < I; ++i) acc += wd[i] * hbuf[i];
            if (w2_bias) acc += oracle_bf16_value(w2_bias[(int64_t)e * H + n]);
            y[n] = acc;
        }
        free(wd);
    }
    free(xv);
}

/* out[t] = sum over the token's topk slots (ascending) of weight * expert
 * MLP(x[t]); the router weight is applied at the combine, the default of
 * apply() in [P2] (apply_router_weight_on_input off). W4A16: bf16
 * activations, weights dequantized ([P2] get_fused_moe_quant_config, the
 * EMULATION comment). */
void oracle_moe_forward_ex(const uint16_t* x, const uint8_t* w13, const void* w13_scale,
                           const uint16_t* w13_bias, const uint8_t* w2, const void* w2_scale,
                           const uint16_t* w2_bias, double swiglu_limit, int fmt,
                           const int32_t* ids, const float* weights,
                           int T, int H, int I, int E, int topk,
                           const int32_t* tokens, int n_tokens, double* out) {
    double* hbuf = (double*)malloc(sizeof(double) * (size_t)I);
    double* y = (double*)malloc(sizeof(double) * (size_t)H);
    int count = tokens ? n_tokens : T;
    for (int it = 0; it < count; ++it) {
        int t = tokens ? tokens[it] : it;
        double* o = out + (int64_t)it * H;
        for (int n = 0; n < H; ++n) o[n] = 0.0;
        for (int j = 0; j < topk; ++j) {
            int e = ids[(int64_t)t * topk + j];
            if (e < 0 || e >= E) continue;
            expert_mlp(x + (int64_t)t * H, w13, w13_scale, w2, w2_scale, fmt,
                       w13_bias, w2_bias, swiglu_limit, e, H, I, hbuf, y);
            double wj = (double)weights[(int64_t)t * topk + j];
            for (int n = 0; n < H; ++n) o[n] += wj * y[n];
        }
    }
    free(y);
    free(hbuf);
}

void oracle_moe_forward(const uint16_t* x, const uint8_t* w13, const void* w13_scale,
                        const uint8_t* w2, const void* w2_scale, int fmt,
                        const int32_t* ids, const float* weights,
                        int T, int H, int I, int E, int topk,
                        const int32_t* tokens, int n_tokens, double* out) {
    oracle_moe_forward_ex(x, w13, w13_scale, NULL, w2, w2_scale, NULL, 0.0, fmt, ids, weights,
                          T, H, I, E, topk, tokens, n_tokens, out);
}

/* --------------------------------------------------------------- requant -- */

/* [P2] convert(): decode the MXFP4 block to float, multiply by its e8m0
 * scale, cast to bf16, then quantize each 1x32 group to int4 with one scale
 * (per_1x32_i4_quant) and pack two codes per byte. The pages do not print the
 * quantizer; the reading used: scale = bf16(float32(amax) / 7), codes =
 * clamp(round_half_even(v / scale), -8, 7) with a float32 divide by the
 * stored bf16 scale, an all-zero group giving scale 0 and codes 0; codes are
 * packed with the even k in the low nibble. [P1] Changes: experts are done
 * a bounded number at a time, so the range [lo, hi) is an argument. */
void oracle_requant_int4g32(const uint8_t* w, const uint8_t* scale_e8m0,
                            int E, int N, int K, int lo, int hi,
                            uint8_t* w_int4, uint16_t* scale_bf16) {
    (void)E;
    for (int e = lo; e < hi; ++e) {
        for (int n = 0; n < N; ++n) {
            int64_t row = (int64_t)e * N + n;
            const uint8_t* wrow = w + row * (K / 2);
            uint8_t* orow = w_int4 + row * (K / 2);
            for (int g = 0; g < K / 32; ++g) {
                float v[32];
                float amax = 0.0f;
                double s = oracle_e8m0_value(scale_e8m0[row * (K / 32) + g]);
                for (int i = 0; i < 32; ++i) {
                    int k = g * 32 + i;
                    float f = (float)(oracle_e2m1_value(oracle_nibble(wrow, k)) * s);
                    v[i] = (float)oracle_bf16_value(oracle_f32_to_bf16_rne(f));
                    if (fabsf(v[i]) > amax) amax = fabsf(v[i]);
                }
                uint16_t sb = oracle_f32_to_bf16_rne(amax / 7.0f);
                float sf = (float)oracle_bf16_value(sb);
                scale_bf16[row * (K / 32) + g] = sb;
                for (int i = 0; i < 32; ++i) {
                    int q = 0;
                    if (sf != 0.0f) {
                        float r = rintf(v[i] / sf); /* ties to even */
                        /* Outside the domain (e8m0 bytes 253-255, where the
                         * decoded values overflow bf16) the quotient can be
                         * inf / inf = NaN; such an element gets code 0 so the
                         * oracle stays defined there (no float -> int
                         * conversion of NaN). */
                        if (isnan(r)) r = 0.0f;
                        if (r > 7.0f) r = 7.0f;
                        if (r < -8.0f) r = -8.0f;
                        q = (int)r;
                    }
                    int k = g * 32 + i;
                    uint8_t nib = (uint8_t)(q & 0xF);
                    if ((k & 1) == 0)
                        orow[k >> 1] = nib;
                    else
                        orow[k >> 1] |= (uint8_t)(nib << 4);
                }
            }
        }
    }
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

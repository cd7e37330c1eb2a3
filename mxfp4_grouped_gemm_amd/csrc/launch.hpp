// Host-side launchers of the kernels; each checks nothing (the C ABI in
// abi.cpp validates first) and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

hipError_t launch_route_topk(const float* logits, int T, int E, int topk, int renorm, int32_t* ids,
                             float* weights, hipStream_t s);

hipError_t launch_align_sort(const int32_t* ids, int P, int topk, int E, int bm, int64_t cap,
                             int32_t* sorted_ids, int32_t* block_expert, int32_t* expert_offsets,
                             int32_t* num_post_pad, hipStream_t s);

// One token over 129-1024 experts (topk <= 64): routing by a whole
// workgroup; with sorted_ids non-null also the align/sort outputs (capacity
// topk * bm).
bool route_one_token_eligible(int T, int E, int topk);
hipError_t launch_route_one_token(const float* logits, int E, int topk, int renorm, int bm, int32_t* ids,
                                  float* weights, int32_t* sorted_ids, int32_t* block_expert,
                                  int32_t* expert_offsets, int32_t* num_post_pad, hipStream_t s);

// Routing and align/sort in one workgroup (T <= 64, T*topk <= 4096).
bool route_align_fusable(int T, int E, int topk);
hipError_t launch_route_align(const float* logits, int T, int E, int topk, int renorm, int bm,
                              int64_t cap, int32_t* ids, float* weights, int32_t* sorted_ids,
                              int32_t* block_expert, int32_t* expert_offsets, int32_t* num_post_pad,
                              hipStream_t s);

// Problem description shared by the two GEMM stages.
struct MoeGemmArgs {
    const uint16_t* x;       // bf16 [T, H]
    const uint8_t* w13;      // [E, 2I, H/2]
    const void* w13_scale;   // [E, 2I, H/32]
    const uint8_t* w2;       // [E, H, I/2]
    const void* w2_scale;    // [E, H, I/32]
    const int32_t* sorted_ids;
    const int32_t* block_expert;
    const int32_t* num_post_pad;
    uint16_t* h;             // bf16 [cap, I]   (workspace; GEMV path: [P, I] by pair)
    float* y;                // fp32 [P, H]     (workspace)
    const int32_t* topk_ids;     // [T, topk]
    const float* topk_weights;   // [T, topk]
    uint16_t* out;               // bf16 [T, H]
    const uint16_t* w13_bias;    // bf16 [E, 2I] (gate, then up) or null
    const uint16_t* w2_bias;     // bf16 [E, H] or null (added at the combine)
    float swiglu_limit;          // > 0: gate and up clamped to [-limit, limit]
    int T, H, I, E, topk, bm;
    int64_t cap;
    int fmt;
};

// GEMM1 epilogue of one (row, column i): gate g and up u after the expert's
// optional w13 bias and the optional clamp, as SwiGLU's inputs.
struct GluTerms {
    float bg, bu, lim;
    bool bias;
    __device__ __forceinline__ void load(const MoeGemmArgs& a, int e, int i) {
        bias = a.w13_bias != nullptr;
        lim = a.swiglu_limit;
        bg = bu = 0.0f;
        if (bias) {
            const uint16_t* b = a.w13_bias + (int64_t)e * 2 * a.I;
            bg = __uint_as_float((uint32_t)b[i] << 16);
            bu = __uint_as_float((uint32_t)b[a.I + i] << 16);
        }
    }
    __device__ __forceinline__ void apply(float& g, float& u) const {
        if (bias) {
            g += bg;
            u += bu;
        }
        if (lim > 0.0f) {
            g = fminf(fmaxf(g, -lim), lim);
            u = fminf(fmaxf(u, -lim), lim);
        }
    }
};

// Split-K workgroup kernels (any block size up to 64).
hipError_t launch_stage1(const MoeGemmArgs& a, hipStream_t s);
hipError_t launch_stage2(const MoeGemmArgs& a, hipStream_t s);
// One-wave-per-tile decode kernels (block size 16 or 32); stage 1 or 2.
hipError_t launch_decode_stage(const MoeGemmArgs& a, int stage, hipStream_t s);
// GEMV-shaped decode kernels (blocks of at most 8 token rows, MXFP4, H a
// multiple of 256 and I of 128, both up to 4096). h and y are stored by pair
// index.
bool gemv_eligible(const MoeGemmArgs& a);
hipError_t launch_gemv_stage(const MoeGemmArgs& a, int stage, hipStream_t s);
// The same blocks (16 rows, 2-16 of them holding pairs) with the multiply-
// adds on the matrix core (4x4x4 MFMA products over 16 K segments); MXFP4,
// H and I multiples of 64 up to 4096.
bool gemv_mfma_eligible(const MoeGemmArgs& a);
hipError_t launch_gemv_mfma_stage(const MoeGemmArgs& a, int stage, hipStream_t s);
// The same with the block's activation rows staged once per workgroup in LDS
// and up to 8 token rows per pass (blocks holding many rows).
hipError_t launch_gemv_mfma_x_stage(const MoeGemmArgs& a, int stage, hipStream_t s);
// The same products with the block's rows resident in LDS for a run of
// units, one 8-wave workgroup per compute unit (MXFP4, H and I multiples of
// 512 up to 4096).
bool gemv_resident_eligible(const MoeGemmArgs& a);
hipError_t launch_gemv_resident_stage(const MoeGemmArgs& a, int stage, hipStream_t s);

// LDS-tiled MFMA kernels for prefill sizes (MXFP4, 32-row blocks, H and I
// multiples of 256). Stage 1 first cuts the sorted blocks into super-blocks
// (list in the workspace, prefill_list_bytes(cap) bytes); stage 2 reuses it.
constexpr int64_t kPrefillMinPairs = 32;
bool prefill_eligible(const MoeGemmArgs& a);
int64_t prefill_list_bytes(int64_t cap);
hipError_t launch_prefill(const MoeGemmArgs& a, int stage, void* list_ws, hipStream_t s);

// The layer for one token, router logits in: routing inside the gate_up
// launch, then down and combine. stages: bit 0 routing + gate_up, bit 1
// down + combine.
bool t1_eligible(const MoeGemmArgs& a);
hipError_t launch_t1_layer(const MoeGemmArgs& a, const float* logits, int renorm, int32_t* topk_ids,
                           float* topk_weights, int32_t* sorted_ids, int32_t* block_expert,
                           int32_t* expert_offsets, int32_t* num_post_pad, unsigned stages, hipStream_t s);

// out[t] = sum_j weight[t, j] * (y[t*topk + j] + w2_bias[ids[t, j]]) (no
// bias term when w2_bias is null).
hipError_t launch_combine(const float* y, const int32_t* ids, const float* weights,
                          const uint16_t* w2_bias, int T, int H, int E, int topk, uint16_t* out,
                          hipStream_t s);

hipError_t launch_requant(const uint8_t* w, const uint8_t* scale, int N, int K, int lo, int hi,
                          uint8_t* q, uint16_t* qs, hipStream_t s);

}  // namespace moe

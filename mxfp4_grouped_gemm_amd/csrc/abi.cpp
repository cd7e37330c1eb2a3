// C ABI of the A16W4 MoE library: argument validation, workspace layout and
// kernel selection. Every check runs before anything is enqueued, so an
// error leaves the stream untouched (the shape checks of
// Mxfp4MoEMethod._setup_kernel and the fail-closed activation check of the
// MXFP4-to-int4 pull request).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/moe_a16w4.h"
#include "launch.hpp"

namespace {

thread_local char g_err[512] = "no error";

moe_status fail(moe_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

moe_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return MOE_OK;
    return fail(MOE_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Largest activation buffer (x or h) the GEMM kernels address with 32-bit
// buffer offsets, keeping kOob (2^31) past the end of every record.
constexpr int64_t kMaxRecordBytes = 0x7fff0000LL;
// Blocks of the 64-row kernels run along grid.y.
constexpr int64_t kMaxGridY = 65535;

bool valid_bm(int bm) { return bm == 16 || bm == 32 || bm == 64 || bm == 128 || bm == 256; }

// Block sizes the GEMM kernels are built for.
bool forward_bm(int bm) { return bm == 16 || bm == 32 || bm == 64; }

int64_t capacity(int T, int topk, int E, int bm) {
    const int64_t P = (int64_t)T * topk;
    const int64_t groups = P < E ? P : E;
    const int64_t cap = P + groups * (bm - 1);
    return (cap + bm - 1) / bm * bm;
}

int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

struct WsLayout {
    int64_t h_off, h_bytes, y_off, y_bytes, list_off, list_bytes, total;
};

WsLayout ws_layout(int T, int H, int I, int E, int topk, int bm) {
    WsLayout L;
    const int64_t cap = capacity(T, topk, E, bm);
    L.h_off = 0;
    L.h_bytes = align_up(cap * I * 2, 256);
    L.y_off = L.h_off + L.h_bytes;
    L.y_bytes = align_up((int64_t)T * topk * H * 4, 256);
    L.list_off = L.y_off + L.y_bytes;
    L.list_bytes = bm == 32 ? align_up(moe::prefill_list_bytes(cap), 256) : 0;
    L.total = L.list_off + L.list_bytes;
    return L;
}

// Every check of the forward, before anything is enqueued; fills the
// kernel arguments and the workspace layout. A call with T == 0 passes with
// a.T == 0 (nothing to launch).
moe_status prepare_forward(const char* fn, const uint16_t* x, const uint8_t* w13, const void* w13_scale,
                           const uint16_t* w13_bias, const uint8_t* w2, const void* w2_scale,
                           const uint16_t* w2_bias, moe_wfmt fmt, moe_act act, float swiglu_limit,
                           const int32_t* topk_ids, const float* topk_weights,
                           const int32_t* sorted_ids, const int32_t* block_expert,
                           const int32_t* num_post_pad, int T, int H, int I, int E, int topk,
                           int block_m, uint16_t* out, void* workspace, size_t workspace_bytes,
                           moe::MoeGemmArgs& a, WsLayout& L) {
    a.T = 0;
    if (!(swiglu_limit >= 0.0f))
        return fail(MOE_ERR_INVALID_ARG, "%s: swiglu_limit %g must be >= 0 (0 = no clamp)", fn,
                    (double)swiglu_limit);
    if (act != MOE_ACT_SWIGLU)
        return fail(MOE_ERR_UNSUPPORTED, "%s: activation %d is not implemented (only SwiGLU); "
                    "refusing to compute a different activation", fn, (int)act);
    if (fmt != MOE_W_MXFP4 && fmt != MOE_W_INT4G32)
        return fail(MOE_ERR_UNSUPPORTED, "%s: weight format %d unknown", fn, (int)fmt);
    if (T < 0) return fail(MOE_ERR_INVALID_ARG, "%s: T=%d < 0", fn, T);
    if (H < 32 || H % 32 != 0) return fail(MOE_ERR_INVALID_ARG, "%s: H=%d must be a positive multiple of 32", fn, H);
    if (I < 32 || I % 32 != 0) return fail(MOE_ERR_INVALID_ARG, "%s: I=%d must be a positive multiple of 32", fn, I);
    if (E < 1) return fail(MOE_ERR_INVALID_ARG, "%s: E=%d < 1", fn, E);
    if (topk < 1 || topk > E) return fail(MOE_ERR_INVALID_ARG, "%s: topk=%d outside [1, E=%d]", fn, topk, E);
    if (!valid_bm(block_m)) return fail(MOE_ERR_INVALID_ARG, "%s: block_m=%d invalid", fn, block_m);
    if (!forward_bm(block_m))
        return fail(MOE_ERR_UNSUPPORTED, "%s: block_m=%d not implemented (16, 32, 64)", fn, block_m);
    const int64_t P = (int64_t)T * topk;
    const int64_t cap = capacity(T, topk, E, block_m);
    if (P + cap >= (int64_t)0x7fffffff)
        return fail(MOE_ERR_UNSUPPORTED, "%s: problem too large", fn);
    // The activation kernels address x [T, H] and h [cap, I] through buffer
    // records of at most 2^31 bytes (their masked lanes use offsets past
    // 2^31), and the 64-row kernels index blocks by grid.y.
    if ((int64_t)T * H * 2 > kMaxRecordBytes || cap * I * 2 > kMaxRecordBytes)
        return fail(MOE_ERR_UNSUPPORTED,
                    "%s: T=%d gives activations beyond 2^31 bytes (x %lld B, h %lld B); "
                    "split the batch", fn, T, (long long)((int64_t)T * H * 2), (long long)(cap * I * 2));
    if (block_m == 64 && cap / block_m > kMaxGridY)
        return fail(MOE_ERR_UNSUPPORTED, "%s: %lld blocks of 64 rows exceed the grid", fn,
                    (long long)(cap / block_m));
    if (T == 0) return MOE_OK;  // nothing to launch (a.T == 0)
    const void* ptrs[] = {x, w13, w13_scale, w2, w2_scale, topk_ids, topk_weights,
                          sorted_ids, block_expert, num_post_pad, out, workspace};
    for (const void* p : ptrs)
        if (!p) return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
    for (const void* p : ptrs)
        if (!aligned(p, 16)) return fail(MOE_ERR_INVALID_ARG, "%s: pointer %p not 16-byte aligned", fn, p);
    if (!aligned(workspace, 256)) return fail(MOE_ERR_INVALID_ARG, "%s: workspace not 256-byte aligned", fn);
    if (!aligned(w13_bias, 16) || !aligned(w2_bias, 16))
        return fail(MOE_ERR_INVALID_ARG, "%s: bias pointers must be 16-byte aligned", fn);
    L = ws_layout(T, H, I, E, topk, block_m);
    if ((int64_t)workspace_bytes < L.total)
        return fail(MOE_ERR_INVALID_ARG, "%s: workspace %zu bytes < %lld needed", fn, workspace_bytes,
                    (long long)L.total);

    a.x = x;
    a.w13 = w13;
    a.w13_scale = w13_scale;
    a.w2 = w2;
    a.w2_scale = w2_scale;
    a.sorted_ids = sorted_ids;
    a.block_expert = block_expert;
    a.num_post_pad = num_post_pad;
    a.h = (uint16_t*)((char*)workspace + L.h_off);
    a.y = (float*)((char*)workspace + L.y_off);
    a.T = T;
    a.H = H;
    a.I = I;
    a.E = E;
    a.topk = topk;
    a.bm = block_m;
    a.cap = cap;
    a.fmt = (int)fmt;
    a.topk_ids = topk_ids;
    a.topk_weights = topk_weights;
    a.out = out;
    a.w13_bias = w13_bias;
    a.w2_bias = w2_bias;
    a.swiglu_limit = swiglu_limit;
    return MOE_OK;
}

// Routing and align/sort for validated arguments: one launch where the
// fused kernel applies, else the two kernels.
moe_status launch_route_align_any(const float* logits, int T, int E, int topk, int renormalize, int block_m,
                                  int64_t cap, int32_t* topk_ids, float* topk_weights, int32_t* sorted_ids,
                                  int32_t* block_expert, int32_t* expert_offsets, int32_t* num_post_pad,
                                  const char* fn, hipStream_t s) {
    const int64_t P = (int64_t)T * topk;
    if (T > 0 && moe::route_align_fusable(T, E, topk))
        return hip_status(moe::launch_route_align(logits, T, E, topk, renormalize, block_m, cap, topk_ids,
                                                  topk_weights, sorted_ids, block_expert, expert_offsets,
                                                  num_post_pad, s),
                          fn);
    if (T > 0) {
        const moe_status st = hip_status(
            moe::launch_route_topk(logits, T, E, topk, renormalize, topk_ids, topk_weights, s), fn);
        if (st != MOE_OK) return st;
    }
    return hip_status(moe::launch_align_sort(topk_ids, (int)P, topk, E, block_m, cap, sorted_ids, block_expert,
                                             expert_offsets, num_post_pad, s),
                      fn);
}

// The forward's launches for prepared arguments (stages: MOE_STAGE_* bits).
moe_status launch_forward(const moe::MoeGemmArgs& a, const WsLayout& L, void* workspace, unsigned stages,
                          hipStream_t s) {
    const int64_t P = (int64_t)a.T * a.topk;
    const int block_m = a.bm;
    moe_status st = MOE_OK;
    // Kernel family per shape: GEMV waves for blocks of <= 8 token rows,
    // the LDS-tiled MFMA kernels at prefill sizes, wave-per-tile MFMA
    // kernels for other 16/32-row blocks, split-K workgroups for 64.
    const bool decode = block_m <= 32;
    const bool gemv = decode && moe::gemv_eligible(a);
    const bool prefill = !gemv && moe::prefill_eligible(a) && P >= moe::kPrefillMinPairs;
    void* list = (char*)workspace + L.list_off;
    if (stages & MOE_STAGE_GATE_UP) {
        st = hip_status(prefill ? moe::launch_prefill(a, 1, list, s)
                        : decode ? moe::launch_decode_stage(a, 1, s) : moe::launch_stage1(a, s),
                        "moe_a16w4_forward (gate_up)");
        if (st != MOE_OK) return st;
    }
    if (stages & MOE_STAGE_DOWN) {
        st = hip_status(prefill ? moe::launch_prefill(a, 2, list, s)
                        : decode ? moe::launch_decode_stage(a, 2, s) : moe::launch_stage2(a, s),
                        "moe_a16w4_forward (down)");
        if (st != MOE_OK) return st;
    }
    if (stages & MOE_STAGE_COMBINE)
        st = hip_status(moe::launch_combine(a.y, a.topk_ids, a.topk_weights, a.w2_bias, a.T, a.H, a.E, a.topk, a.out, s),
                        "moe_a16w4_forward (combine)");
    return st;
}

}  // namespace

extern "C" {

const char* moe_last_error(void) { return g_err; }

int64_t moe_align_sort_capacity(int T, int topk, int E, int block_m) {
    if (T < 0 || topk < 1 || E < 1 || !valid_bm(block_m)) return -1;
    return capacity(T, topk, E, block_m);
}

int moe_default_block_m(int T, int topk, int E) {
    (void)topk;
    (void)E;
    // 16-row blocks on the matrix-core decode kernels up to 48 tokens (MXFP4
    // gate_up with the block's rows resident in LDS: 190 against 233 us on
    // the 32-row tiles at 16 tokens, 225 against 263 at 32, 255 against 266
    // at 48, but 285 against 269 at 64); above, the 32-row tiles.
    if (T <= 48) return 16;
    return 32;
}

moe_status moe_route_topk(const float* logits, int T, int E, int topk, int renormalize,
                          int32_t* topk_ids, float* topk_weights, void* stream) {
    if (T < 0) return fail(MOE_ERR_INVALID_ARG, "moe_route_topk: T=%d < 0", T);
    if (E < 1 || E > 1024) return fail(MOE_ERR_UNSUPPORTED, "moe_route_topk: E=%d outside [1, 1024]", E);
    if (topk < 1 || topk > E) return fail(MOE_ERR_INVALID_ARG, "moe_route_topk: topk=%d outside [1, E=%d]", topk, E);
    if (topk > 64) return fail(MOE_ERR_UNSUPPORTED, "moe_route_topk: topk=%d > 64", topk);
    if (T == 0) return MOE_OK;
    if (!logits || !topk_ids || !topk_weights)
        return fail(MOE_ERR_INVALID_ARG, "moe_route_topk: null pointer");
    if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_weights, 4))
        return fail(MOE_ERR_INVALID_ARG, "moe_route_topk: misaligned pointer");
    return hip_status(moe::launch_route_topk(logits, T, E, topk, renormalize, topk_ids, topk_weights,
                                             (hipStream_t)stream),
                      "moe_route_topk");
}

moe_status moe_align_sort(const int32_t* topk_ids, int T, int topk, int E, int block_m,
                          int32_t* sorted_ids, int32_t* block_expert, int32_t* expert_offsets,
                          int32_t* num_post_pad, void* stream) {
    if (T < 0 || topk < 1) return fail(MOE_ERR_INVALID_ARG, "moe_align_sort: T=%d topk=%d", T, topk);
    if (E < 1 || E > 1024) return fail(MOE_ERR_UNSUPPORTED, "moe_align_sort: E=%d outside [1, 1024]", E);
    if (!valid_bm(block_m))
        return fail(MOE_ERR_INVALID_ARG, "moe_align_sort: block_m=%d not in {16,32,64,128,256}", block_m);
    const int64_t P = (int64_t)T * topk;
    const int64_t cap = capacity(T, topk, E, block_m);
    if (P + cap >= (int64_t)0x7fffffff)
        return fail(MOE_ERR_UNSUPPORTED, "moe_align_sort: T*topk=%lld too large", (long long)P);
    if (!expert_offsets || !num_post_pad || (P > 0 && (!topk_ids || !sorted_ids || !block_expert)))
        return fail(MOE_ERR_INVALID_ARG, "moe_align_sort: null pointer");
    if (!aligned(topk_ids, 4) || !aligned(sorted_ids, 4) || !aligned(block_expert, 4) ||
        !aligned(expert_offsets, 4) || !aligned(num_post_pad, 4))
        return fail(MOE_ERR_INVALID_ARG, "moe_align_sort: misaligned pointer");
    return hip_status(moe::launch_align_sort(topk_ids, (int)P, topk, E, block_m, cap, sorted_ids, block_expert,
                                             expert_offsets, num_post_pad, (hipStream_t)stream),
                      "moe_align_sort");
}

moe_status moe_route_align(const float* logits, int T, int E, int topk, int renormalize,
                           int block_m, int32_t* topk_ids, float* topk_weights,
                           int32_t* sorted_ids, int32_t* block_expert, int32_t* expert_offsets,
                           int32_t* num_post_pad, void* stream) {
    const char* fn = "moe_route_align";
    if (T < 0) return fail(MOE_ERR_INVALID_ARG, "%s: T=%d < 0", fn, T);
    if (E < 1 || E > 1024) return fail(MOE_ERR_UNSUPPORTED, "%s: E=%d outside [1, 1024]", fn, E);
    if (topk < 1 || topk > E) return fail(MOE_ERR_INVALID_ARG, "%s: topk=%d outside [1, E=%d]", fn, topk, E);
    if (topk > 64) return fail(MOE_ERR_UNSUPPORTED, "%s: topk=%d > 64", fn, topk);
    if (!valid_bm(block_m))
        return fail(MOE_ERR_INVALID_ARG, "%s: block_m=%d not in {16,32,64,128,256}", fn, block_m);
    const int64_t P = (int64_t)T * topk;
    const int64_t cap = capacity(T, topk, E, block_m);
    if (P + cap >= (int64_t)0x7fffffff)
        return fail(MOE_ERR_UNSUPPORTED, "%s: T*topk=%lld too large", fn, (long long)P);
    if (!expert_offsets || !num_post_pad ||
        (P > 0 && (!logits || !topk_ids || !topk_weights || !sorted_ids || !block_expert)))
        return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
    const void* ptrs[] = {logits, topk_ids, topk_weights, sorted_ids, block_expert, expert_offsets,
                          num_post_pad};
    for (const void* p : ptrs)
        if (!aligned(p, 4)) return fail(MOE_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
    return launch_route_align_any(logits, T, E, topk, renormalize, block_m, cap, topk_ids, topk_weights,
                                  sorted_ids, block_expert, expert_offsets, num_post_pad, fn,
                                  (hipStream_t)stream);
}

int64_t moe_a16w4_workspace_size(int T, int H, int I, int E, int topk, int block_m) {
    if (T < 0 || H < 32 || I < 32 || E < 1 || topk < 1 || !valid_bm(block_m)) return -1;
    return ws_layout(T, H, I, E, topk, block_m).total;
}

moe_status moe_a16w4_forward(const uint16_t* x, const uint8_t* w13, const void* w13_scale,
                             const uint8_t* w2, const void* w2_scale, moe_wfmt fmt, moe_act act,
                             const int32_t* topk_ids, const float* topk_weights,
                             const int32_t* sorted_ids, const int32_t* block_expert,
                             const int32_t* num_post_pad, int T, int H, int I, int E, int topk,
                             int block_m, uint16_t* out, void* workspace, size_t workspace_bytes,
                             void* stream) {
    return moe_a16w4_forward_stages(x, w13, w13_scale, w2, w2_scale, fmt, act, topk_ids,
                                    topk_weights, sorted_ids, block_expert, num_post_pad, T, H, I,
                                    E, topk, block_m, out, workspace, workspace_bytes,
                                    MOE_STAGE_ALL, stream);
}

moe_status moe_a16w4_forward_stages(const uint16_t* x, const uint8_t* w13, const void* w13_scale,
                                    const uint8_t* w2, const void* w2_scale, moe_wfmt fmt,
                                    moe_act act, const int32_t* topk_ids,
                                    const float* topk_weights, const int32_t* sorted_ids,
                                    const int32_t* block_expert, const int32_t* num_post_pad, int T,
                                    int H, int I, int E, int topk, int block_m, uint16_t* out,
                                    void* workspace, size_t workspace_bytes, unsigned stages,
                                    void* stream) {
    return moe_a16w4_forward_ex(x, w13, w13_scale, nullptr, w2, w2_scale, nullptr, fmt, act, 0.0f,
                                topk_ids, topk_weights, sorted_ids, block_expert, num_post_pad, T, H,
                                I, E, topk, block_m, out, workspace, workspace_bytes, stages, stream);
}

moe_status moe_a16w4_forward_ex(const uint16_t* x, const uint8_t* w13, const void* w13_scale,
                                const uint16_t* w13_bias, const uint8_t* w2, const void* w2_scale,
                                const uint16_t* w2_bias, moe_wfmt fmt, moe_act act,
                                float swiglu_limit, const int32_t* topk_ids,
                                const float* topk_weights, const int32_t* sorted_ids,
                                const int32_t* block_expert, const int32_t* num_post_pad, int T,
                                int H, int I, int E, int topk, int block_m, uint16_t* out,
                                void* workspace, size_t workspace_bytes, unsigned stages,
                                void* stream) {
    const char* fn = "moe_a16w4_forward";
    if (stages == 0 || (stages & ~MOE_STAGE_ALL))
        return fail(MOE_ERR_INVALID_ARG, "%s: stage mask 0x%x invalid", fn, stages);
    moe::MoeGemmArgs a;
    WsLayout L;
    const moe_status st = prepare_forward(fn, x, w13, w13_scale, w13_bias, w2, w2_scale, w2_bias, fmt, act,
                                          swiglu_limit, topk_ids, topk_weights, sorted_ids, block_expert,
                                          num_post_pad, T, H, I, E, topk, block_m, out, workspace,
                                          workspace_bytes, a, L);
    if (st != MOE_OK || a.T == 0) return st;
    return launch_forward(a, L, workspace, stages, (hipStream_t)stream);
}

moe_status moe_a16w4_forward_monolithic(const uint16_t* x, const float* router_logits, const uint8_t* w13,
                                        const void* w13_scale, const uint16_t* w13_bias, const uint8_t* w2,
                                        const void* w2_scale, const uint16_t* w2_bias, moe_wfmt fmt,
                                        moe_act act, float swiglu_limit, int renormalize, int T, int H,
                                        int I, int E, int topk, int block_m, int32_t* topk_ids,
                                        float* topk_weights, int32_t* sorted_ids, int32_t* block_expert,
                                        int32_t* expert_offsets, int32_t* num_post_pad, uint16_t* out,
                                        void* workspace, size_t workspace_bytes, unsigned stages,
                                        void* stream) {
    const char* fn = "moe_a16w4_forward_monolithic";
    const unsigned down_combine = MOE_STAGE_DOWN | MOE_STAGE_COMBINE;
    if (stages != MOE_STAGE_ALL && stages != MOE_STAGE_GATE_UP && stages != down_combine)
        return fail(MOE_ERR_INVALID_ARG, "%s: stage mask 0x%x invalid (all, gate_up, or down|combine)", fn,
                    stages);
    if (E < 1 || E > 1024) return fail(MOE_ERR_UNSUPPORTED, "%s: E=%d outside [1, 1024]", fn, E);
    if (topk > 64) return fail(MOE_ERR_UNSUPPORTED, "%s: topk=%d > 64", fn, topk);
    moe::MoeGemmArgs a;
    WsLayout L;
    moe_status st = prepare_forward(fn, x, w13, w13_scale, w13_bias, w2, w2_scale, w2_bias, fmt, act,
                                    swiglu_limit, topk_ids, topk_weights, sorted_ids, block_expert,
                                    num_post_pad, T, H, I, E, topk, block_m, out, workspace, workspace_bytes,
                                    a, L);
    if (st != MOE_OK || a.T == 0) return st;
    if (!router_logits || !expert_offsets)
        return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (!aligned(router_logits, 16) || !aligned(expert_offsets, 4))
        return fail(MOE_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
    hipStream_t s = (hipStream_t)stream;
    if (moe::t1_eligible(a))
        return hip_status(moe::launch_t1_layer(a, router_logits, renormalize, topk_ids, topk_weights, sorted_ids,
                                               block_expert, expert_offsets, num_post_pad,
                                               ((stages & MOE_STAGE_GATE_UP) ? 1u : 0u) |
                                                   ((stages & down_combine) ? 2u : 0u),
                                               s),
                          fn);
    if (stages & MOE_STAGE_GATE_UP) {
        st = launch_route_align_any(router_logits, T, E, topk, renormalize, block_m, a.cap, topk_ids,
                                    topk_weights, sorted_ids, block_expert, expert_offsets, num_post_pad, fn, s);
        if (st != MOE_OK) return st;
    }
    return launch_forward(a, L, workspace, stages, s);
}

moe_status mxfp4_to_int4g32_requant(const uint8_t* w, const uint8_t* scale_e8m0, int E, int N, int K,
                                    int expert_lo, int expert_hi, uint8_t* w_int4,
                                    uint16_t* scale_bf16, void* stream) {
    const char* fn = "mxfp4_to_int4g32_requant";
    if (E < 1 || N < 1) return fail(MOE_ERR_INVALID_ARG, "%s: E=%d N=%d", fn, E, N);
    if (K < 32 || K % 32 != 0) return fail(MOE_ERR_INVALID_ARG, "%s: K=%d must be a positive multiple of 32", fn, K);
    if (expert_lo < 0 || expert_lo > expert_hi || expert_hi > E)
        return fail(MOE_ERR_INVALID_ARG, "%s: expert range [%d, %d) outside [0, %d]", fn, expert_lo, expert_hi, E);
    if (expert_lo == expert_hi) return MOE_OK;
    if (!w || !scale_e8m0 || !w_int4 || !scale_bf16) return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (!aligned(w, 16) || !aligned(w_int4, 16) || !aligned(scale_bf16, 2))
        return fail(MOE_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
    return hip_status(moe::launch_requant(w, scale_e8m0, N, K, expert_lo, expert_hi, w_int4, scale_bf16,
                                          (hipStream_t)stream),
                      fn);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free forward: the workspace is a device array of this file
// (MOE_NOALLOC_SCRATCH_BYTES), loaded with the library's code on each GPU it
// runs on and kept until the process ends. Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the
// symbol): its device address is looked up once per device, with that device
// current, and that address is the workspace of every call on the device.
namespace {

static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the first
// call on that device), or an error status.
moe_status scratch_on_current_device(void** ptr, const char* fn) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, fn);
    if (dev < 0 || dev >= kMaxDevices)
        return fail(MOE_ERR_UNSUPPORTED, "%s: device %d beyond the %d the library tracks", fn, dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, fn);
        if (!p || !aligned(p, 256)) return fail(MOE_ERR_HIP, "%s: scratch address %p unusable", fn, p);
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_a16w4_forward_noalloc(
    const uint16_t* x, const uint8_t* w13, const void* w13_scale, const uint8_t* w2,
    const void* w2_scale, moe_wfmt fmt, moe_act act, const int32_t* topk_ids,
    const float* topk_weights, const int32_t* sorted_ids, const int32_t* block_expert,
    const int32_t* num_post_pad, int T, int H, int I, int E, int topk, int block_m, uint16_t* out,
    void* stream) {
    const char* fn = "moe_a16w4_forward_noalloc";
    const int64_t need = moe_a16w4_workspace_size(T, H, I, E, topk, block_m);
    if (need < 0)
        return fail(MOE_ERR_INVALID_ARG, "%s: invalid sizes T=%d H=%d I=%d E=%d topk=%d block_m=%d", fn,
                    T, H, I, E, topk, block_m);
    if (need > (int64_t)MOE_NOALLOC_SCRATCH_BYTES)
        return fail(MOE_ERR_UNSUPPORTED,
                    "%s: this batch needs %lld workspace bytes, above the %lld-byte scratch of the "
                    "allocation-free call; use moe_a16w4_forward with a caller workspace or a smaller batch",
                    fn, (long long)need, (long long)MOE_NOALLOC_SCRATCH_BYTES);
    if (T == 0) return MOE_OK;
    void* ws = nullptr;
    const moe_status st = scratch_on_current_device(&ws, fn);
    if (st != MOE_OK) return st;
    return moe_a16w4_forward(x, w13, w13_scale, w2, w2_scale, fmt, act, topk_ids, topk_weights,
                             sorted_ids, block_expert, num_post_pad, T, H, I, E, topk, block_m, out, ws,
                             (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
}

// Top-k weighted combine: out[t] = sum over slots j (ascending) of
// weight[t, j] * y[t*topk + j], fp32 accumulation, bf16 output. The router
// weight is applied here, after the expert MLP -- the default of apply() on
// the vLLM mxfp4 API page (apply_router_weight_on_input off).
//
// One thread per 4 output columns. For topk <= 16 all slot rows are fetched
// at once with branch-free buffer loads (a slot whose expert id is outside
// [0, E) was never placed by the sort; its load gets an out-of-range offset
// and contributes zero), so the kernel is one memory round trip.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

typedef __amdgpu_buffer_rsrc_t rsrc_t;

template <int KMAX>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const int32_t* __restrict__ ids,
                                                      const float* __restrict__ weights, int T,
                                                      int H, int E, int topk,
                                                      uint16_t* __restrict__ out) {
    const int cpr = H / 4;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)T * cpr) return;
    const int t = (int)(idx / cpr);
    const int n = (int)(idx % cpr) * 4;
    const int64_t P = (int64_t)T * topk;
    const rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(y), (short)0,
                                                        (int)(P * H * 4), 0x00020000);
    f32x4 v[KMAX];
    float wj[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        const int64_t p = (int64_t)t * topk + j;
        const int e = j < topk ? ids[p] : -1;
        const bool ok = (unsigned)e < (unsigned)E;
        wj[j] = ok ? weights[p] : 0.0f;
        const uint32_t off = ok ? (uint32_t)((p * H + n) * 4) : 0x80000000u;
        v[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ry, off, 0, 0));
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        if (j >= topk) break;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(wj[j], v[j][i], acc[i]);
    }
    u32x2 o;
    o[0] = pack_bf16x2(acc[0], acc[1]);
    o[1] = pack_bf16x2(acc[2], acc[3]);
    *(u32x2*)(out + (int64_t)t * H + n) = o;
}

// Any topk: slot loop.
__global__ __launch_bounds__(256) void combine_loop_kernel(const float* __restrict__ y,
                                                           const int32_t* __restrict__ ids,
                                                           const float* __restrict__ weights,
                                                           int T, int H, int E, int topk,
                                                           uint16_t* __restrict__ out) {
    const int cpr = H / 4;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)T * cpr) return;
    const int t = (int)(idx / cpr);
    const int n = (int)(idx % cpr) * 4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < topk; ++j) {
        const int64_t p = (int64_t)t * topk + j;
        const int e = ids[p];
        if ((unsigned)e >= (unsigned)E) continue;
        const float wv = weights[p];
        const f32x4 v = *(const f32x4*)(y + p * H + n);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(wv, v[i], acc[i]);
    }
    u32x2 o;
    o[0] = pack_bf16x2(acc[0], acc[1]);
    o[1] = pack_bf16x2(acc[2], acc[3]);
    *(u32x2*)(out + (int64_t)t * H + n) = o;
}

hipError_t launch_combine(const float* y, const int32_t* ids, const float* weights, int T, int H,
                          int E, int topk, uint16_t* out, hipStream_t s) {
    const int64_t threads = (int64_t)T * (H / 4);
    const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
    const int64_t ybytes = (int64_t)T * topk * H * 4;
    if (topk <= 16 && ybytes < 0x7fff0000LL)
        hipLaunchKernelGGL(combine_kernel<16>, grid, block, 0, s, y, ids, weights, T, H, E, topk, out);
    else
        hipLaunchKernelGGL(combine_loop_kernel, grid, block, 0, s, y, ids, weights, T, H, E, topk, out);
    return hipGetLastError();
}

}  // namespace moe

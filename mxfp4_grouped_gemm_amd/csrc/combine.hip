// Top-k weighted combine: out[t] = sum over slots j (ascending) of
// weight[t, j] * y[t*topk + j], fp32 accumulation, bf16 output. The router
// weight is applied here, after the expert MLP -- the default of apply() on
// the vLLM mxfp4 API page (apply_router_weight_on_input off).
//
// One thread per 8 output columns: two 16-byte fp32 loads per slot, one
// 16-byte bf16 store. Pairs whose expert id is outside [0, E) were never
// placed by the sort and contribute nothing.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const int32_t* __restrict__ ids,
                                                      const float* __restrict__ weights, int T,
                                                      int H, int E, int topk,
                                                      uint16_t* __restrict__ out) {
    const int cpr = H / 8;
    const int64_t chunk = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (chunk >= (int64_t)T * cpr) return;
    const int t = (int)(chunk / cpr);
    const int n = (int)(chunk % cpr) * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < topk; ++j) {
        const int64_t p = (int64_t)t * topk + j;
        const int e = ids[p];
        if ((unsigned)e >= (unsigned)E) continue;
        const float wj = weights[p];
        const f32x4* src = (const f32x4*)(y + p * H + n);
        const f32x4 v0 = src[0], v1 = src[1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[i] = fmaf(wj, v0[i], acc[i]);
            acc[4 + i] = fmaf(wj, v1[i], acc[4 + i]);
        }
    }
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
    *(u32x4*)(out + (int64_t)t * H + n) = o;
}

hipError_t launch_combine(const float* y, const int32_t* ids, const float* weights, int T, int H,
                          int E, int topk, uint16_t* out, hipStream_t s) {
    const int64_t chunks = (int64_t)T * (H / 8);
    const dim3 grid((unsigned)((chunks + 255) / 256)), block(256);
    hipLaunchKernelGGL(combine_kernel, grid, block, 0, s, y, ids, weights, T, H, E, topk, out);
    return hipGetLastError();
}

}  // namespace moe

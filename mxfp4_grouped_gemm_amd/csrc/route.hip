// Softmax top-k routing kernel: one 64-lane wave per token (route.hpp).
#include "launch.hpp"
#include "route.hpp"

namespace moe {

template <int VPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int topk, int renorm,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ weights) {
    __shared__ uint64_t rk[4][64 * VPL <= 128 ? 64 * VPL : 1];
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    route_token<VPL>(logits + (int64_t)t * E, E, topk, renorm, ids + (int64_t)t * topk,
                     weights + (int64_t)t * topk, nullptr, rk[threadIdx.x >> 6]);
}

hipError_t launch_route_topk(const float* logits, int T, int E, int topk, int renorm, int32_t* ids,
                             float* weights, hipStream_t s) {
    if (route_one_token_eligible(T, E, topk))
        return launch_route_one_token(logits, E, topk, renorm, 0, ids, weights, nullptr, nullptr, nullptr,
                                      nullptr, s);
    const dim3 grid((T + 3) / 4), block(256);
    const int vpl = (E + 63) / 64;
    if (vpl <= 1)
        hipLaunchKernelGGL(route_topk_kernel<1>, grid, block, 0, s, logits, T, E, topk, renorm, ids, weights);
    else if (vpl <= 2)
        hipLaunchKernelGGL(route_topk_kernel<2>, grid, block, 0, s, logits, T, E, topk, renorm, ids, weights);
    else if (vpl <= 4)
        hipLaunchKernelGGL(route_topk_kernel<4>, grid, block, 0, s, logits, T, E, topk, renorm, ids, weights);
    else if (vpl <= 8)
        hipLaunchKernelGGL(route_topk_kernel<8>, grid, block, 0, s, logits, T, E, topk, renorm, ids, weights);
    else
        hipLaunchKernelGGL(route_topk_kernel<16>, grid, block, 0, s, logits, T, E, topk, renorm, ids, weights);
    return hipGetLastError();
}

}  // namespace moe

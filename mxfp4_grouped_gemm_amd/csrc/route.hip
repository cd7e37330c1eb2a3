// Softmax top-k routing: one 64-lane wave per token.
//
// The routing inside apply_monolithic (vLLM mxfp4 API page, Mxfp4MoEMethod)
// is not printed on the pages; this is plain softmax top-k: rank the experts
// by logit, keep the first topk (equal logits: lower index first), weight
// each kept expert by its softmax probability, renormalised over the kept
// ones on request.
//
// Each lane holds E/64 logits in registers; topk rounds of a wave-wide
// argmax (butterfly over (value, index), ties to the lower index) pick the
// experts in descending order. Lane j keeps the j-th pick, so the weights
// come from one more wave reduction.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
    return v > bv || (v == bv && i < bi);
}

template <int VPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int topk, int renorm,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ weights) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const float* row = logits + (int64_t)t * E;

    float v[VPL];
    bool avail[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int e = lane + 64 * i;
        avail[i] = e < E;
        v[i] = avail[i] ? row[e] : 0.0f;
    }

    float my_v = 0.0f;  // the pick this lane keeps (lane j <-> slot j)
    int my_id = 0;
    for (int j = 0; j < topk; ++j) {
        float bv = 0.0f;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int e = lane + 64 * i;
            if (avail[i] && (bi == 0x7fffffff || v[i] > bv)) {
                bv = v[i];
                bi = e;
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(bv, off);
            const int oi = __shfl_xor(bi, off);
            if (oi != 0x7fffffff && (bi == 0x7fffffff || better(ov, oi, bv, bi))) {
                bv = ov;
                bi = oi;
            }
        }
        // bi is now the same in every lane; its owner retires it.
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (lane + 64 * i == bi) avail[i] = false;
        if (lane == j) {
            my_v = bv;
            my_id = bi;
        }
    }

    // Softmax probabilities relative to the largest logit (slot 0).
    const float lmax = __shfl(my_v, 0);
    const bool kept = lane < topk;
    const float num = kept ? expf(my_v - lmax) : 0.0f;
    float denom;
    if (renorm) {
        denom = num;
    } else {
        denom = 0.0f;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (lane + 64 * i < E) denom += expf(v[i] - lmax);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) denom += __shfl_xor(denom, off);
    if (kept) {
        const int64_t o = (int64_t)t * topk + lane;
        ids[o] = my_id < E ? my_id : 0;
        weights[o] = num / denom;
    }
}

hipError_t launch_route_topk(const float* logits, int T, int E, int topk, int renorm, int32_t* ids,
                             float* weights, hipStream_t s) {
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

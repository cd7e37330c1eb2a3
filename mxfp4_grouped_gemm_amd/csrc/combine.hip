// Top-k weighted combine: out[t] = sum over slots j (ascending) of
// weight[t, j] * y[t*topk + j], fp32 accumulation, bf16 output. The router
// weight is applied here, after the expert MLP -- the default of apply() on
// the vLLM mxfp4 API page (apply_router_weight_on_input off).
//
// One thread per 4 output columns. For topk <= 16 a workgroup owns 1024
// columns of one token and all slot rows are fetched at once with branch-
// free buffer loads (a slot whose expert id is outside [0, E) was never
// placed by the sort; its load gets an out-of-range offset and contributes
// zero): the ids come in with scalar loads, then one vector round trip.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

template <int KMAX>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const int32_t* __restrict__ ids,
                                                      const float* __restrict__ weights, int T,
                                                      int H, int E, int topk,
                                                      uint16_t* __restrict__ out) {
    // Workgroup = (token t, 1024 columns): the token's slot ids and weights
    // are the same for every lane, so they come in with scalar loads and the
    // slot masks are uniform.
    const int cblocks = (H + 1023) / 1024;
    const int t = (int)(blockIdx.x / cblocks);
    const int n = ((int)(blockIdx.x % cblocks) * 256 + (int)threadIdx.x) * 4;
    const int64_t P = (int64_t)T * topk;
    const rsrc_t ry = make_rsrc(y, (uint32_t)(P * H * 4));
    f32x4 v[KMAX];
    float wj[KMAX];
    // Branch-free, so that every load is issued before the first wait: slots
    // past topk re-read the last slot's id and weight and get weight 0 and an
    // out-of-range row (adding 0 * 0 leaves the sum unchanged).
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        const int64_t p = (int64_t)t * topk + (j < topk ? j : topk - 1);
        const int e = ids[p];
        const float w = weights[p];
        const bool ok = j < topk && (unsigned)e < (unsigned)E;
        wj[j] = ok ? w : 0.0f;
        const uint32_t off = (ok && n < H) ? (uint32_t)((p * H + n) * 4) : kOob;
        v[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ry, off, 0, 0));
    }
    if (n >= H) return;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(wj[j], v[j][i], acc[i]);
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
    const int64_t ybytes = (int64_t)T * topk * H * 4;
    if (topk <= 16 && ybytes < 0x7fff0000LL) {
        const dim3 grid((unsigned)((int64_t)T * ((H + 1023) / 1024))), block(256);
        hipLaunchKernelGGL(combine_kernel<16>, grid, block, 0, s, y, ids, weights, T, H, E, topk, out);
    } else {
        const int64_t threads = (int64_t)T * (H / 4);
        const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
        hipLaunchKernelGGL(combine_loop_kernel, grid, block, 0, s, y, ids, weights, T, H, E, topk, out);
    }
    return hipGetLastError();
}

}  // namespace moe

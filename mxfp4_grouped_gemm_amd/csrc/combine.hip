// Top-k weighted combine: out[t] = sum over slots j (ascending) of
// weight[t, j] * y[t*topk + j], fp32 accumulation, bf16 output. The router
// weight is applied here, after the expert MLP -- the default of apply() on
// the vLLM mxfp4 API page (apply_router_weight_on_input off). With expert
// biases (create_weights under has_bias) the slot's w2 bias row joins its
// y row here: weight * (y + w2_bias[expert]).
//
// One thread per 4 output columns. For topk <= 16 a workgroup owns 1024
// columns of one token and all slot rows are fetched at once with branch-
// free buffer loads, together with the slot ids and weights (a slot whose
// expert id is outside [0, E) was never placed by the sort and contributes
// zero): one vector round trip.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

template <int KMAX, bool BIAS>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const int32_t* __restrict__ ids,
                                                      const float* __restrict__ weights,
                                                      const uint16_t* __restrict__ w2_bias, int T,
                                                      int H, int E, int topk,
                                                      uint16_t* __restrict__ out) {
    // Workgroup = (token t, 1024 columns).
    const int cblocks = (H + 1023) / 1024;
    const int t = (int)(blockIdx.x / cblocks);
    const int n = ((int)(blockIdx.x % cblocks) * 256 + (int)threadIdx.x) * 4;
    const int64_t P = (int64_t)T * topk;
    const rsrc_t ry = make_rsrc(y, (uint32_t)(P * H * 4));
    // y is read exactly once: streaming (nt) loads (42 -> 39 us at 1024 tokens).
    // The token's slot ids and weights arrive as one vector load each (lane
    // j holds slot j) together with the y rows, whose offsets depend only on
    // the slot: one memory round trip. Slots past topk get an out-of-range
    // row; a row whose id is outside [0, E) was never written and is
    // replaced by zeros after the load.
    const int lane = (int)threadIdx.x & 63;
    const int64_t p0 = (int64_t)t * topk;
    const int jl = lane < topk ? lane : topk - 1;
    const int id_l = ids[p0 + jl];
    const float w_l = weights[p0 + jl];
    f32x4 v[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        const uint32_t off = (j < topk && n < H) ? (uint32_t)(((p0 + j) * H + n) * 4) : kOob;
        v[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ry, off, 0, kNt));
    }
    // Bias rows of the slots' experts (4 bf16 per lane and slot): their
    // addresses need the ids, so they follow the y loads.
    u32x2 bv[KMAX];
    if constexpr (BIAS) {
        const rsrc_t rb = make_rsrc(w2_bias, (uint32_t)((int64_t)E * H * 2));
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            const int e = __builtin_amdgcn_readlane(id_l, j);
            const bool ok = j < topk && n < H && (unsigned)e < (unsigned)E;
            bv[j] = bld8(rb, ok ? ((uint32_t)e * (uint32_t)H + (uint32_t)n) * 2u : kOob);
        }
    }
    if (n >= H) return;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        const int e = __builtin_amdgcn_readlane(id_l, j);
        const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w_l), j));
        const bool ok = j < topk && (unsigned)e < (unsigned)E;
        f32x4 vj = ok ? v[j] : zero;
        const float w = ok ? wj : 0.0f;
        if constexpr (BIAS) {
            vj[0] += __uint_as_float(bv[j][0] << 16);
            vj[1] += __uint_as_float(bv[j][0] & 0xffff0000u);
            vj[2] += __uint_as_float(bv[j][1] << 16);
            vj[3] += __uint_as_float(bv[j][1] & 0xffff0000u);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(w, vj[i], acc[i]);
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
                                                           const uint16_t* __restrict__ w2_bias,
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
        f32x4 v = *(const f32x4*)(y + p * H + n);
        if (w2_bias) {
            const uint16_t* b = w2_bias + (int64_t)e * H + n;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] += __uint_as_float((uint32_t)b[i] << 16);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(wv, v[i], acc[i]);
    }
    u32x2 o;
    o[0] = pack_bf16x2(acc[0], acc[1]);
    o[1] = pack_bf16x2(acc[2], acc[3]);
    *(u32x2*)(out + (int64_t)t * H + n) = o;
}

hipError_t launch_combine(const float* y, const int32_t* ids, const float* weights,
                          const uint16_t* w2_bias, int T, int H, int E, int topk, uint16_t* out,
                          hipStream_t s) {
    const int64_t ybytes = (int64_t)T * topk * H * 4;
    if (topk <= 16 && ybytes < 0x7fff0000LL) {
        const dim3 grid((unsigned)((int64_t)T * ((H + 1023) / 1024))), block(256);
        if (w2_bias)
            hipLaunchKernelGGL((combine_kernel<16, true>), grid, block, 0, s, y, ids, weights, w2_bias, T, H,
                               E, topk, out);
        else
            hipLaunchKernelGGL((combine_kernel<16, false>), grid, block, 0, s, y, ids, weights, w2_bias, T,
                               H, E, topk, out);
    } else {
        const int64_t threads = (int64_t)T * (H / 4);
        const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
        hipLaunchKernelGGL(combine_loop_kernel, grid, block, 0, s, y, ids, weights, w2_bias, T, H, E, topk,
                           out);
    }
    return hipGetLastError();
}

}  // namespace moe

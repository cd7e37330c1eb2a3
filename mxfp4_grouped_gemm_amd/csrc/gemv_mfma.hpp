// Building blocks of the decode GEMMs whose multiply-adds run on the matrix
// core (v_mfma_f32_4x4x4_16b_bf16, sixteen independent 4x4x4 products per
// instruction). Lane 4b + r holds K segment b of weight row r and of token
// row r; the sixteen products of one MFMA are the sixteen K segments of a
// 4-row x 4-token product, summed across lanes once per unit (seg_sum).
#pragma once

#include "gemv.hpp"

namespace moe {

constexpr int kGmSets = 4;  // row sets of 4 weight rows per wave

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma4x4(bf16x4_t a, bf16x4_t b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a, b, c, 0, 0, 0);
}

// Sum over the 16 lanes 4b + j (b = 0..15) of each j; every lane gets its j's
// total. Rotations by 4 and 8 within 16-lane rows, then the two row swaps.
__device__ __forceinline__ float seg_sum(float v) {
    v = ror_add<0x124>(v);  // row_ror:4
    v = ror_add<0x128>(v);  // row_ror:8
    float o = v;
    permlane16_swap(v, o);
    v += o;
    o = v;
    permlane32_swap(v, o);
    return v + o;
}

// The value of lane 4 (lane / 4) + i (the same quad), for every lane.
template <int I>
__device__ __forceinline__ float quad_bcast(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x55 * I, 0xF, 0xF, false));
}

// int4-g32 weights: a lane's 16 code bytes are one 32-group of its row, so
// the products of a chunk are folded per group. The codes enter as code + 136
// (exact in bf16; the activations permuted to the codes' element order), xs
// holds the chunk's activation sums of each token and segment (an MFMA
// against ones), and acc gains scale * (sum of x (code + 136) - 136 xs), the
// scale of row slot i coming from lane 4 seg + i.
__device__ __forceinline__ void gm_int4_fold(const f32x4& t, const f32x4& xs, float sc, f32x4& acc) {
    const float s0 = quad_bcast<0>(sc), s1 = quad_bcast<1>(sc), s2 = quad_bcast<2>(sc), s3 = quad_bcast<3>(sc);
    acc[0] = fmaf(fmaf(-136.0f, xs[0], t[0]), s0, acc[0]);
    acc[1] = fmaf(fmaf(-136.0f, xs[1], t[1]), s1, acc[1]);
    acc[2] = fmaf(fmaf(-136.0f, xs[2], t[2]), s2, acc[2]);
    acc[3] = fmaf(fmaf(-136.0f, xs[3], t[3]), s3, acc[3]);
}

// Row sets after seg_sum: acc[s][i] (row slot i of set s) for this lane's
// token j = lane & 3.
__device__ __forceinline__ void gm_reduce(f32x4 (&acc)[kGmSets]) {
#pragma unroll
    for (int s = 0; s < kGmSets; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[s][i] = seg_sum(acc[s][i]);
}

}  // namespace moe

// Wave-level softmax top-k routing of one token (device code).
//
// The plain softmax top-k that apply_monolithic performs in-kernel (vLLM
// mxfp4 API page, Mxfp4MoEMethod): rank the experts by logit, keep the first
// topk (equal logits: lower index first), weight them by their softmax
// probabilities, renormalised over the kept experts on request.
//
// Up to 128 experts, every lane ranks its own experts directly: it counts
// the experts ordered before each of them (larger key, or equal key and lower
// index) against the token's keys in the wave's LDS scratch, and keeps those
// ranked below topk. For more experts, selection is a radix select over
// order-preserving 32-bit keys: 16 rounds of (compare, ballot, popcount) over
// two key bits find the k-th largest key; keys above it are kept and the
// ties at it are taken lowest index first; the kept experts are then ranked
// against each other in a scalar loop of at most topk steps. A single token
// over more than 128 experts is routed by a whole workgroup instead
// (route_t1.hip).
#pragma once

#include "common.hpp"

namespace moe {

// Order-preserving key of a float: larger float -> larger key; -0 maps to +0
// so that equal logits compare equal.
__device__ __forceinline__ uint32_t route_key(float v) {
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float route_key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ int wave_popc(bool pred) { return __popcll(__ballot(pred)); }

template <int CTRL>
__device__ __forceinline__ uint32_t ror_max_u32(uint32_t v) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
    return v > o ? v : o;
}

// Maximum over the wave (all 64 lanes active).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = ror_max_u32<0x128>(v);  // row_ror:8
    v = ror_max_u32<0x124>(v);  // row_ror:4
    v = ror_max_u32<0x122>(v);  // row_ror:2
    v = ror_max_u32<0x121>(v);  // row_ror:1 -- every lane holds its row's maximum
    uint32_t m = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    const uint32_t m1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t m2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    const uint32_t m3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    m = m1 > m ? m1 : m;
    m = m2 > m ? m2 : m;
    return m3 > m ? m3 : m;
}

// Routes one token with one wave. Lane-local slots i hold expert lane + 64 i
// (VPL * 64 >= E). Writes ids[rank] and weights[rank] for rank < topk.
// rk: this wave's LDS scratch of 64 * VPL entries (used when VPL <= 2).
template <int VPL>
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int topk, int renorm,
                                            int32_t* __restrict__ ids, float* __restrict__ weights,
                                            int32_t* __restrict__ ids_lds, uint64_t* __restrict__ rk) {
    const int lane = threadIdx.x & 63;
    float val[VPL];
    uint32_t key[VPL];
    bool ok[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int e = lane + 64 * i;
        ok[i] = e < E;
        val[i] = ok[i] ? row[e] : 0.0f;
        key[i] = route_key(val[i]);
    }
    bool sel[VPL];
    int rank[VPL];
    uint32_t kmax = 0u;
    if constexpr (VPL <= 2) {
    // Up to 128 experts: every lane counts, for each of its experts, the
    // experts ranked before it -- larger key, or equal key and lower index:
    // one 64-bit compare of (key, ~index) against each entry of the token's
    // keys in wave-private LDS (broadcast reads). No scalar chains.
    uint64_t* kk = rk;
    uint64_t k64[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const uint32_t e = (uint32_t)(lane + 64 * i);
        k64[i] = ok[i] ? ((uint64_t)key[i] << 32) | (uint64_t)~e : 0ull;
        kk[e] = k64[i];
        rank[i] = 0;
    }
    wave_lds_sync();
    for (int j = 0; j < E; j += 2) {
        const uint64_t kj0 = kk[j], kj1 = kk[j + 1];  // entries up to 64 * VPL hold 0 past E
#pragma unroll
        for (int i = 0; i < VPL; ++i) rank[i] += (kj0 > k64[i] ? 1 : 0) + (kj1 > k64[i] ? 1 : 0);
    }
    wave_lds_sync();  // the next token's keys overwrite this wave's entries
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        sel[i] = ok[i] && rank[i] < topk;
        if (sel[i] && rank[i] == 0) kmax = key[i];
    }
    kmax = wave_max_u32(kmax);
    } else {
    // k-th largest key: the largest T with count(key >= T) >= topk, two key
    // bits per round (three independent counts). Slots past E get key 0,
    // which no candidate (always >= 1) counts.
    uint32_t kv[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) kv[i] = ok[i] ? key[i] : 0u;
    uint32_t thr = 0u;
#pragma unroll
    for (int bit = 30; bit >= 0; bit -= 2) {
        const uint32_t c1 = thr | (1u << bit), c2 = thr | (2u << bit), c3 = thr | (3u << bit);
        int n1 = 0, n2 = 0, n3 = 0;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            n1 += __popcll(__builtin_amdgcn_ballot_w64(kv[i] >= c1));
            n2 += __popcll(__builtin_amdgcn_ballot_w64(kv[i] >= c2));
            n3 += __popcll(__builtin_amdgcn_ballot_w64(kv[i] >= c3));
        }
        thr = n3 >= topk ? c3 : n2 >= topk ? c2 : n1 >= topk ? c1 : thr;
    }
    int above = 0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) above += wave_popc(ok[i] && key[i] > thr);
    // Keep everything above thr, then ties at thr in index order (slot-major).
    int need = topk - above;
    const uint64_t below_me = (1ull << lane) - 1ull;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const bool tie = ok[i] && key[i] == thr;
        const uint64_t tm = __ballot(tie);
        const int before = __popcll(tm & below_me);
        sel[i] = (ok[i] && key[i] > thr) || (tie && before < need);
        const int c = __popcll(tm);
        need -= c < need ? c : need;
    }
    // Rank the kept experts: by key descending, then index ascending. The
    // largest kept key gives the softmax shift.
#pragma unroll
    for (int i = 0; i < VPL; ++i) rank[i] = 0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        uint64_t m = __ballot(sel[i]);
        while (m) {
            const int src = __ffsll((unsigned long long)m) - 1;
            m &= m - 1ull;
            const uint32_t kv = (uint32_t)__builtin_amdgcn_readlane((int)key[i], src);
            const int ev = src + 64 * i;
            kmax = kv > kmax ? kv : kmax;
#pragma unroll
            for (int j = 0; j < VPL; ++j) {
                const int e = lane + 64 * j;
                rank[j] += (kv > key[j] || (kv == key[j] && ev < e)) ? 1 : 0;
            }
        }
    }
    }
    const float lmax = route_key_value(kmax);
    float ex[VPL];
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        ex[i] = ok[i] ? expf(val[i] - lmax) : 0.0f;
        if (renorm ? sel[i] : ok[i]) part += ex[i];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        if (sel[i] && rank[i] < topk) {
            const int e = lane + 64 * i;
            ids[rank[i]] = e;
            weights[rank[i]] = ex[i] / part;
            if (ids_lds) ids_lds[rank[i]] = e;
        }
    }
}

}  // namespace moe

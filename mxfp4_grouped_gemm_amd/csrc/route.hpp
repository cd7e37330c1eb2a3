// Wave-level softmax top-k routing of one token (device code).
//
// The plain softmax top-k that apply_monolithic performs in-kernel (vLLM
// mxfp4 API page, Mxfp4MoEMethod): rank the experts by logit, keep the first
// topk (equal logits: lower index first), weight them by their softmax
// probabilities, renormalised over the kept experts on request.
//
// Up to 128 experts, one round of guesses (else a few radix rounds) finds a
// key threshold that at least topk and only a few more experts reach; every
// lane then ranks its candidates directly: it counts the candidates ordered
// before each of them (larger key, or equal key and lower index) against
// their keys in the wave's LDS scratch, and keeps those ranked below topk.
// For more experts, selection is a radix select over
// order-preserving 32-bit keys: 16 rounds of (compare, ballot, popcount) over
// two key bits find the k-th largest key; keys above it are kept and the
// ties at it are taken lowest index first; the kept experts are then ranked
// against each other in a scalar loop of at most topk steps. A single token
// over more than 128 experts is routed by a whole workgroup instead
// (route_t1.hip).
#pragma once

#include "common.hpp"
#include "gemv.hpp"

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

// Candidate threshold for the top-k of up to 64 VPL keys (kv: the lane's
// order-preserving keys, 0 for slots past E, n: the count of valid keys on
// entry): the largest thr, refined B key bits a round (2^B - 1 compares and
// ballots per slot, all independent), with at least need keys >= thr,
// stopping as soon as at most stop keys reach it. On return n = the count of
// keys >= thr. A radix select carried to the last bit gives the need-th
// largest key itself.
template <int VPL, int B>
__device__ __forceinline__ uint32_t key_threshold(const uint32_t (&kv)[VPL], int need, int stop, int& n) {
    constexpr int C = (1 << B) - 1;
    uint32_t thr = 0u;
    for (int bit = 32 - B; bit >= 0 && n > stop; bit -= B) {
        int ge = 0;  // candidates c (1..C) with count(key >= thr | c << bit) >= need
#pragma unroll
        for (int c = 1; c <= C; ++c) {
            const uint32_t t = thr | ((uint32_t)c << bit);
            int cnt = 0;
#pragma unroll
            for (int i = 0; i < VPL; ++i) cnt += __popcll(__builtin_amdgcn_ballot_w64(kv[i] >= t));
            ge += cnt >= need ? 1 : 0;  // counts fall as c grows
        }
        thr |= (uint32_t)ge << bit;
        if (ge > 0) {
            int cnt = 0;
#pragma unroll
            for (int i = 0; i < VPL; ++i) cnt += __popcll(__builtin_amdgcn_ballot_w64(kv[i] >= thr));
            n = cnt;
        }
    }
    return thr;
}

// The 64-lane sum with the pairing of a xor butterfly over lane offsets 32,
// 16, 8, 4, 2, 1 (each lane adds its partner's partial sum to its own, so
// every lane ends with the same bits), by register swaps and DPP rotations
// instead of six LDS permutes: after the first two steps a row's values are
// symmetric under xor 8, so a rotation by 8, 4, 2, 1 meets a lane holding
// the xor partner's value.
__device__ __forceinline__ float wave_sum_butterfly(float v) {
    float a = v, b = v;
    permlane32_swap(a, b);
    v = a + b;
    a = v;
    b = v;
    permlane16_swap(a, b);
    return row16_sum(a + b);
}

// The lane's logits of one token (slot i: expert lane + 64 i; zero past E),
// all issued before any is used: one round trip.
template <int VPL>
__device__ __forceinline__ void route_load(const float* __restrict__ row, int E, float (&val)[VPL]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int e = lane + 64 * i;
        val[i] = e < E ? row[e] : 0.0f;
    }
}

// Candidate threshold from one round of guesses, for up to 64 VPL keys (kv
// and n as for key_threshold; ok: the slot holds an expert): 15 values
// spread evenly between the token's smallest and largest logit, as keys
// (lane c holds guess c), each counted with one ballot per slot. The largest
// guess that at least need keys reach is a valid threshold; if none
// qualifies, or more than stop keys reach the best one, the radix rounds of
// key_threshold take over. One round of independent counts instead of ~5
// dependent ones. kmax: the largest key (the token's first expert).
template <int VPL>
__device__ __forceinline__ uint32_t key_guess_threshold(const uint32_t (&kv)[VPL], const bool (&ok)[VPL], int E,
                                                        int need, int stop, int& n, uint32_t& kmax) {
    uint32_t hi = 0u, lo_inv = 0u;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        hi = kv[i] > hi ? kv[i] : hi;
        const uint32_t inv = ok[i] ? ~kv[i] : 0u;
        lo_inv = inv > lo_inv ? inv : lo_inv;
    }
    hi = wave_max_u32(hi);
    const uint32_t lo = ~wave_max_u32(lo_inv);
    kmax = hi;
    const float vlo = route_key_value(lo), vhi = route_key_value(hi);
    const uint32_t g = route_key(vlo + (vhi - vlo) * ((float)(threadIdx.x & 15) * 0.0625f));
    uint32_t thr = 0u;
    n = E;
#pragma unroll
    for (int c = 1; c < 16; ++c) {
        const uint32_t t = (uint32_t)__builtin_amdgcn_readlane((int)g, c);
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < VPL; ++i) cnt += __popcll(__builtin_amdgcn_ballot_w64(kv[i] >= t));
        if (cnt >= need) {  // guesses rise with c: the last that qualifies is the largest
            thr = t;
            n = cnt;
        }
    }
    if (n > stop) {
        n = E;
        thr = key_threshold<VPL, 2>(kv, need, stop, n);
    }
    return thr;
}

// Inclusive prefix sum over the 64 lanes of a wave (all active), by DPP
// instead of six LDS permutes: row shifts by 1, 2, 4 and 8 scan each 16-lane
// row (lanes shifted in from outside the row add 0), then lane 15's total
// is broadcast into rows 1 and 3 and lane 31's into rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
    return v;
}

// Routes one token with one wave from its loaded logits (route_load).
// Writes ids[rank] and weights[rank] for rank < topk (and ids_lds[rank] if
// given). rk: this wave's LDS scratch of 64 * VPL entries (used only when
// VPL <= 2).
template <int VPL>
__device__ __forceinline__ void route_token_vals(const float (&val)[VPL], int E, int topk, int renorm,
                                                 int32_t* __restrict__ ids, float* __restrict__ weights,
                                                 int32_t* __restrict__ ids_lds, uint64_t* __restrict__ rk) {
    const int lane = threadIdx.x & 63;
    uint32_t key[VPL];
    bool ok[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        ok[i] = lane + 64 * i < E;
        key[i] = route_key(val[i]);
    }
    bool sel[VPL];
    int rank[VPL];
    uint32_t kmax = 0u;
    if constexpr (VPL <= 2) {
    // Up to 128 experts. First a threshold thr with at least topk keys >= thr
    // (so every kept expert has key >= thr) and few more: the best of 15
    // guesses between the smallest and largest logit (N(0,1) logits: ~20 of
    // 112 reach it), else radix rounds of two key bits, as in the radix
    // select below, stopping once at most topk + 16 keys reach it. Only
    // those candidates are then ranked exactly: each lane compares its
    // (key, ~index) against the candidates' entries, compacted into
    // wave-private LDS (broadcast reads); a candidate's rank among them is
    // its rank among all experts, since
    // every other expert has a smaller key. No scalar chains beyond the
    // rounds, and the compare count is the candidates', not E. In the fused
    // route + align kernel (16 waves routing on one CU) the kernel went from
    // 8.9 to 6.7 us at 16 tokens of 112 experts and from 13.9 to 10.0 us at
    // 32 with the radix rounds alone (~190 ns each, latency-bound), to 6.2
    // and 9.2 us with the guesses first. Four key bits a round (15 compares
    // per slot) took longer than two.
    uint32_t kv[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) kv[i] = ok[i] ? key[i] : 0u;
    int n = E;
    const uint32_t thr = key_guess_threshold<VPL>(kv, ok, E, topk, topk + 16, n, kmax);
    uint64_t* kk = rk;
    uint64_t k64[VPL];
    bool cand[VPL];
    const uint64_t below_me = (1ull << lane) - 1ull;
    int base = 0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const uint32_t e = (uint32_t)(lane + 64 * i);
        k64[i] = ((uint64_t)key[i] << 32) | (uint64_t)~e;
        cand[i] = ok[i] && key[i] >= thr;
        const uint64_t m = __ballot(cand[i]);
        if (cand[i]) kk[base + __popcll(m & below_me)] = k64[i];
        base += __popcll(m);
        rank[i] = 0;
    }
    // Zero entries up to a multiple of 4 (never above a candidate's entry);
    // base <= E <= 64 VPL, a multiple of 4, so they stay inside the scratch.
    const int n4 = (base + 3) & ~3;
    if (base + lane < n4) kk[base + lane] = 0ull;
    wave_lds_sync();
    for (int j = 0; j < n4; j += 4) {
        const uint64_t kj0 = kk[j], kj1 = kk[j + 1], kj2 = kk[j + 2], kj3 = kk[j + 3];
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            rank[i] += (kj0 > k64[i] ? 1 : 0) + (kj1 > k64[i] ? 1 : 0) + (kj2 > k64[i] ? 1 : 0) +
                       (kj3 > k64[i] ? 1 : 0);
    }
    wave_lds_sync();  // the next token's entries overwrite this wave's scratch
#pragma unroll
    for (int i = 0; i < VPL; ++i) sel[i] = cand[i] && rank[i] < topk;
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
    part = wave_sum_butterfly(part);
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

// Loads and routes one token with one wave (route_load, route_token_vals).
template <int VPL>
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int topk, int renorm,
                                            int32_t* __restrict__ ids, float* __restrict__ weights,
                                            int32_t* __restrict__ ids_lds, uint64_t* __restrict__ rk) {
    float val[VPL];
    route_load<VPL>(row, E, val);
    route_token_vals<VPL>(val, E, topk, renorm, ids, weights, ids_lds, rk);
}

}  // namespace moe

// Routing of a single token over 129-1024 experts by one 1024-thread
// workgroup, optionally with the align/sort outputs (the plain softmax top-k
// of apply_monolithic on the vLLM mxfp4 API page, Mxfp4MoEMethod).
//
// Thread e holds expert e. The k-th largest order-preserving key comes from
// a 64-bin histogram of the logits between their minimum and maximum when
// the bins reaching topk from the top hold at most 64 keys (wave 0 then
// picks it among them); otherwise from a radix select over the whole
// workgroup: four rounds of an 8-bit digit,
// each an LDS histogram of the digit over the keys that match the digits
// chosen so far and a scan of the 256 bins (wave 0) from the top. Keys above
// it are kept, and the ties at it are taken lowest index first (one
// workgroup scan of the "above" and "equal" predicates in index order also
// gives every expert's position among the kept ones). Wave 0 then ranks the
// at most 64 kept experts against each other and forms the softmax terms
// laid out as the single-wave routing holds them (expert lane + 64 i in
// slot i of lane `lane`), summed in the same order, so ids and weights equal
// its results bit for bit.
//
// With one token every kept expert holds exactly one pair, so the align /
// sort outputs follow from the routing: block j (experts in ascending
// order) holds pair rank(expert) in its first row and padding elsewhere;
// expert e's segment starts at (kept experts below e) * block_m.
#include "launch.hpp"
#include "route.hpp"

namespace moe {

constexpr int kT1RouteThreads = 1024;

template <bool ALIGN>
__global__ __launch_bounds__(kT1RouteThreads) void route_one_token_kernel(
    const float* __restrict__ logits, int E, int topk, int renorm, int bm, int32_t* __restrict__ ids,
    float* __restrict__ weights, int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ num_post_pad) {
    __shared__ float lv[kT1RouteThreads];
    __shared__ uint8_t kept[kT1RouteThreads];
    __shared__ uint32_t hist[256];
    __shared__ uint32_t s_prefix;
    __shared__ int s_need;
    __shared__ int wgt[kT1RouteThreads / 64], weq[kT1RouteThreads / 64];
    __shared__ int list[64];
    __shared__ uint64_t kk[68];  // kept experts' (key, ~index), zeros up to a multiple of 4
    __shared__ uint32_t wmax[kT1RouteThreads / 64], wmin_inv[kT1RouteThreads / 64];
    __shared__ uint32_t ckey[64];
    __shared__ int s_bin, s_ncand, s_slot;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int e = tid;
    const bool ok = e < E;
    const float v = ok ? logits[e] : 0.0f;
    const uint32_t key = ok ? route_key(v) : 0u;  // valid keys are >= 1
    lv[e] = v;

    // 1. The k-th largest key. First from a 64-bin histogram of the logits
    // between the token's smallest and largest: the bins from the top down
    // to the one where the count reaches topk hold every key from the k-th
    // largest up (bins rise with the value); when they hold at most 64 keys,
    // wave 0 finds the k-th largest among them. Non-finite extremes, equal
    // extremes or more candidates (heavy ties) take the radix select.
    uint32_t prefix = 0u;
    int need = topk;
    const uint32_t wmx = wave_max_u32(key), wmn = wave_max_u32(ok ? ~key : 0u);
    if (lane == 0) {
        wmax[wave] = wmx;
        wmin_inv[wave] = wmn;
    }
    if (tid < 64) {
        hist[tid] = 0u;
        ckey[tid] = 0u;  // below every key of a finite logit
    }
    if (tid == 0) s_slot = 0;
    __syncthreads();
    uint32_t kmx = 0u, kmn_inv = 0u;
#pragma unroll
    for (int w = 0; w < kT1RouteThreads / 64; ++w) {
        kmx = wmax[w] > kmx ? wmax[w] : kmx;
        kmn_inv = wmin_inv[w] > kmn_inv ? wmin_inv[w] : kmn_inv;
    }
    const float lo = route_key_value(~kmn_inv), hi = route_key_value(kmx);
    const bool binned = __builtin_isfinite(lo) && __builtin_isfinite(hi) && hi > lo;  // uniform
    const float scale = binned ? 64.0f / (hi - lo) : 0.0f;
    int bin = 0;
    if (binned) {
        const float f = (v - lo) * scale;  // rises with v
        bin = f >= 63.0f ? 63 : (f > 0.0f ? (int)f : 0);
        if (ok) atomicAdd(&hist[bin], 1u);
    }
    __syncthreads();
    if (wave == 0) {
        // Lane l holds bin 63 - l; inclusive counts from the top.
        const uint32_t c = hist[63 - lane];
        const uint32_t incl = (uint32_t)wave_incl_scan((int)c);
        const uint64_t reach = __ballot(incl >= (uint32_t)topk);
        const int l = reach ? __ffsll((unsigned long long)reach) - 1 : 63;
        if (lane == 0) {
            s_bin = 63 - l;
            s_ncand = binned ? (int)__builtin_amdgcn_readlane((int)incl, l) : E + 1;
        }
    }
    __syncthreads();
    const int cbin = s_bin, ncand = s_ncand;
    if (ncand <= 64) {
        if (ok && bin >= cbin) ckey[atomicAdd(&s_slot, 1)] = key;
        __syncthreads();
        if (wave == 0) {
            // The k-th largest key: the candidate with fewer than topk keys
            // above it and at least topk at or above it.
            // Entries past ncand are zero and count for no candidate; read
            // four at a time (ncand <= 64, so i + 3 < 64).
            const uint32_t kj = lane < ncand ? ckey[lane] : 0u;
            int above = 0, atleast = 0;
            for (int i = 0; i < ncand; i += 4) {
                const uint32_t k0 = ckey[i], k1 = ckey[i + 1], k2 = ckey[i + 2], k3 = ckey[i + 3];
                above += (k0 > kj ? 1 : 0) + (k1 > kj ? 1 : 0) + (k2 > kj ? 1 : 0) + (k3 > kj ? 1 : 0);
                atleast += (k0 >= kj ? 1 : 0) + (k1 >= kj ? 1 : 0) + (k2 >= kj ? 1 : 0) + (k3 >= kj ? 1 : 0);
            }
            if (lane < ncand && above < topk && atleast >= topk) {  // lanes holding that key agree
                s_prefix = kj;
                s_need = topk - above;
            }
        }
        __syncthreads();
        prefix = s_prefix;
        need = s_need;
    } else {
    // Radix select: 8 bits a round from the top.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int shift = 24 - 8 * r;
        if (tid < 256) hist[tid] = 0u;
        __syncthreads();
        const bool match = ok && (r == 0 || (key >> (shift + 8)) == (prefix >> (shift + 8)));
        if (match) atomicAdd(&hist[(key >> shift) & 255u], 1u);
        __syncthreads();
        if (wave == 0) {
            // Lane l holds digits 255 - 4l .. 252 - 4l, highest first.
            uint32_t c[4], local = 0u;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                c[q] = hist[255 - 4 * lane - q];
                local += c[q];
            }
            const uint32_t incl = (uint32_t)wave_incl_scan((int)local);
            const uint32_t excl = incl - local;
            if (excl < (uint32_t)need && (uint32_t)need <= incl) {  // exactly one lane
                uint32_t before = excl;
                int q = 0;
#pragma unroll
                for (int t = 0; t < 3; ++t) {
                    if (before + c[q] < (uint32_t)need) {
                        before += c[q];
                        ++q;
                    }
                }
                s_prefix = prefix | ((uint32_t)(255 - 4 * lane - q) << shift);
                s_need = need - (int)before;
            }
        }
        __syncthreads();
        prefix = s_prefix;
        need = s_need;
    }
    }
    const uint32_t thr = prefix;  // the k-th largest key; take `need` of the keys equal to it

    // 2. Keep the keys above thr and the first `need` equal ones (index
    // order); pos = kept experts below e.
    const bool gt = ok && key > thr, eq = ok && key == thr;
    const uint64_t below = (1ull << lane) - 1ull;
    const uint64_t mgt = __ballot(gt), meq = __ballot(eq);
    if (lane == 0) {
        wgt[wave] = __popcll(mgt);
        weq[wave] = __popcll(meq);
    }
    __syncthreads();
    int gt_before = __popcll(mgt & below), eq_before = __popcll(meq & below);
    for (int w = 0; w < wave; ++w) {
        gt_before += wgt[w];
        eq_before += weq[w];
    }
    const bool sel = gt || (eq && eq_before < need);
    const int pos = gt_before + (eq_before < need ? eq_before : need);
    kept[e] = sel ? 1 : 0;
    if (sel) {
        list[pos] = e;
        kk[pos] = ((uint64_t)key << 32) | (uint64_t)~(uint32_t)e;
    }
    if (tid < 4) kk[topk + tid] = 0ull;
    if (ALIGN) {
        if (ok) expert_offsets[e] = pos * bm;
        if (tid == 0) {
            expert_offsets[E] = topk * bm;
            *num_post_pad = topk * bm;
        }
        // One token: P = topk, capacity topk * bm; padding rows hold P.
        for (int i = tid; i < topk * bm; i += kT1RouteThreads)
            if (i % bm != 0) sorted_ids[i] = topk;
    }
    __syncthreads();

    // 3. Wave 0: ranks among the kept experts, softmax in the single-wave
    // routing's order, outputs.
    if (wave == 0) {
        // Rank = kept entries ordered before this one: larger key, or equal
        // key and lower index (one 64-bit compare of (key, ~index)); the
        // entries are read four at a time with no dependent chain.
        const bool has = lane < topk;
        const int ej = has ? list[lane] : 0;
        const uint64_t kj = has ? kk[lane] : 0ull;
        int rank = 0;
        for (int i = 0; i < topk; i += 4) {
            const uint64_t k0 = kk[i], k1 = kk[i + 1], k2 = kk[i + 2], k3 = kk[i + 3];
            rank += (k0 > kj ? 1 : 0) + (k1 > kj ? 1 : 0) + (k2 > kj ? 1 : 0) + (k3 > kj ? 1 : 0);
        }
        const uint32_t kmax = wave_max_u32((uint32_t)(kj >> 32));
        const float lmax = route_key_value(kmax);
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < kT1RouteThreads / 64; ++i) {  // unrolled: every read in flight at once
            const int x = lane + 64 * i;
            if (x < E) {
                const float ex = expf(lv[x] - lmax);
                if (!renorm || kept[x]) part += ex;
            }
        }
        part = wave_sum_butterfly(part);
        if (has) {
            ids[rank] = ej;
            weights[rank] = expf(lv[ej] - lmax) / part;
            if (ALIGN) {
                block_expert[lane] = ej;
                sorted_ids[lane * bm] = rank;
            }
        }
    }
}

bool route_one_token_eligible(int T, int E, int topk) {
    return T == 1 && E > 128 && E <= kT1RouteThreads && topk >= 1 && topk <= 64 && topk <= E;
}

hipError_t launch_route_one_token(const float* logits, int E, int topk, int renorm, int bm, int32_t* ids,
                                  float* weights, int32_t* sorted_ids, int32_t* block_expert,
                                  int32_t* expert_offsets, int32_t* num_post_pad, hipStream_t s) {
    if (sorted_ids)
        hipLaunchKernelGGL(route_one_token_kernel<true>, dim3(1), dim3(kT1RouteThreads), 0, s, logits, E, topk,
                           renorm, bm, ids, weights, sorted_ids, block_expert, expert_offsets, num_post_pad);
    else
        hipLaunchKernelGGL(route_one_token_kernel<false>, dim3(1), dim3(kT1RouteThreads), 0, s, logits, E, topk,
                           renorm, bm, ids, weights, nullptr, nullptr, nullptr, nullptr);
    return hipGetLastError();
}

}  // namespace moe

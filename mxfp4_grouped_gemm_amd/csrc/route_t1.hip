// Routing of a single token over 129-1024 experts by one 1024-thread
// workgroup, optionally with the align/sort outputs (the plain softmax top-k
// of apply_monolithic on the vLLM mxfp4 API page, Mxfp4MoEMethod).
//
// Thread e holds expert e. The k-th largest order-preserving key is found
// by a radix select over the whole workgroup: four rounds of an 8-bit digit,
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
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int e = tid;
    const bool ok = e < E;
    const float v = ok ? logits[e] : 0.0f;
    const uint32_t key = ok ? route_key(v) : 0u;  // valid keys are >= 1
    lv[e] = v;

    // 1. The k-th largest key, 8 bits a round from the top.
    uint32_t prefix = 0u;
    int need = topk;
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
            uint32_t incl = local;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t o = __shfl_up(incl, off);
                if (lane >= off) incl += o;
            }
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
    if (sel) list[pos] = e;
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
        const bool has = lane < topk;
        const int ej = has ? list[lane] : 0;
        const uint32_t kj = has ? route_key(lv[ej]) : 0u;
        int rank = 0;
        for (int i = 0; i < topk; ++i) {
            const uint32_t ki = route_key(lv[list[i]]);
            rank += (ki > kj || (ki == kj && i < lane)) ? 1 : 0;  // list is in index order
        }
        const uint32_t kmax = wave_max_u32(kj);
        const float lmax = route_key_value(kmax);
        float part = 0.0f;
        for (int i = 0; 64 * i < E; ++i) {
            const int x = lane + 64 * i;
            if (x < E) {
                const float ex = expf(lv[x] - lmax);
                if (!renorm || kept[x]) part += ex;
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
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

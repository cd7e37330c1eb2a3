// Token-to-expert align/sort: group the (token, slot) pairs by expert, in
// ascending pair index within each expert, and pad every expert segment to
// a multiple of the GEMM block. The two-stage MoE GEMM of the pages (the
// MXFP4-to-int4 pull request, Test plan) consumes such per-expert blocks;
// the grouping rule itself is the plain stable one.
//
// One 1024-thread workgroup. Counts come from LDS atomic adds (order does
// not matter for a count). Positions never come from atomic order. When
// every token's pairs name distinct experts (the routing's always do), a
// token-by-expert bit matrix in LDS (bit t of expert e's row set when token
// t chose e) gives each pair its rank directly: the set bits of its
// expert's row below its token, from a per-word prefix of the row, so the
// pairs are placed in one pass (at 1024 tokens x 15 slots: 29 -> 5 us, see
// the launcher). Otherwise (a token naming an expert twice, or a matrix too
// large for the LDS) pairs are processed in tiles of 1024, each wave ORs one
// bit per pair into a per-(wave, expert) 64-bit mask, and a pair's rank is
// the popcount of the bits below it plus the counts of earlier waves and
// tiles. Both are the stable counting sort, bit-identical run to run.
//
// route_align_kernel runs the routing of up to 64 tokens (route.hpp, one
// wave per token) in the same workgroup and sorts straight from LDS, saving
// a launch and a round trip of the ids through memory at decode sizes;
// route_align_small_kernel does the same for up to 32 tokens with a sort
// that has no loop over pairs.
#include "common.hpp"
#include "launch.hpp"
#include "route.hpp"

namespace moe {

constexpr int kSortThreads = 1024;
constexpr int kSortWaves = kSortThreads / 64;
constexpr int kMaxExperts = 1024;
constexpr int kFusedMaxPairs = 4096;

struct SortShared {
    unsigned long long masks[kSortWaves * kMaxExperts];  // or the bit matrix, its prefixes and the sorted rows
    int counts[kMaxExperts];
    int running[kMaxExperts];
    int offs[kMaxExperts + 1];
    int nvalid, nbits;
};
// 32-bit words of the mask table, which the token bit matrix path reuses.
constexpr int kBitWords = kSortWaves * kMaxExperts * 2;

// Eight ids per thread in flight (clamped index, no branch): one memory round
// trip per 8192 pairs instead of per 1024. f(p, t, e) for every pair p =
// t * topk + slot, e = -1 past P; the token index advances by the stride
// (no integer division per pair: at 15 pairs per thread the divisions alone
// took microseconds).
template <class F>
__device__ __forceinline__ void for_each_id(const int32_t* ids, int P, int topk, int tid, F&& f) {
    const int dq = kSortThreads / topk, dr = kSortThreads % topk;
    int t = tid / topk, r = tid % topk;
    for (int base = 0; base < P; base += 8 * kSortThreads) {
        int ev[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int p = base + u * kSortThreads + tid;
            ev[u] = ids[p < P ? p : P - 1];
            if (p >= P) ev[u] = -1;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            f(base + u * kSortThreads + tid, t, ev[u]);
            t += dq;
            r += dr;
            if (r >= topk) {
                r -= topk;
                ++t;
            }
        }
    }
}

// ids: global or LDS (generic pointer).
// Inlined into each kernel, so that the LDS tables are addressed as LDS (a
// called function saw generic pointers: flat instructions, and the old
// tiled pass took 29 us at 15,360 pairs).
__device__ __forceinline__ void align_sort_body(SortShared& sh, const int32_t* ids, int P, int topk, int E,
                                                int bm, int64_t cap, int32_t* __restrict__ sorted_ids,
                                                int32_t* __restrict__ block_expert,
                                                int32_t* __restrict__ expert_offsets,
                                                int32_t* __restrict__ num_post_pad) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    // Token bit matrix: row e (W words) holds bit t for token t = p / topk;
    // then the rows' prefixes and the sorted rows themselves, written to
    // LDS and copied out in order (scattered 4-byte stores from one CU took
    // half of the pass at 15,360 pairs). The pairs' ids stay in registers
    // (kFastIds per thread) from one round trip to the placement.
    // Rows are RS words apart, RS odd, so the words of one token column in
    // different rows fall in different LDS banks (a stride of 32 words put
    // every row's word in one bank: the atomics of a wave serialised).
    // The sorted rows sit at r + r / 32 (segment starts are multiples of the
    // block, so unpadded their stores would fall in two banks).
    constexpr int kFastIds = 16;
    const int W = (P / topk + 31) / 32, RS = W | 1;
    bool fast = P <= kFastIds * kSortThreads && 2 * (int64_t)E * RS + cap + cap / 32 + 1 <= kBitWords;
    uint32_t* const bits = (uint32_t*)sh.masks;
    uint32_t* const pre = bits + E * RS;
    int32_t* const srt = (int32_t*)(pre + E * RS);

    for (int e = tid; e < E; e += kSortThreads) {
        sh.counts[e] = 0;
        sh.running[e] = 0;
    }
    if (tid == 0) sh.nvalid = sh.nbits = 0;
    if (fast) {
        for (int i = tid; i < E * RS; i += kSortThreads) bits[i] = 0u;
        for (int i = tid; i < (int)(cap + cap / 32 + 1); i += kSortThreads) srt[i] = P;
    }
    // Pair k of this thread: p = k * kSortThreads + tid, token tv[k].
    int ev[kFastIds], tv[kFastIds];
    if (fast) {
        const int dq = kSortThreads / topk, dr = kSortThreads % topk;
        int t = tid / topk, r = tid % topk;
#pragma unroll
        for (int k = 0; k < kFastIds; ++k) {
            const int p = k * kSortThreads + tid;
            ev[k] = p < P ? ids[p] : -1;
            tv[k] = t;
            t += dq;
            r += dr;
            if (r >= topk) {
                r -= topk;
                ++t;
            }
        }
    }
    __syncthreads();
    if (fast) {
        // Bits only (no count atomics, no returned values): a token naming an
        // expert twice sets one bit for two pairs, which the totals below
        // detect.
        int nv = 0;
#pragma unroll
        for (int k = 0; k < kFastIds; ++k) {
            const int e = ev[k], t = tv[k];
            if ((unsigned)e < (unsigned)E) {
                atomicOr(&bits[e * RS + (t >> 5)], 1u << (t & 31));
                ++nv;
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) nv += __shfl_xor(nv, off);
        if (lane == 0) atomicAdd(&sh.nvalid, nv);
        __syncthreads();
        // Row prefixes: a thread per row, eight words read at a time.
        for (int e = tid; e < E; e += kSortThreads) {
            int run = 0;
            for (int w0 = 0; w0 < W; w0 += 8) {
                uint32_t v[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) v[k] = w0 + k < W ? bits[e * RS + w0 + k] : 0u;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    if (w0 + k < W) pre[e * RS + w0 + k] = run;
                    run += __popc(v[k]);
                }
            }
            sh.counts[e] = run;
            atomicAdd(&sh.nbits, run);
        }
        __syncthreads();
        fast = sh.nbits == sh.nvalid;
        if (!fast) {
            for (int e = tid; e < E; e += kSortThreads) sh.counts[e] = 0;
            __syncthreads();
        }
    }
    if (!fast) {
        for_each_id(ids, P, topk, tid, [&](int, int, int e) {
            if ((unsigned)e < (unsigned)E) atomicAdd(&sh.counts[e], 1);
        });
        __syncthreads();
    }

    // Exclusive scan of the padded segment lengths (wave 0, 64 at a time).
    if (wv == 0) {
        int carry = 0;
        for (int base = 0; base < E; base += 64) {
            const int e = base + lane;
            const int c = e < E ? sh.counts[e] : 0;
            const int padded = (c + bm - 1) / bm * bm;
            const int incl = wave_incl_scan(padded);
            if (e < E) sh.offs[e] = carry + incl - padded;
            carry += __builtin_amdgcn_readlane(incl, 63);
        }
        if (lane == 0) sh.offs[E] = carry;
    }
    __syncthreads();

    const int total = sh.offs[E];
    for (int e = tid; e <= E; e += kSortThreads) expert_offsets[e] = sh.offs[e];
    if (tid == 0) num_post_pad[0] = total;

    // Block -> expert map, padding rows of every segment and the unused
    // tail (the padding is already in the LDS rows on the bit matrix path).
    for (int e = wv; e < E; e += kSortWaves) {
        const int start = sh.offs[e], end = sh.offs[e + 1], c = sh.counts[e];
        if (!fast)
            for (int r = start + c + lane; r < end; r += 64) sorted_ids[r] = P;
        for (int b = start / bm + lane; b < end / bm; b += 64) block_expert[b] = e;
    }
    if (!fast)
        for (int64_t r = total + tid; r < cap; r += kSortThreads) sorted_ids[r] = P;
    for (int64_t b = total / bm + tid; b < cap / bm; b += kSortThreads) block_expert[b] = -1;

    if (fast) {
        // Pair p of token t and expert e ranks after the tokens before t
        // that chose e: its row's prefix plus the set bits below t.
#pragma unroll
        for (int k = 0; k < kFastIds; ++k) {
            const int e = ev[k], t = tv[k];
            if ((unsigned)e < (unsigned)E) {
                const int w = e * RS + (t >> 5);
                const int r = sh.offs[e] + pre[w] + __popc(bits[w] & ((1u << (t & 31)) - 1u));
                srt[r + (r >> 5)] = k * kSortThreads + tid;
            }
        }
        __syncthreads();
        for (int r = tid; r < (int)cap; r += kSortThreads) sorted_ids[r] = srt[r + (r >> 5)];
        return;
    }

    // Stable scatter, 1024 pairs per tile; the next tile's id is loaded
    // while this one is placed.
    int e_next = P > 0 ? ids[tid < P ? tid : P - 1] : -1;
    for (int base = 0; base < P; base += kSortThreads) {
        const int p = base + tid;
        const int e = p < P ? e_next : -1;
        const int pn = p + kSortThreads;
        e_next = pn < P ? ids[pn] : -1;
        for (int i = tid; i < kSortWaves * E; i += kSortThreads) sh.masks[i] = 0ull;
        __syncthreads();
        const bool valid = (unsigned)e < (unsigned)E;
        if (valid) atomicOr(&sh.masks[wv * E + e], 1ull << lane);
        __syncthreads();
        if (valid) {
            int rank = sh.running[e];
            for (int v = 0; v < wv; ++v) rank += __popcll(sh.masks[v * E + e]);
            rank += __popcll(sh.masks[wv * E + e] & ((1ull << lane) - 1ull));
            sorted_ids[sh.offs[e] + rank] = p;
        }
        __syncthreads();
        for (int ee = tid; ee < E; ee += kSortThreads) {
            int s = 0;
            for (int v = 0; v < kSortWaves; ++v) s += __popcll(sh.masks[v * E + ee]);
            sh.running[ee] += s;
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(kSortThreads) void align_sort_kernel(
    const int32_t* __restrict__ ids, int P, int topk, int E, int bm, int64_t cap,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ num_post_pad) {
    __shared__ SortShared sh;
    align_sort_body(sh, ids, P, topk, E, bm, cap, sorted_ids, block_expert, expert_offsets, num_post_pad);
}

template <int VPL>
__global__ __launch_bounds__(kSortThreads) void route_align_kernel(
    const float* __restrict__ logits, int T, int E, int topk, int renorm, int bm, int64_t cap,
    int32_t* __restrict__ ids, float* __restrict__ weights, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ block_expert, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ num_post_pad) {
    __shared__ SortShared sh;
    __shared__ int32_t ids_lds[kFusedMaxPairs];
    const int wv = threadIdx.x >> 6;
    // The routing scratch aliases the sort's mask table, which is written only
    // after the barrier below.
    for (int t = wv; t < T; t += kSortWaves)
        route_token<VPL>(logits + (int64_t)t * E, E, topk, renorm, ids + (int64_t)t * topk,
                         weights + (int64_t)t * topk, ids_lds + t * topk,
                         reinterpret_cast<uint64_t*>(sh.masks) + wv * 128);
    __syncthreads();
    align_sort_body(sh, ids_lds, T * topk, topk, E, bm, cap, sorted_ids, block_expert, expert_offsets,
                    num_post_pad);
}

// Up to 32 tokens: NW waves route the tokens (a token per wave at a time)
// while the workgroup clears the LDS tables; then the sort has no loop over
// pairs. A token routes to an expert at most once, so an expert's pairs are
// a bitmask of tokens (LDS atomic OR): its count is a popcount and a pair's
// rank within the expert the popcount of the lower tokens (pairs of one
// expert are in token order, which is pair order). Padded segment starts
// come from one wave scan over the experts (lane l owns experts VPL*l ..);
// sorted_ids and block_expert are assembled in LDS and copied out with
// coalesced stores. Same outputs as align_sort_body.
constexpr int kSmallTokens = 32;        // token bitmasks are 32-bit

constexpr int kSmallPairs = 512;
constexpr int64_t kSmallCapMax = 4096;  // e.g. 480 pairs of 112 experts at block_m 32

template <int VPL, int NW>
__global__ __launch_bounds__(NW * 64) void route_align_small_kernel(
    const float* __restrict__ logits, int T, int E, int topk, int renorm, int bm, int64_t cap,
    int32_t* __restrict__ ids, float* __restrict__ weights, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ block_expert, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ num_post_pad) {
    constexpr int NT = NW * 64;
    __shared__ int32_t ids_lds[kSmallPairs];
    __shared__ uint32_t tokens[kMaxExperts];
    __shared__ int32_t start[kMaxExperts];
    __shared__ int32_t srt[kSmallCapMax];
    __shared__ int32_t blk[kSmallCapMax / 16];
    __shared__ uint64_t rk[NW][64 * VPL <= 128 ? 64 * VPL : 1];  // routing scratch per wave
    const int tid = threadIdx.x;
    const int wv = tid >> 6;
    const int lane = tid & 63;
    const int P = T * topk;
    const int ncap = (int)cap, nblk = (int)(cap / bm);
    for (int i = tid; i < E; i += NT) tokens[i] = 0u;
    for (int i = tid; i < ncap; i += NT) srt[i] = P;
    for (int i = tid; i < nblk; i += NT) blk[i] = -1;
    for (int t = wv; t < T; t += NW)
        route_token<VPL>(logits + (int64_t)t * E, E, topk, renorm, ids + (int64_t)t * topk,
                         weights + (int64_t)t * topk, ids_lds + t * topk, rk[wv]);
    __syncthreads();
    for (int p = tid; p < P; p += NT) {
        const int e = ids_lds[p];
        if ((unsigned)e < (unsigned)E) atomicOr(&tokens[e], 1u << (p / topk));
    }
    __syncthreads();
    if (wv == 0) {
        // Padded lengths of this lane's experts and their exclusive prefix.
        int pad[VPL], local = 0;
#pragma unroll
        for (int c = 0; c < VPL; ++c) {
            const int x = VPL * lane + c;
            const int len = x < E ? __popc(tokens[x]) : 0;
            pad[c] = (len + bm - 1) & -bm;  // block_m is a power of two
            local += pad[c];
        }
        const int incl = wave_incl_scan(local);
        const int total = __builtin_amdgcn_readlane(incl, 63);
        const int lgbm = __builtin_ctz((unsigned)bm);
        int base = incl - local;
#pragma unroll
        for (int c = 0; c < VPL; ++c) {
            const int x = VPL * lane + c;
            if (x < E) {
                expert_offsets[x] = base;
                start[x] = base;
                for (int b = base >> lgbm; b < (base + pad[c]) >> lgbm; ++b) blk[b] = x;
            }
            base += pad[c];
        }
        if (lane == 0) {
            expert_offsets[E] = total;
            num_post_pad[0] = total;
        }
    }
    __syncthreads();
    for (int p = tid; p < P; p += NT) {
        const int e = ids_lds[p];
        const int t = p / topk;
        if ((unsigned)e < (unsigned)E) srt[start[e] + __popc(tokens[e] & ((1u << t) - 1u))] = p;
    }
    __syncthreads();
    for (int i = tid; i < ncap; i += NT) sorted_ids[i] = srt[i];
    for (int i = tid; i < nblk; i += NT) block_expert[i] = blk[i];
}

hipError_t launch_align_sort(const int32_t* ids, int P, int topk, int E, int bm, int64_t cap,
                             int32_t* sorted_ids, int32_t* block_expert, int32_t* expert_offsets,
                             int32_t* num_post_pad, hipStream_t s) {
    hipLaunchKernelGGL(align_sort_kernel, dim3(1), dim3(kSortThreads), 0, s, ids, P, topk, E, bm, cap,
                       sorted_ids, block_expert, expert_offsets, num_post_pad);
    return hipGetLastError();
}

bool route_align_fusable(int T, int E, int topk) {
    return T <= 64 && (int64_t)T * topk <= kFusedMaxPairs && E <= kMaxExperts;
}

hipError_t launch_route_align(const float* logits, int T, int E, int topk, int renorm, int bm,
                              int64_t cap, int32_t* ids, float* weights, int32_t* sorted_ids,
                              int32_t* block_expert, int32_t* expert_offsets, int32_t* num_post_pad,
                              hipStream_t s) {
    if (route_one_token_eligible(T, E, topk) && cap == (int64_t)topk * bm)
        return launch_route_one_token(logits, E, topk, renorm, bm, ids, weights, sorted_ids, block_expert,
                                      expert_offsets, num_post_pad, s);
    const dim3 grid(1), block(kSortThreads);
    const int vpl = (E + 63) / 64;
    const bool small = T <= kSmallTokens && T * topk <= kSmallPairs && cap <= kSmallCapMax;
#define MOE_LAUNCH_RA(V)                                                                                   \
    do {                                                                                                   \
        if (small && T <= 4)                                                                               \
            hipLaunchKernelGGL((route_align_small_kernel<V, 4>), dim3(1), dim3(256), 0, s, logits, T, E,   \
                               topk, renorm, bm, cap, ids, weights, sorted_ids, block_expert,             \
                               expert_offsets, num_post_pad);                                              \
        else if (small)                                                                                    \
            hipLaunchKernelGGL((route_align_small_kernel<V, 16>), dim3(1), dim3(1024), 0, s, logits, T, E, \
                               topk, renorm, bm, cap, ids, weights, sorted_ids, block_expert,             \
                               expert_offsets, num_post_pad);                                              \
        else                                                                                               \
            hipLaunchKernelGGL(route_align_kernel<V>, grid, block, 0, s, logits, T, E, topk, renorm, bm,   \
                               cap, ids, weights, sorted_ids, block_expert, expert_offsets, num_post_pad); \
    } while (0)
    if (vpl <= 1) MOE_LAUNCH_RA(1);
    else if (vpl <= 2) MOE_LAUNCH_RA(2);
    else if (vpl <= 4) MOE_LAUNCH_RA(4);
    else if (vpl <= 8) MOE_LAUNCH_RA(8);
    else MOE_LAUNCH_RA(16);
#undef MOE_LAUNCH_RA
    return hipGetLastError();
}

}  // namespace moe

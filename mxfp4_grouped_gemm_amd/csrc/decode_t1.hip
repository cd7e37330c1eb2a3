// The layer for one token (decode, T = 1), router logits in (the in-kernel
// routing of apply_monolithic on the vLLM mxfp4 API page): three launches
// instead of four.
//
// With one token every chosen expert holds exactly one (token, slot) pair,
// so the grouping that align/sort does for larger batches is fixed by the
// routing itself: slot j is its expert's only row, and h and y are indexed
// by slot. route_gate_up_t1_kernel is the GEMV gate_up of gemm_gemv.hip (a
// wave per (slot, column pair), weights decoded in registers, SwiGLU in the
// epilogue) with the routing folded in: a persistent grid (one round of
// resident workgroups) where every workgroup first routes the token itself
// -- the ranking split over its 4 waves -- and then walks its units; the
// token's activation row is loaded once per wave. Workgroup 0 also writes
// the routing and the align/sort arrays for the caller. The block-major down
// GEMV and the combine kernel follow, as on the general path.
//
// Measured at H = 3584, I = 3072, E = 112, topk = 15 (8 rotating weight
// sets): route + align 5.7 us and gate_up 29.7 us as two launches become one
// 30.9 us launch. Two ways of folding the combine into the down GEMV were
// slower than the down kernel and the combine kernel together (22.0 us):
// a token-major workgroup per 4 output rows whose waves take the slots in
// turn (23.5 us: each wave runs four slots one after another), and a
// persistent 16-wave workgroup per CU with one slot per wave, its h row in
// registers and a 4-deep ring of 2-row groups (24.8 us). Measured and not
// kept either: this gate_up with the next unit's weights prefetched before
// the current one is decoded (123 VGPRs, 4 waves per SIMD: 32.5 against
// 31.4 us), and a persistent down GEMV reading the slots' experts once per
// wave (23.4 us for down + combine, 25.8 with prefetch, against 22.1).
#include "gemv.hpp"
#include "route.hpp"

namespace moe {

constexpr int kT1Waves = 4;

// Caller-visible routing and align/sort outputs written by workgroup 0.
struct T1Outputs {
    int32_t* topk_ids;        // [topk]
    float* topk_weights;      // [topk]
    int32_t* sorted_ids;      // [topk * bm]
    int32_t* block_expert;    // [topk]
    int32_t* expert_offsets;  // [E + 1]
    int32_t* num_post_pad;    // [1]
    int bm;
};

// Workgroup 0, wave 0: the routing and the align/sort arrays of one token
// (each chosen expert one block holding the pair of its slot; blocks in
// ascending expert order), the same values moe_route_align produces.
__device__ __forceinline__ void t1_write_outputs(const MoeGemmArgs& a, const int32_t* sid, const float* swt,
                                                 const T1Outputs& o, int32_t* blk_e, int32_t* blk_j,
                                                 int lane) {
    const int E = a.E, topk = a.topk, bm = o.bm;
    if (lane < topk) {
        o.topk_ids[lane] = sid[lane];
        o.topk_weights[lane] = swt[lane];
    }
    // Slot of each of this lane's experts (lane, lane + 64), -1 if not chosen.
    int slot[2] = {-1, -1};
    for (int j = 0; j < topk; ++j) {
        const int e = sid[j];
        if (e == lane) slot[0] = j;
        if (e == lane + 64) slot[1] = j;
    }
    const uint64_t m0 = __ballot(slot[0] >= 0), m1 = __ballot(slot[1] >= 0);
    const uint64_t below = (1ull << lane) - 1ull;
    const int before0 = __popcll(m0 & below);
    const int before1 = __popcll(m0) + __popcll(m1 & below);
    if (slot[0] >= 0) {
        blk_e[before0] = lane;
        blk_j[before0] = slot[0];
    }
    if (slot[1] >= 0) {
        blk_e[before1] = lane + 64;
        blk_j[before1] = slot[1];
    }
    if (lane < E) o.expert_offsets[lane] = before0 * bm;
    if (lane + 64 < E) o.expert_offsets[lane + 64] = before1 * bm;
    if (lane == 0) {
        o.expert_offsets[E] = topk * bm;
        *o.num_post_pad = topk * bm;
    }
    wave_lds_sync();
    if (lane < topk) o.block_expert[lane] = blk_e[lane];
    for (int i = lane; i < topk * bm; i += 64) o.sorted_ids[i] = (i % bm == 0) ? blk_j[i / bm] : topk;
}

// Routes the token for a workgroup (E <= 128, topk <= 64), in wave 0 alone:
// the selection and ranks of route_token<2> (a candidate threshold from one
// round of guesses, then each candidate ranked against the candidates in
// LDS by (key, ~index)) and the same softmax terms summed in the same order,
// so ids and weights are bit-identical to it. Leaves sid[rank] / swt[rank]
// in LDS for rank < topk. Every thread of the workgroup must call it.
// Per-workgroup clocks: routing 1.8-2.6 us (median over the launch) against
// 2.4-2.8 us for every expert counted against every key with the count
// split over the four waves (VALU-bound with six workgroups per CU routing
// at once), and 2.3-3.1 us with radix rounds in place of the guesses.
struct T1RouteLds {
    uint64_t key[128];
};

__device__ __forceinline__ void t1_route(const float* __restrict__ row, int E, int topk, int renorm,
                                         T1RouteLds& r, int32_t* sid, float* swt, int wave, int lane) {
    if (wave == 0) {
        float val[2];
        uint32_t key[2], kv[2];
        bool ok[2];
        // Both logits of the lane in one round trip (branch-free loads).
        const rsrc_t rl = make_rsrc(row, (uint32_t)E * 4u);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int e = lane + 64 * i;
            val[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, e < E ? 4u * (uint32_t)e : kOob, 0, 0));
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            ok[i] = lane + 64 * i < E;
            key[i] = route_key(val[i]);
            kv[i] = ok[i] ? key[i] : 0u;
        }
        int n = E;
        uint32_t kmax;
        const uint32_t thr = key_guess_threshold<2>(kv, ok, E, topk, topk + 16, n, kmax);
        // Candidates (key >= thr) compacted in index order; zero entries up
        // to a multiple of 4 (base <= E <= 128).
        const uint64_t below_me = (1ull << lane) - 1ull;
        uint64_t k64[2];
        bool cand[2];
        int base = 0;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            k64[i] = ((uint64_t)key[i] << 32) | (uint64_t)~(uint32_t)(lane + 64 * i);
            cand[i] = ok[i] && key[i] >= thr;
            const uint64_t m = __ballot(cand[i]);
            if (cand[i]) r.key[base + __popcll(m & below_me)] = k64[i];
            base += __popcll(m);
        }
        const int n4 = (base + 3) & ~3;
        if (base + lane < n4) r.key[base + lane] = 0ull;
        wave_lds_sync();
        int rank[2] = {0, 0};
        for (int j = 0; j < n4; j += 4) {
            const uint64_t kj0 = r.key[j], kj1 = r.key[j + 1], kj2 = r.key[j + 2], kj3 = r.key[j + 3];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                rank[i] += (kj0 > k64[i] ? 1 : 0) + (kj1 > k64[i] ? 1 : 0) + (kj2 > k64[i] ? 1 : 0) +
                           (kj3 > k64[i] ? 1 : 0);
        }
        bool sel[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) sel[i] = cand[i] && rank[i] < topk;
        const float lmax = route_key_value(kmax);
        float ex[2];
        float psum = 0.0f;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            ex[i] = ok[i] ? expf(val[i] - lmax) : 0.0f;
            if (renorm ? sel[i] : ok[i]) psum += ex[i];
        }
        psum = wave_sum_butterfly(psum);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            if (sel[i]) {
                sid[rank[i]] = lane + 64 * i;
                swt[rank[i]] = ex[i] / psum;
            }
        }
    }
    __syncthreads();
}

// Persistent: gridDim.x workgroups (at most one round of resident ones)
// route the token once each, then walk the units u = (slot u / (I / 2),
// column pair u % (I / 2)) with a stride of the grid's waves.
template <int NCH, bool EPI>
__global__ __launch_bounds__(kT1Waves * 64) __attribute__((amdgpu_waves_per_eu(6)))
void route_gate_up_t1_kernel(MoeGemmArgs a, const float* __restrict__ logits, int renorm, T1Outputs o) {
    __shared__ __attribute__((aligned(16))) uint8_t lds_scale[kT1Waves][4 * 64 * NCH];
    __shared__ T1RouteLds rl;
    __shared__ int32_t sid[64], blk_e[64], blk_j[64];
    __shared__ float swt[64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    t1_route(logits, a.E, a.topk, renorm, rl, sid, swt, wave, lane);
    if (blockIdx.x == 0 && wave == 0) t1_write_outputs(a, sid, swt, o, blk_e, blk_j, lane);
    const int upb = a.I / 2;
    const int units = a.topk * upb;
    // The token's activation row, the same for every unit: loaded once.
    const int H = a.H, I = a.I, nblk = H / 32;
    u32x4 x[NCH][4];
    issue_x<NCH>(x, make_rsrc(a.x, (uint32_t)(H * 2)), 0u, nblk, lane);
    for (int u = (int)blockIdx.x * kT1Waves + wave; u < units; u += (int)gridDim.x * kT1Waves) {
        const int j = __builtin_amdgcn_readfirstlane(u / upb);
        const int e = __builtin_amdgcn_readfirstlane(sid[j]);
        const int i0 = (u % upb) * 2;
        const int64_t slab_rows = 2 * (int64_t)I;
        const rsrc_t rw = make_rsrc(a.w13 + e * slab_rows * (H / 2), (uint32_t)(slab_rows * (H / 2)));
        const rsrc_t rs = make_rsrc((const uint8_t*)a.w13_scale + e * slab_rows * nblk, (uint32_t)(slab_rows * nblk));
        GemvWeights<NCH> W;
        W.issue(rw, rs, GemvRows{i0, 2, I + i0}, nblk, lane);
        W.stage_scales(lds_scale[wave], nblk, lane);
        wave_lds_sync();
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        gemv_dot<NCH>(W, lds_scale[wave], x, nblk, lane, acc);
        float v[4] = {acc[0], acc[2], acc[1], acc[3]};
        float gs = reduce4(v), us = gs;
        permlane32_swap(gs, us);
        if ((lane & 15) == 0 && lane < 32) {
            if constexpr (EPI) {
                GluTerms glu;
                glu.load(a, e, i0 + (lane >> 4));
                glu.apply(gs, us);
            }
            a.h[(int64_t)j * I + i0 + (lane >> 4)] = f32_to_bf16_bits(swiglu(gs, us));
        }
        wave_lds_sync();  // the next unit overwrites this wave's scale bytes
    }
}

bool t1_eligible(const MoeGemmArgs& a) {
    return a.T == 1 && a.fmt == kFmtMxfp4 && a.E <= 128 && a.topk <= 64 && a.H % 256 == 0 &&
           a.I % 128 == 0 && a.H <= 4096 && a.I <= 4096;
}

hipError_t launch_t1_layer(const MoeGemmArgs& a, const float* logits, int renorm, int32_t* topk_ids,
                           float* topk_weights, int32_t* sorted_ids, int32_t* block_expert,
                           int32_t* expert_offsets, int32_t* num_post_pad, unsigned stages, hipStream_t s) {
    const T1Outputs o{topk_ids, topk_weights, sorted_ids, block_expert, expert_offsets, num_post_pad, a.bm};
    MoeGemmArgs b = a;
    b.topk_ids = topk_ids;
    b.topk_weights = topk_weights;
    if (stages & 1u) {
        static int cus = 0;  // compute units: the persistent grid holds one round of workgroups
        if (!cus) {
            int dev = 0, n = 0;
            cus = (hipGetDevice(&dev) == hipSuccess &&
                   hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
                      ? n
                      : 256;
        }
        // One round of resident workgroups (6 waves per SIMD: 24 per CU).
        constexpr int kPerCu = 24 / kT1Waves;
        const int64_t wgs = ((int64_t)a.topk * (a.I / 2) + kT1Waves - 1) / kT1Waves;
        const dim3 grid((unsigned)(wgs < kPerCu * cus ? wgs : kPerCu * cus)), block(kT1Waves * 64);
        const int nch = (a.H / 32 + 63) / 64;
        const bool epi = a.w13_bias || a.swiglu_limit > 0.0f;
#define MOE_T1A(NC, EP) hipLaunchKernelGGL((route_gate_up_t1_kernel<NC, EP>), grid, block, 0, s, b, logits, renorm, o)
        if (nch == 1) {
            if (epi) MOE_T1A(1, true);
            else MOE_T1A(1, false);
        } else {
            if (epi) MOE_T1A(2, true);
            else MOE_T1A(2, false);
        }
#undef MOE_T1A
    }
    if (stages & 2u) {
        // Block-major down GEMV (h and y by slot), then the combine kernel.
        const hipError_t err = launch_gemv_stage(b, 2, s);
        if (err != hipSuccess) return err;
        return launch_combine(b.y, topk_ids, topk_weights, b.w2_bias, b.T, b.H, b.E, b.topk, b.out, s);
    }
    return hipGetLastError();
}

}  // namespace moe

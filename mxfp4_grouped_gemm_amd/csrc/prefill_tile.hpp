// Prefill-sized grouped GEMMs (bf16 MFMA over MXFP4 or int4-g32 weights):
// the tile constants, the LDS layouts, the per-tile main loop pf_tile and the
// single-wave kernel template. gemm_prefill.hip holds the super-block pass,
// the 4-wave kernels, the MXFP4 single-wave kernels and the launcher;
// gemm_prefill_int4.hip the int4 single-wave kernels (built with MFMA results
// in VGPRs, see there).
//
// At prefill every expert holds on the order of a hundred token rows, so the
// layer is a dense contraction and runs on v_mfma_f32_32x32x16_bf16. The
// pages' two-stage MoE GEMM (the MXFP4-to-int4 pull request, Test plan) is
// kept: stage 1 = gate_up GEMM + SwiGLU into h, stage 2 = down GEMM into y by
// pair index, then the weighted combine.
//
// Work unit. The align/sort pads each expert segment to 32-row blocks. A
// small kernel cuts every run of blocks of one expert into super-blocks of
// at most 8 blocks (256 rows). A workgroup owns (super-block, N tile): its 4
// waves share the super-block's activation rows through LDS, each wave owns
// two 32-column weight blocks and all of the super-block's 32-row blocks, so
// every decoded weight fragment feeds up to 8 MFMAs and the weight bytes of
// an (expert, N tile) are read once from HBM.
//  * Activations: 64-element K chunks; global loads run four chunks ahead
//    in registers, then go to one of three LDS buffers (one barrier per
//    chunk, and the next chunk's first MFMA operands are read before it). A row is 128 bytes and its 16-byte pieces are XOR-swizzled by
//    (row/2)%8, so a 16-lane group of MFMA operand reads or of stores touches
//    all 64 banks once. (Loads straight into LDS were tried: the compiler
//    then waits for every outstanding load before each LDS read.)
//  * Weights: lane (n = l%32, half = l/32) takes 16 bytes = one MX block of
//    weight row n per chunk; the K order inside a chunk is permuted (half h
//    covers elements 32h..32h+31 as four 8-element MFMA k-steps), and the
//    activation operand reads use the same order, so the sums are unchanged.
//    Four chunks of weights are in flight in a register ring; the e8m0 byte
//    of each block rides with it. Decoding uses the scaled fp4 -> bf16
//    converts (exact).
//  * The super-block's row count (1..8 blocks) selects a specialisation of
//    the main loop, so padding beyond the last 32-row block costs nothing.
// Workgroups of one super-block sit on one XCD (consecutive workgroup ids go
// round-robin over the 8 XCDs), so its activation rows stay in that L2.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kPfThreads = 256;
constexpr int kPfBlockRows = 32;   // align/sort block size this path expects
constexpr int kPfMaxBlocks = 8;    // 32-row blocks per super-block (prefill sizes)
constexpr int kPfMaxBlocksSmall = 2;  // the same when experts hold few rows
constexpr int kPfChunk = 64;       // K elements per pipeline step
constexpr int kPfRowBytes = kPfChunk * 2;
constexpr int kPfABufs = 3;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Weights are staged per wave, four chunks (256 K elements) at a time: the
// wave's 64 weight rows x 128 bytes of codes (swizzled like the activation
// tile) and 64 rows x 8 e8m0 bytes.
constexpr int kPfWRows = 64;
constexpr int kPfStage = 4;  // chunks per weight stage
// Single-wave tiles up to this many tokens (at most one 32-row block per
// expert needs T <= 32). For MXFP4 gate_up, from 14 tokens on the blocks
// fill up and the 4-wave tiles, which share each activation chunk between
// four waves, are faster (1-2 % at 14-16 tokens); int4 gate_up and both
// formats' down stay on the single-wave tiles up to 32 (the 4-wave int4
// tiles split every weight into two MFMAs: 548 against 305 us at 24 tokens).
constexpr int kPfDirectMaxTokens1 = 13;
constexpr int kPfDirectMaxTokens1Int4 = 32;
constexpr int kPfDirectMaxTokens2 = 32;
template <int NBMAX>
struct __attribute__((aligned(16))) PfShared {
    uint8_t a[kPfABufs][NBMAX * kPfBlockRows * kPfRowBytes];
    uint8_t b[4][kPfWRows * 128];
    uint8_t bs[4][kPfWRows * 16];
    int32_t rows[NBMAX * kPfBlockRows];  // sorted_ids of the super-block
};

// Single-wave workgroups (one 32-row block each): the wave's weight stage
// and the block's sorted ids only; activations go straight to registers.
struct __attribute__((aligned(16))) PfSharedDirect {
    uint8_t b[1][kPfWRows * 128];
    uint8_t bs[1][kPfWRows * 16];
    int32_t rows[kPfBlockRows];
};

// The shared activation buffer `buf` (none in single-wave workgroups).
template <int NBMAX>
__device__ __forceinline__ uint8_t* a_buf(PfShared<NBMAX>& sh, int buf) { return sh.a[buf]; }
__device__ __forceinline__ uint8_t* a_buf(PfSharedDirect&, int) { return nullptr; }

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

}  // namespace

// ---------------------------------------------------------------------------
// Main loop of one (super-block, N tile), NB 32-row blocks.
//   STAGE 1: A = x rows gathered by pair / topk, K = H; wave w owns gate
//            columns n0+32w.. and the matching up columns; epilogue SwiGLU
//            -> h[sorted row] (bf16).
//   STAGE 2: A = h rows (contiguous), K = I; wave w owns columns
//            n0+64w.. +64 of w2; epilogue y[pair] (fp32).
//   DIRECT: a single-wave workgroup and one 32-row block (NB = 1): the wave
//            loads its MFMA activation operands straight from global memory
//            (L2) into a ring of registers, so there is no shared tile and
//            no workgroup barrier; the wave streams its weights on its own.
// EPI: compile the optional expert-bias / clamp epilogue of stage 1 (kernels
// launched without bias or clamp are built without it).
template <int STAGE, int FMT, int NB, bool DIRECT, class SH, bool EPI = true>
__device__ __forceinline__ void pf_tile(const MoeGemmArgs& a, SH& sh, int e, int row0, int n0) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int P = a.T * a.topk;
    const int K = STAGE == 1 ? a.H : a.I;
    const int nchunks = K / kPfChunk;
    constexpr int SB = FMT == kFmtMxfp4 ? 1 : 2;  // bytes per group scale
    // int4 in single-wave tiles: every MFMA k-step stays inside one 32-group
    // (k-steps 0, 1 of a chunk take its first group, 2, 3 the second); the
    // codes enter as code + 136, the group's sums start from -136 * sum(x)
    // and its scale is applied to the group's fp32 result (see the k-loop).
    constexpr bool GS = FMT == kFmtInt4g32 && DIRECT;

    // --- activations: thread t moves row 32i + t/8, logical piece t%8 of
    // every 32-row block i; in LDS the piece sits at t%8 ^ ((row/2) % 8).
    const int arow = tid >> 3;
    const int apiece = tid & 7;
    const uint32_t lds_w = (uint32_t)arow * kPfRowBytes + (uint32_t)((apiece ^ ((arow >> 1) & 7)) << 4);
    const int half = lane >> 5;
    const int nl = lane & 31;
    rsrc_t ra;
    uint32_t aoff[NB];
    if constexpr (DIRECT) {
        // Lane (nl, half): row nl of the block, logical pieces 4*half.. of a
        // chunk (the operand order of the MFMA k-steps).
        static_assert(NB == 1, "direct tiles hold one block");
        const int p = sh.rows[nl];
        if (STAGE == 1) {
            ra = make_rsrc(a.x, (uint32_t)((int64_t)a.T * a.H * 2));
            aoff[0] = (p >= 0 && p < P) ? (uint32_t)(p / a.topk) * (uint32_t)(2 * a.H) + (GS ? 32u : 64u) * half : kOob;
        } else {
            ra = make_rsrc(a.h, (uint32_t)(a.cap * a.I * 2));
            aoff[0] = (p >= 0 && p < P) ? (uint32_t)(row0 + nl) * (uint32_t)(2 * a.I) + (GS ? 32u : 64u) * half : kOob;
        }
    } else if constexpr (STAGE == 1) {
        ra = make_rsrc(a.x, (uint32_t)((int64_t)a.T * a.H * 2));
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int p = sh.rows[32 * i + arow];
            aoff[i] = (p >= 0 && p < P) ? (uint32_t)(p / a.topk) * (uint32_t)(2 * a.H) + 16u * apiece : kOob;
        }
    } else {
        ra = make_rsrc(a.h, (uint32_t)(a.cap * a.I * 2));
#pragma unroll
        for (int i = 0; i < NB; ++i)
            aoff[i] = (uint32_t)(row0 + 32 * i + arow) * (uint32_t)(2 * a.I) + 16u * apiece;
    }

    // --- weights. Staging row r (0..63) of wave w: block r / 32 of the wave
    // (stage 1: gate columns n0+32w.., then the matching up rows; stage 2:
    // columns n0+64w..+64), row r % 32 of it.
    rsrc_t rw, rs;
    auto grow = [&](int r) -> uint32_t {
        if (STAGE == 1) return (uint32_t)((r < 32 ? 0 : a.I) + n0 + 32 * w + (r & 31));
        return (uint32_t)(n0 + 64 * w + r);
    };
    if (STAGE == 1) {
        const int64_t slab = 2 * (int64_t)a.I;
        rw = make_rsrc(a.w13 + (int64_t)e * slab * (a.H / 2), (uint32_t)(slab * (a.H / 2)));
        rs = make_rsrc((const uint8_t*)a.w13_scale + (int64_t)e * slab * (a.H / 32) * SB, (uint32_t)(slab * (a.H / 32) * SB));
    } else {
        rw = make_rsrc(a.w2 + (int64_t)e * a.H * (a.I / 2), (uint32_t)((int64_t)a.H * (a.I / 2)));
        rs = make_rsrc((const uint8_t*)a.w2_scale + (int64_t)e * a.H * (a.I / 32) * SB, (uint32_t)((int64_t)a.H * (a.I / 32) * SB));
    }
    // Stage loads: instruction j moves rows 8j..8j+7, eight lanes (128
    // contiguous bytes, one cache line) per row; the scale bytes of row
    // `lane` come with one 8-byte load.
    uint32_t boff[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) boff[j] = grow(8 * j + (lane >> 3)) * (uint32_t)(K / 2) + 16u * (lane & 7);
    const uint32_t soff = grow(lane) * (uint32_t)(K / 32 * SB);
    const int nstages = nchunks / kPfStage;
    // Register slots for weight stages in flight: two when the tile is
    // small (memory-bound decode batches: a stage round trip per four
    // chunks would bound the stream), else one.
    constexpr int BR = 1;
    u32x4 braw[BR][8];
    // the stage's 8 group scales of row `lane`: 8 e8m0 bytes or 8 bf16
    using svec = typename std::conditional<FMT == kFmtMxfp4, u32x2, u32x4>::type;
    constexpr int SVB = (int)sizeof(svec);
    svec sraw[BR];
    // The stage advance is a scalar offset; stages past the end (never
    // consumed) are not loaded (a uniform branch).
    auto issue_bstage = [&](int slot, int st) {
        if (st >= nstages) return;
#pragma unroll
        for (int j = 0; j < 8; ++j) braw[slot][j] = bld16snt(rw, boff[j], 128u * st);
        if constexpr (FMT == kFmtMxfp4)
            sraw[slot] = bld8s(rs, soff, 8u * st);
        else
            sraw[slot] = bld16s(rs, soff, 16u * st);
    };
    uint8_t* const wl = sh.b[w];
    uint8_t* const sl = sh.bs[w];
    auto store_bstage = [&](int slot) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int r = 8 * j + (lane >> 3);
            *(u32x4*)(wl + r * 128 + (((lane & 7) ^ ((r >> 1) & 7)) << 4)) = braw[slot][j];
        }
        *(svec*)(sl + lane * SVB) = sraw[slot];
    };
    // MFMA B operand of chunk j of the stage, block nb: row 32nb + nl,
    // logical piece 2j + half (16 bytes = one MX block of 32 codes).
    // GS: dwords 2*half, 2*half + 1 of both groups of chunk j (k-step s takes
    // dword s & 1 of group s >> 1).
    auto read_bchunk = [&](u32x4 (&dst)[2], int j) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const int r = 32 * nb + nl;
            if constexpr (GS) {
                const u32x2 g0 = *(const u32x2*)(wl + r * 128 + (((2 * j) ^ ((r >> 1) & 7)) << 4) + 8 * half);
                const u32x2 g1 = *(const u32x2*)(wl + r * 128 + (((2 * j + 1) ^ ((r >> 1) & 7)) << 4) + 8 * half);
                dst[nb] = u32x4{g0[0], g0[1], g1[0], g1[1]};
            } else {
                dst[nb] = *(const u32x4*)(wl + r * 128 + (((2 * j + half) ^ ((r >> 1) & 7)) << 4));
            }
        }
    };
    auto read_scales = [&](svec (&dst)[2]) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) dst[nb] = *(const svec*)(sl + (32 * nb + nl) * SVB);
    };
    // Scale of chunk j (group 2j + half of the stage): the e8m0 byte as the
    // fp4 converts' scale operand, or the bf16 int4 group scale as a float.
    auto scale_of = [&](const svec& w8, int j) -> float {
        if constexpr (FMT == kFmtMxfp4) {
            const uint32_t word = j < 2 ? w8[0] : w8[1];
            return e8m0_scale_operand((word >> (16 * (j & 1) + 8 * half)) & 0xffu);
        } else {
            return __uint_as_float(((w8[j] >> (16 * half)) & 0xffffu) << 16);
        }
    };
    // Decoded weight operand of one k-step: MXFP4 is exact in bf16; int4 is
    // an exact hi + lo pair (two MFMAs).
    struct Bop {
        bf16x8 hi, lo;
    };
    auto decode = [&](uint32_t d, float sc) -> Bop {
        Bop r;
        if constexpr (FMT == kFmtMxfp4) r.hi = mxfp4x8_to_bf16(d, sc);
        else if constexpr (GS) r.hi = int4x8_to_bf16_biased(d);
        else int4x8_to_bf16_hilo(d, sc, r.hi, r.lo);
        return r;
    };
    // GS: the bf16 group scale of weight block nb for k-step s of chunk u.
    auto gscale = [&](const svec& w8, int u, int s) -> float {
        return __uint_as_float(((w8[u] >> (16 * (s >> 1))) & 0xffffu) << 16);
    };

    // Activation ring: chunk k lives in slot k % DA from its load (DA chunks
    // before it is stored to LDS) to that store. Vector-memory counts retire
    // in order, so this depth is the latency budget of every load; it is as
    // deep as the registers allow. Chunks past the end are issued with
    // out-of-range offsets (zeros, no traffic).
    constexpr int DA = (NB >= 3 && NB <= 6 && FMT == kFmtMxfp4) ? 4 : 2;
    u32x4 ar[DA][NB];
    // Chunks past the end re-read the last one (never consumed); padding
    // rows carry kOob in the vector offset.
    auto issue_a = [&](int slot, int c) {
        const uint32_t so = (uint32_t)(kPfRowBytes * (c < nchunks ? c : nchunks - 1));
#pragma unroll
        for (int i = 0; i < NB; ++i) ar[slot][i] = bld16s(ra, aoff[i], so);
    };
    // DIRECT: chunk c's four k-step operands sit in ring slot c % DD from
    // their load (issued when chunk c - DD finished with the slot) to the
    // chunk's MFMAs. For int4 the ring holds a whole stage, so the oldest
    // activation load is never younger than the weight stage that the next
    // store waits for; for MXFP4 two chunks, which brings the kernel to 160
    // registers and three waves per SIMD (2-3 % faster at 16-32 tokens).
    constexpr int DD = FMT == kFmtMxfp4 ? 2 : 4;
    u32x4 ad[DIRECT ? DD : 1][4];
    auto issue_ad = [&](int slot, int c) {
        const uint32_t so = (uint32_t)(kPfRowBytes * (c < nchunks ? c : nchunks - 1));
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
            ad[slot][s4] = bld16s(ra, aoff[0] + (GS ? 64u * (s4 >> 1) + 16u * (s4 & 1) : 16u * s4), so);
    };
    auto store_a = [&](int slot, int buf) {
#pragma unroll
        for (int i = 0; i < NB; ++i)
            *(u32x4*)(a_buf(sh, buf) + 32 * i * kPfRowBytes + lds_w) = ar[slot][i];
    };
    // MFMA A operand from LDS: row 32i + nl, logical piece 4*half + s.
    const int sw = (nl >> 1) & 7;
    bf16x8 av[2][NB];
    auto read_a = [&](int dst, int buf, int s) {
        const uint8_t* base = a_buf(sh, buf) + nl * kPfRowBytes + (((4 * half + s) ^ sw) << 4);
#pragma unroll
        for (int i = 0; i < NB; ++i) av[dst][i] = *(const bf16x8*)(base + 32 * i * kPfRowBytes);
    };

    f32x16 acc[NB][2];
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
    // GS: one group's sums per weight block and its activation row sums x -136.
    f32x16 gacc[2], gsum;

    // Activations: three LDS buffers; at step c, chunk c is read from buffer
    // c%3, chunk c+1 already sits in buffer (c+1)%3 (so the first operands of
    // the next step are read before the step's barrier) and chunk c+2 is
    // stored into buffer (c+2)%3, the one chunk c-1 used.
    // Weights: stage t (chunks 4t..4t+3) is written to the wave's LDS in
    // chunk 4t-2, after the last read of stage t-1 (chunk 4t-1's operands,
    // read one chunk ahead); stage t+1 is then loaded into the registers.
    if constexpr (DIRECT) {
#pragma unroll
        for (int k = 0; k < DD; ++k) issue_ad(k, k);
        issue_bstage(0, 0);
        store_bstage(0);
#pragma unroll
        for (int t = 1; t <= BR; ++t) issue_bstage(t % BR, t);
        wave_lds_sync();
    } else {
        issue_a(0, 0);
        issue_a(1, 1);
        issue_bstage(0, 0);
        store_a(0, 0);
        store_a(1, 1);
        store_bstage(0);
#pragma unroll
        for (int t = 1; t <= BR; ++t) issue_bstage(t % BR, t);
#pragma unroll
        for (int k = 2; k < 2 + DA; ++k) issue_a(k % DA, k);
        __syncthreads();
    }
    // Small tiles (1-2 blocks) have too few MFMAs per k-step to cover an LDS
    // read between consecutive steps: they read a whole chunk's operands one
    // chunk ahead instead.
    constexpr bool CP = NB <= 2 && FMT == kFmtMxfp4 && !DIRECT;
    bf16x8 avc[4][NB], avn[4][NB];
    auto read_a_chunk = [&](bf16x8 (&dst)[4][NB], int buf) {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            const uint8_t* base = a_buf(sh, buf) + nl * kPfRowBytes + (((4 * half + s4) ^ sw) << 4);
#pragma unroll
            for (int i = 0; i < NB; ++i) dst[s4][i] = *(const bf16x8*)(base + 32 * i * kPfRowBytes);
        }
    };
    if (CP) read_a_chunk(avc, 0);
    else if (!DIRECT) read_a(0, 0, 0);
    u32x4 bcur[2], bnext[2];
    svec scur[2], snext[2];
    read_scales(scur);
    read_bchunk(bcur, 0);
    // Decoded weights of the current k-step; the next step's are decoded
    // while this step's MFMAs run.
    Bop b0 = decode(bcur[0][0], scale_of(scur[0], 0));
    Bop b1 = decode(bcur[1][0], scale_of(scur[1], 0));

    int buf = 0;  // chunk c's LDS buffer, c % 3
    // Unrolled over BR stages so every register slot index is a constant;
    // u4 = chunk within its stage.
    for (int c0 = 0; c0 < nchunks; c0 += kPfStage * BR) {
#pragma unroll
        for (int uu = 0; uu < kPfStage * BR; ++uu) {
            const int u = uu & 3;
            const int tslot = uu >> 2;  // this stage's index modulo BR
            const int c = c0 + uu;
            const int buf1 = buf == 2 ? 0 : buf + 1;
            const int buf2 = buf1 == 2 ? 0 : buf1 + 1;
            const float sc0 = scale_of(scur[0], u);
            const float sc1 = scale_of(scur[1], u);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                if (s == 0) {
                    // next chunk's weight operands (and, at the stage's last
                    // chunk, the next stage's scales)
                    if (u < 3) read_bchunk(bnext, u + 1);
                    else {
                        read_bchunk(bnext, 0);
                        read_scales(snext);
                    }
                    if (!DIRECT) {
                        store_a((u + 2) % DA, buf2);  // A(c+2)
                        issue_a((u + 2) % DA, c + 2 + DA);
                    }
                    if (u == 2) {  // next stage into LDS, its slot reloaded BR stages ahead
                        const int slot = (tslot + 1) % BR;
                        store_bstage(slot);
                        issue_bstage(slot, (c0 + 4 * tslot) / kPfStage + 1 + BR);
                    }
                    if (CP) read_a_chunk(avn, buf1);
                }
                // Operands of the next k-step (the next chunk's first at s = 3).
                Bop n0, n1;
                if (s < 3) {
                    if (!CP && !DIRECT) read_a((s + 1) & 1, buf, s + 1);
                    n0 = decode(bcur[0][s + 1], sc0);
                    n1 = decode(bcur[1][s + 1], sc1);
                } else {
                    if (!CP && !DIRECT) read_a(0, buf1, 0);
                    const svec* sn = u < 3 ? scur : snext;
                    n0 = decode(bnext[0][0], scale_of(sn[0], (u + 1) & 3));
                    n1 = decode(bnext[1][0], scale_of(sn[1], (u + 1) & 3));
                }
                if constexpr (GS) {
                    // Group s >> 1 of the chunk (k-steps s, s + 1). At the
                    // first k-step both activation operands of the group
                    // (already in registers) are summed against a constant
                    // -136 operand; that row sum, shared by both weight
                    // blocks, seeds the blocks' group accumulators, so after
                    // the two k-steps of codes + 136 they hold sum(x * code)
                    // (exact products, fp32 sums) and the group's scale is
                    // applied with one FMA per element.
                    const bf16x8 ai = perm_x_int4(__builtin_bit_cast(bf16x8, ad[u % DD][s]));
                    if ((s & 1) == 0) {
                        const bf16x8 ai1 = perm_x_int4(__builtin_bit_cast(bf16x8, ad[u % DD][s + 1]));
                        const bf16x8 m136 = __builtin_bit_cast(bf16x8, u32x4{0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u});
                        const f32x16 zero = {};
                        gsum = mfma32(ai, m136, zero);
                        gsum = mfma32(ai1, m136, gsum);
                        gacc[0] = mfma32(ai, b0.hi, gsum);
                        gacc[1] = mfma32(ai, b1.hi, gsum);
                    } else {
                        gacc[0] = mfma32(ai, b0.hi, gacc[0]);
                        gacc[1] = mfma32(ai, b1.hi, gacc[1]);
                        const float g0 = gscale(scur[0], u, s), g1 = gscale(scur[1], u, s);
#pragma unroll
                        for (int q = 0; q < 16; ++q) {
                            acc[0][0][q] = fmaf(gacc[0][q], g0, acc[0][0][q]);
                            acc[0][1][q] = fmaf(gacc[1][q], g1, acc[0][1][q]);
                        }
                        // Pin the update here: left to the compiler it was
                        // sunk past later groups, whose products then needed
                        // fresh accumulator registers (224 AGPRs, one wave per
                        // SIMD).
                        asm volatile("" : "+v"(acc[0][0]), "+v"(acc[0][1]));
                    }
                } else {
#pragma unroll
                for (int i = 0; i < NB; ++i) {
                    const bf16x8 ai = DIRECT ? __builtin_bit_cast(bf16x8, ad[u % DD][s])
                                             : CP ? avc[s][i] : av[s & 1][i];
                    acc[i][0] = mfma32(ai, b0.hi, acc[i][0]);
                    acc[i][1] = mfma32(ai, b1.hi, acc[i][1]);
                    if constexpr (FMT != kFmtMxfp4) {
                        acc[i][0] = mfma32(ai, b0.lo, acc[i][0]);
                        acc[i][1] = mfma32(ai, b1.lo, acc[i][1]);
                    }
                }
                }
                // Interleave: each MFMA pair is followed by an operand read
                // and a couple of converts for the next step (and at s = 0 by
                // the stores and loads), so the matrix core is fed while the
                // VALU and LDS work proceeds. Not for the 1-2 block tiles that
                // read whole chunks ahead: there the compiler's own order was
                // 4 % faster (decode batches of 32 tokens), and for 3-8 blocks
                // 1-2 % slower.
                if constexpr (!CP)
#pragma unroll
                for (int i = 0; i < NB; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
                    if (s == 0) {
                        __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);  // DS write
                        __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);  // VMEM read
                    }
                    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU
                }
                __builtin_amdgcn_sched_barrier(0);  // one k-step per scheduling region
                b0 = n0;
                b1 = n1;
            }
            bcur[0] = bnext[0];
            bcur[1] = bnext[1];
            if (u == 3) {
                scur[0] = snext[0];
                scur[1] = snext[1];
            }
            if (CP) {
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
                    for (int i = 0; i < NB; ++i) avc[s4][i] = avn[s4][i];
            }
            // Barrier: A(c+2) visible, buffer c%3 free for A(c+3). Only the
            // LDS operations older than the last NB (the next chunk's first
            // operand reads, issued in the k-step just before) must be
            // complete; those reads stay in flight across the barrier.
            // (With chunk-level reads every LDS operation completes first.)
            if (DIRECT) {
                issue_ad(u % DD, c + DD);  // the slot this chunk used
                wave_lds_sync();
            } else if (CP) {
                __syncthreads();
            } else {
                asm volatile("s_waitcnt lgkmcnt(%0)\n\ts_barrier" ::"n"(NB) : "memory");
            }
            buf = buf1;
        }
    }

    // --- epilogue. acc[i][j][q]: row 32i + 8(q/4) + 4*half + q%4, column nl.
    // For a fixed (i, q) the wave holds two rows of 32 consecutive columns,
    // so one 2- or 4-byte store per lane writes two contiguous segments; the
    // row offset is wave-uniform and goes in the scalar offset.
    if (STAGE == 1) {
        // Padding rows store nothing (out-of-range offset): the down GEMM's
        // results for them are dropped, so their h values are never used.
        const rsrc_t rh = make_rsrc(a.h, (uint32_t)(a.cap * a.I * 2));
        const uint32_t vbase = ((uint32_t)(row0 + 4 * half) * (uint32_t)a.I + (uint32_t)(n0 + 32 * w + nl)) * 2u;
        // Expert bias / clamp (optional): a separate store loop, so the plain
        // epilogue is unchanged.
        if (EPI && (a.w13_bias || a.swiglu_limit > 0.0f)) {
            GluTerms glu;
            glu.load(a, e, n0 + 32 * w + nl);
#pragma unroll
            for (int i = 0; i < NB; ++i)
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int r = 32 * i + 8 * (q >> 2) + 4 * half + (q & 3);
                    const int p = sh.rows[r];
                    const uint32_t soff = (uint32_t)(32 * i + 8 * (q >> 2) + (q & 3)) * (uint32_t)(2 * a.I);
                    float g = acc[i][0][q], u = acc[i][1][q];
                    glu.apply(g, u);
                    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(swiglu_fast(g, u)), rh,
                                                          (p >= 0 && p < P) ? vbase : kOob, soff, 0);
                }
            return;
        }
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int r = 32 * i + 8 * (q >> 2) + 4 * half + (q & 3);
                const int p = sh.rows[r];
                const uint32_t soff = (uint32_t)(32 * i + 8 * (q >> 2) + (q & 3)) * (uint32_t)(2 * a.I);
                __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(swiglu_fast(acc[i][0][q], acc[i][1][q])),
                                                      rh, (p >= 0 && p < P) ? vbase : kOob, soff, 0);
            }
    } else {
        const rsrc_t ry = make_rsrc(a.y, (uint32_t)((int64_t)P * a.H * 4));
        const uint32_t col4 = (uint32_t)(n0 + 64 * w + nl) * 4u;
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int r = 32 * i + 8 * (q >> 2) + 4 * half + (q & 3);
                const int p = sh.rows[r];
                // Padding rows get an out-of-range offset: the store is dropped.
                const uint32_t off = (p >= 0 && p < P) ? (uint32_t)p * (uint32_t)(4 * a.H) + col4 : kOob;
                // The store builtin takes integer data. (A bit_cast of the vector
                // element was folded to element 0 by the compiler.)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][0][q]), ry, off, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][1][q]), ry, off, 128, 0);
            }
    }
}

// One workgroup per (32-row block, 64 weight rows), for small batches: a
// token routes to an expert at most once, so with T <= 32 no expert holds
// more than one block and the blocks are the whole work list (no super-block
// pass). Correct for any block list; an expert with several blocks would
// just stream its weights once per block.
template <int STAGE, int FMT>
__global__ __launch_bounds__(64) void prefill_direct_kernel(MoeGemmArgs a, int nblocks, int ntiles) {
    __shared__ PfSharedDirect sh;
    // Workgroup ids go round-robin over the 8 XCDs: block blk lives on XCD
    // blk % 8 with all of its N tiles, so its activation rows stay in one L2.
    const int b = blockIdx.x;
    const int xcd = b & 7, j = b >> 3;
    const int blk = 8 * (j / ntiles) + xcd;
    const int nt = j % ntiles;
    if (blk >= nblocks) return;
    const int e = a.block_expert[blk];
    if (e < 0 || e >= a.E) return;
    const int row0 = blk * kPfBlockRows;
    if (threadIdx.x < kPfBlockRows) sh.rows[threadIdx.x] = a.sorted_ids[row0 + threadIdx.x];
    wave_lds_sync();
    pf_tile<STAGE, FMT, 1, true>(a, sh, e, row0, nt * (STAGE == 1 ? 32 : 64));
}

// Single-wave int4 kernels (gemm_prefill_int4.hip).
hipError_t launch_prefill_direct_int4(const MoeGemmArgs& a, int stage, dim3 grid, int nblocks, int ntiles,
                                      hipStream_t s);

}  // namespace moe

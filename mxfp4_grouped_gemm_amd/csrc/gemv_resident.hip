// Decode GEMMs (MXFP4 or int4-g32 weights, expert blocks of up to 16 token
// rows) with the block's activation rows resident in LDS, in a persistent
// grid of one 8-wave workgroup per compute unit.
//
// The products are those of gemv_mfma.hip (v_mfma_f32_4x4x4_16b_bf16, lane
// 4 seg + r holding MX block (int4: 32-group) seg of weight row r and the
// same K range of token row r, 16 weight rows x up to 16 token rows per
// wave), but the activation side no longer travels with every chunk of
// weights:
//  * the workgroup copies the rows of its current expert block (all of K,
//    up to 16 rows: 115 KB at K = 3584) into LDS once, when its run of units
//    enters the block, and every wave reads its MFMA operands from there;
//  * the workgroup owns a contiguous run of steps (a step = 8 consecutive
//    units of one block, one per wave), so it changes block at most a few
//    times and nothing else is shared: no per-chunk barrier;
//  * each wave holds a whole unit of weight codes in registers (NCH chunks
//    of 4 rows x 256 bytes per instruction) and loads the next unit's chunk
//    c as soon as it has decoded chunk c of the current one, so one unit of
//    weights (28 KB at K = 3584) is in flight per wave at all times, across
//    unit and block boundaries;
//  * the runs are cut so that every workgroup gets the same summed cost: a
//    unit costs more with more token groups, and with equal step counts the
//    few workgroups holding the fullest blocks would finish last.
// The token groups of a block (4 rows each) are multiplied behind uniform
// branches, so blocks of a few rows issue no MFMAs for the empty ones. int4
// weights take at most two groups per pass (the per-chunk group sums need
// the registers of the other two): a block of more than 8 rows runs each
// unit twice. The per-unit scales, the row pairs and (int4) the activation
// sums of each row and 32-group come from LDS, and the stage-1 biases are
// loaded at the start of the unit, so the epilogue never waits on global
// memory behind the next unit's weights.
// LDS rows have a stride of 2 K + 16 bytes and are filled 4 rows x 4 pieces
// (64 bytes apart) per 16 lanes; with K a multiple of 512 both the fill and
// the operand reads touch each of the 64 banks once per 16 lanes.
#include "gemv_mfma.hpp"
#include "route.hpp"  // wave_incl_scan

namespace moe {

constexpr int kPxWaves = 8;   // waves per workgroup: two per SIMD
constexpr int kPxRows = 16;   // token rows of a block held in LDS
constexpr int kPxMaxBlocks = kPxWaves * 64;  // expert blocks a launch may hold: one per thread

template <int NCH>
struct PxRing {
    u32x4 w[NCH][kGmSets];  // 16 code bytes of this lane's row of each set, per chunk
};

template <int STAGE>
struct PxUnit {
    int64_t b;  // expert block
    int e;      // expert (outside [0, E): no weights)
    int c0;     // stage 1: first gate column; stage 2: first row of w2
    rsrc_t rw, rs;  // the expert's weight codes and scales from row c0 on
};

template <int FMT, int STAGE, int NCH, bool EPI>
__global__ __launch_bounds__(kPxWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
void gemv_resident_kernel(MoeGemmArgs a) {
    constexpr bool kInt4 = FMT == kFmtInt4g32;
    constexpr int K = 512 * NCH, nblk = K / 32;  // K = H (stage 1) or I (stage 2)
    constexpr int SB = kInt4 ? 2 : 1;            // bytes per scale
    constexpr int kPassG = kInt4 ? 2 : 4;        // token groups per pass
    constexpr uint32_t xstride = 2u * K + 16u;
    constexpr uint32_t kSpare = kPxRows * xstride;  // a 16-byte slot past the rows
    __shared__ __attribute__((aligned(16))) uint8_t xt[kSpare + 16];
    __shared__ __attribute__((aligned(16))) uint8_t lds_scale[kPxWaves][16 * nblk * SB];
    __shared__ float xsum[kInt4 ? kPxRows * nblk : 1];  // int4: sum of each row's 32-groups
    __shared__ uint32_t rowoff[kPxRows];
    __shared__ int32_t rowpair[kPxRows];
    __shared__ uint32_t wsum[kPxWaves];
    __shared__ int32_t bexp_lds[kPxMaxBlocks];
    __shared__ int64_t bound[2];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = a.H, I = a.I;
    const int upb = STAGE == 1 ? I / 8 : H / 16;  // units per block
    const int spb = upb / kPxWaves;               // steps per block
    const int P = a.T * a.topk;
    // Everything the partition needs in one round trip: the block count,
    // every block's sorted ids and its expert (thread b holds block b).
    const int nbcap = (int)(a.cap / a.bm);  // at most kPxMaxBlocks (launcher)
    const rsrc_t rsid = make_rsrc(a.sorted_ids, (uint32_t)(a.cap * 4));
    u32x4 sid[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) sid[k] = bld16(rsid, tid < nbcap ? (uint32_t)tid * 64u + 16u * k : kOob);
    const int bexp_t = tid < nbcap ? a.block_expert[tid] : -1;
    int64_t nused = *a.num_post_pad / a.bm;
    if (nused > nbcap) nused = nbcap;
    const int64_t S = nused * spb;
    if (S == 0) return;

    // Cost-balanced runs of steps: thread b weighs block b by its rows (the
    // pairs in the sort; measured per unit with every block at 1, 2 or 4
    // groups, 1 : 1.07 : 1.46 for MXFP4; int4 runs 4 groups as two passes of
    // 2), a workgroup scan gives the prefix, and the block that holds each of
    // this workgroup's two cut points places it.
    {
        const bool mine = tid < nused;
        int cnt = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int i = 0; i < 4; ++i) cnt += ((int)sid[k][i] >= 0 && (int)sid[k][i] < P) ? 1 : 0;
        bexp_lds[tid] = bexp_t;
        const uint32_t cost = !mine ? 0u : cnt > 8 ? (kInt4 ? 28u : 19u) : cnt > 4 ? 14u : 13u;
        uint32_t incl = (uint32_t)wave_incl_scan((int)cost);
        if (lane == 63) wsum[wave] = incl;
        if (tid == 0) bound[0] = bound[1] = S;
        __syncthreads();
        uint32_t total = 0;
#pragma unroll
        for (int w = 0; w < kPxWaves; ++w) {
            const uint32_t ws = wsum[w];
            incl += w < wave ? ws : 0u;
            total += ws;
        }
        // 32-bit: total <= 512 blocks x 28, spb <= 64 (H, I <= 4096) and a
        // grid of at most 4096 workgroups (the launcher's bound) keep every
        // product below 2^32.
        const uint32_t tt = total * (uint32_t)spb;
        const uint32_t lo = (incl - cost) * (uint32_t)spb, hi = incl * (uint32_t)spb;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t t = (blockIdx.x + (uint32_t)j) * tt / gridDim.x;
            if (mine && t >= lo && t < hi) bound[j] = (int64_t)tid * spb + (int64_t)((t - lo) / cost);
        }
        __syncthreads();
    }
    const int64_t s0 = bound[0], s1 = bound[1];
    if (s0 >= s1) return;  // uniform per workgroup
    const int seg = lane >> 2, r = lane & 3;
    const int64_t slab_rows = STAGE == 1 ? 2 * (int64_t)I : (int64_t)H;
    const uint8_t* wbase = STAGE == 1 ? a.w13 : a.w2;
    const uint8_t* sbase = (const uint8_t*)(STAGE == 1 ? a.w13_scale : a.w2_scale);
    const rsrc_t rx = STAGE == 1 ? make_rsrc(a.x, (uint32_t)((int64_t)a.T * H * 2))
                                 : make_rsrc(a.h, (uint32_t)((int64_t)P * I * 2));
    uint8_t* lds = lds_scale[wave];
    // This lane's scales in the wave's LDS rows (runs staged in order): row
    // (stage 1) r < 2 ? r + 2s : r + 6 + 2s, (stage 2) r + 4s; element seg
    // of each chunk's 16.
    const int lsc = (STAGE == 1 ? (r < 2 ? r : r + 6) : r) * nblk + seg;
    constexpr int kScSetStride = (STAGE == 1 ? 2 : 4) * nblk;

    // The experts of the workgroup's blocks (at most 64), one per lane: a
    // unit's expert is a lane read (a vector load per unit would be waited
    // for behind the weights already in flight).
    const int64_t b0 = s0 / spb;
    const int bexp = b0 + lane < nused ? bexp_lds[b0 + lane] : -1;
    auto unit_of = [&](int64_t s, PxUnit<STAGE>& u) {
        u.b = s / spb;
        const int q = (int)(s - u.b * spb) * kPxWaves + wave;
        u.c0 = q * (STAGE == 1 ? 8 : 16);
        const int64_t d = u.b - b0;
        u.e = __builtin_amdgcn_readlane(bexp, (int)d);  // d < 64: at most 63 blocks per workgroup (launcher)
        const bool ok = (unsigned)u.e < (unsigned)a.E;
        const int64_t row = (ok ? u.e : 0) * slab_rows + u.c0;
        const uint32_t rows_left = ok ? (uint32_t)(slab_rows - u.c0) : 0u;
        u.rw = make_rsrc(wbase + row * (K / 2), rows_left * (K / 2));
        u.rs = make_rsrc(sbase + row * nblk * SB, rows_left * nblk * SB);
    };
    // Lane offset from row c0 of the unit: this lane's row of set 0 (stage
    // 1: gate c0 + r or up I + c0 + r - 2; stage 2: c0 + r), segment seg. Set
    // s adds a whole number of rows (2 s in stage 1, 4 s in stage 2), which
    // goes into the scalar offset of the load.
    const uint32_t woff = (uint32_t)(STAGE == 1 ? (r < 2 ? r : I + r - 2) : r) * (uint32_t)(K / 2) + 16u * seg;
    constexpr uint32_t kSetStride = (STAGE == 1 ? 2 : 4) * (K / 2);
    // The unit's 16 rows of scales (nblk each, two runs in stage 1) as
    // 16-byte pieces: kScPieces per lane.
    constexpr int kScPieces = (nblk * SB + 63) / 64;
    auto issue_scales = [&](const PxUnit<STAGE>& u, u32x4 (&sc)[kScPieces], uint32_t mask) {
#pragma unroll
        for (int k = 0; k < kScPieces; ++k) {
            const int p = lane + 64 * k;
            constexpr int p0 = (STAGE == 1 ? 8 : 16) * nblk * SB / 16;
            const uint32_t so = p < p0 ? 16u * p : p < nblk * SB ? (uint32_t)I * nblk * SB + 16u * (p - p0) : kOob;
            sc[k] = bld16nt(u.rs, so | mask);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // Every load in one fixed order, here and in the prologue: the wait
    // counts are then exact across the unit loop (vector loads complete in
    // order), so a chunk's first use waits only for that chunk.
    auto issue_chunk = [&](PxRing<NCH>& ring, const PxUnit<STAGE>& u, int c, uint32_t mask) {
#pragma unroll
        for (int s = 0; s < kGmSets; ++s) {
            ring.w[c][s] = bld16snt(u.rw, (woff + 256u * c) | mask, kSetStride * s);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // The block's rows into LDS (int4: each 16-byte piece in the codes'
    // element order, and the sums of each row's 32-groups); returns its
    // token groups (1, 2 or 4).
    auto fill_x = [&](int64_t b) -> int {
        const int64_t row0 = b * a.bm;
        const int p = a.sorted_ids[row0 + (lane & 15)];
        const bool ok = p >= 0 && p < P;
        const int nvalid = __popcll(__builtin_amdgcn_ballot_w64(ok) & 0xFFFFull);
        const int ng = nvalid > 4 ? (nvalid > 8 ? 4 : 2) : 1;
        __syncthreads();  // every wave is done with the previous block's rows
        if (wave == 0 && lane < 16) {
            rowpair[lane] = ok ? p : -1;
            rowoff[lane] = ok ? (STAGE == 1 ? (uint32_t)(p / a.topk) * (uint32_t)(2 * H) : (uint32_t)p * (uint32_t)(2 * I))
                              : kOob;
        }
        __syncthreads();
        // Element i: row 4 rq + rl, 16-byte piece 16 m + 4 pj + n. Branch-
        // free: elements past the end load nothing (kOob) and are stored to a
        // spare slot, so every load is consumed on the one path (a load left
        // pending on some path would make later waits conservative).
        constexpr int mper = K / 128;  // pieces per row / 16
        const int total = 64 * ng * mper;
#pragma unroll 1
        for (int base = 0; base < total; base += kPxWaves * 64 * 2) {
            u32x4 v[2];
            uint32_t dst[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int i = base + kPxWaves * 64 * j + tid;
                const int rl = i & 3, pj = (i >> 2) & 3, n = (i >> 4) & 3, g2 = i >> 6;
                const int rq = g2 / mper, m = g2 - rq * mper;
                const int row = (4 * rq + rl) & (kPxRows - 1), piece = 16 * m + 4 * pj + n;
                const uint32_t ro = i < total ? rowoff[row] : kOob;
                v[j] = bld16(rx, ro + 16u * piece);  // kOob + 16 piece stays past the record
                if constexpr (kInt4) v[j] = __builtin_bit_cast(u32x4, perm_x_int4(__builtin_bit_cast(bf16x8, v[j])));
                dst[j] = i < total ? (uint32_t)row * xstride + 16u * piece : kSpare;
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) *(u32x4*)(xt + dst[j]) = v[j];
        }
        __syncthreads();
        if constexpr (kInt4) {
            // Sum of each (row, 32-group): four 16-byte pieces, fp32, in order.
#pragma unroll 1
            for (int i = tid; i < 4 * ng * nblk; i += kPxWaves * 64) {
                const int row = i / nblk, grp = i - row * nblk;
                const uint8_t* src = xt + (uint32_t)row * xstride + 64u * grp;
                float sum = 0.0f;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const u32x4 v = *(const u32x4*)(src + 16 * k);
#pragma unroll
                    for (int e = 0; e < 4; ++e) sum += __uint_as_float(v[e] << 16) + __uint_as_float(v[e] & 0xffff0000u);
                }
                xsum[i] = sum;
            }
            __syncthreads();
        }
        return ng;
    };

    // Chunk c of a unit against token groups g0 .. g0 + ngp - 1 (acc[g - g0]):
    // the decode and the first group on every path, the others behind uniform
    // branches (whole-chunk bodies per group count let the compiler hoist the
    // shared decode of all four K steps above the branch).
    auto consume = [&](int g0, int ngp, const u32x4 (&w)[kGmSets], int c, f32x4 (&acc)[kPassG][kGmSets]) {
        const int blk = 16 * c + seg;
        if constexpr (!kInt4) {
            float sc[kGmSets];
#pragma unroll
            for (int s = 0; s < kGmSets; ++s) sc[s] = e8m0_scale_operand(lds[lsc + kScSetStride * s + 16 * c]);
            auto group = [&](const bf16x8 (&wv)[kGmSets], int gi, int q) {
                const bf16x8 xv = *(const bf16x8*)(xt + (uint32_t)(4 * (g0 + gi) + r) * xstride + 64u * blk + 16u * q);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const bf16x4_t xh = h ? __builtin_shufflevector(xv, xv, 4, 5, 6, 7)
                                          : __builtin_shufflevector(xv, xv, 0, 1, 2, 3);
#pragma unroll
                    for (int s = 0; s < kGmSets; ++s) {
                        const bf16x4_t wb = h ? __builtin_shufflevector(wv[s], wv[s], 4, 5, 6, 7)
                                              : __builtin_shufflevector(wv[s], wv[s], 0, 1, 2, 3);
                        acc[gi][s] = mfma4x4(wb, xh, acc[gi][s]);
                    }
                }
            };
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                bf16x8 wv[kGmSets];
#pragma unroll
                for (int s = 0; s < kGmSets; ++s) wv[s] = mxfp4x8_to_bf16(w[s][q], sc[s]);
                group(wv, 0, q);
                if (ngp > 1) group(wv, 1, q);
                if (ngp > 2) {
                    group(wv, 2, q);
                    group(wv, 3, q);
                }
            }
        } else {
            // Per group: the products of code + 136 with the permuted
            // activations over the lane's 32-group, then the fold with the
            // group's bf16 scale and activation sum (gm_int4_fold).
            const uint16_t* lsc16 = (const uint16_t*)lds + lsc + 16 * c;
            float sc[kGmSets];
#pragma unroll
            for (int s = 0; s < kGmSets; ++s) sc[s] = bf16_bits_to_f32(lsc16[kScSetStride * s]);
            // K steps outer (the decode shared by the groups), groups inner.
            f32x4 t[kPassG][kGmSets];
#pragma unroll
            for (int gi = 0; gi < kPassG; ++gi)
#pragma unroll
                for (int s = 0; s < kGmSets; ++s) t[gi][s] = f32x4{0.f, 0.f, 0.f, 0.f};
            auto group = [&](const bf16x8 (&wv)[kGmSets], int gi, int q) {
                const bf16x8 xv = *(const bf16x8*)(xt + (uint32_t)(4 * (g0 + gi) + r) * xstride + 64u * blk + 16u * q);
                const bf16x4_t x0 = __builtin_shufflevector(xv, xv, 0, 1, 2, 3);
                const bf16x4_t x1 = __builtin_shufflevector(xv, xv, 4, 5, 6, 7);
#pragma unroll
                for (int s = 0; s < kGmSets; ++s) {
                    t[gi][s] = mfma4x4(__builtin_shufflevector(wv[s], wv[s], 0, 1, 2, 3), x0, t[gi][s]);
                    t[gi][s] = mfma4x4(__builtin_shufflevector(wv[s], wv[s], 4, 5, 6, 7), x1, t[gi][s]);
                }
            };
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                bf16x8 wv[kGmSets];
#pragma unroll
                for (int s = 0; s < kGmSets; ++s) wv[s] = int4x8_to_bf16_biased(w[s][q]);
                group(wv, 0, q);
                if (ngp > 1) group(wv, 1, q);
            }
            auto fold = [&](int gi) {
                const float xs1 = xsum[(4 * (g0 + gi) + r) * nblk + blk];  // token r of the group
                const f32x4 xs = {xs1, xs1, xs1, xs1};
#pragma unroll
                for (int s = 0; s < kGmSets; ++s) gm_int4_fold(t[gi][s], xs, sc[s], acc[gi][s]);
            };
            fold(0);
            if (ngp > 1) fold(1);
            // Each chunk's fold stays in its chunk (the compiler would sink
            // them all to the unit's end, keeping every chunk's products live).
#pragma unroll
            for (int gi = 0; gi < kPassG; ++gi)
#pragma unroll
                for (int s = 0; s < kGmSets; ++s) asm volatile("" : "+v"(acc[gi][s]));
        }
    };
    // One unit (one pass): consumes the ring and refills it with the next
    // unit's chunks (mask: kOob when there is none). The refill is on the one
    // common path, so the loads in flight keep their registers across units
    // (per-unit bodies that each reloaded the ring were joined by register
    // copies, which wait for every load).
    auto run_unit = [&](int g0, int ngp, PxRing<NCH>& ring, const PxUnit<STAGE>& cur, const PxUnit<STAGE>& nxt,
                        uint32_t mask, uint32_t bg, uint32_t bu) {
        f32x4 acc[kPassG][kGmSets];
#pragma unroll
        for (int g = 0; g < kPassG; ++g)
#pragma unroll
            for (int s = 0; s < kGmSets; ++s) acc[g][s] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            consume(g0, ngp, ring.w[c], c, acc);
            issue_chunk(ring, nxt, c, mask);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int gi = 0; gi < kPassG; ++gi) {
            if (gi >= ngp) break;
            gm_reduce(acc[gi]);
            const int pr = rowpair[4 * (g0 + gi) + r];
            if constexpr (STAGE == 1) {
                // Lane 4c + j with c < 8 stores (token j, column c0 + 2 (c & 3) + (c >> 2)).
                const int sel = seg & 3, half = (seg >> 2) & 1;
                const int col = cur.c0 + 2 * sel + half;
                float gv = 0.f, uv = 0.f;
#pragma unroll
                for (int s = 0; s < kGmSets; ++s) {
                    gv = s == sel ? (half ? acc[gi][s][1] : acc[gi][s][0]) : gv;
                    uv = s == sel ? (half ? acc[gi][s][3] : acc[gi][s][2]) : uv;
                }
                if (lane < 32 && pr >= 0) {
                    if constexpr (EPI) {
                        gv += __uint_as_float(bg << 16);
                        uv += __uint_as_float(bu << 16);
                        const float lim = a.swiglu_limit;
                        if (lim > 0.0f) {
                            gv = fminf(fmaxf(gv, -lim), lim);
                            uv = fminf(fmaxf(uv, -lim), lim);
                        }
                    }
                    a.h[(int64_t)pr * I + col] = f32_to_bf16_bits(swiglu(gv, uv));
                }
            } else {
                // Lane 4c + j stores (token j, row n0 + 4 (c & 3) + (c >> 2)).
                const int sel = seg & 3, slot = seg >> 2;
                float v = 0.f;
#pragma unroll
                for (int s = 0; s < kGmSets; ++s)
#pragma unroll
                    for (int i = 0; i < 4; ++i) v = (s == sel && i == slot) ? acc[gi][s][i] : v;
                if (pr >= 0) a.y[(int64_t)pr * H + cur.c0 + 4 * sel + slot] = v;
            }
        }
    };

    PxUnit<STAGE> cur, nxt;
    unit_of(s0, cur);
    u32x4 scn[kScPieces];
    issue_scales(cur, scn, 0u);
    PxRing<NCH> ring;
#pragma unroll
    for (int c = 0; c < NCH; ++c) issue_chunk(ring, cur, c, 0u);
    __builtin_amdgcn_sched_barrier(0);
    int64_t cb = -1;
    int ng = 1, pass = 0;
    for (int64_t s = s0; s < s1;) {
        if (cur.b != cb) {  // uniform: the workgroup's waves change block together
            ng = fill_x(cur.b);
            cb = cur.b;
        }
        // This unit's scales (loaded one unit ahead) into the wave's LDS rows;
        // the previous unit's reads of them are complete (LDS runs in order).
#pragma unroll
        for (int k = 0; k < kScPieces; ++k)
            if (lane + 64 * k < nblk * SB) *(u32x4*)(lds + 16 * (lane + 64 * k)) = scn[k];
        wave_lds_sync();
        // Stage-1 biases of this lane's output column, loaded ahead of the
        // next unit's weights; branch-free (no bias: an empty record reads
        // zeros), and converted only in the epilogue, so nothing waits here.
        uint32_t bg = 0u, bu = 0u;
        if constexpr (EPI && STAGE == 1) {
            const bool ok = a.w13_bias && (unsigned)cur.e < (unsigned)a.E;
            const rsrc_t rb = make_rsrc(ok ? a.w13_bias + (int64_t)cur.e * 2 * I : a.w13_bias, ok ? 4u * I : 0u);
            const uint32_t col = cur.c0 + 2 * (seg & 3) + ((seg >> 2) & 1);
            bg = __builtin_amdgcn_raw_buffer_load_b16(rb, 2u * col, 0, 0);
            bu = __builtin_amdgcn_raw_buffer_load_b16(rb, 2u * (I + col), 0, 0);
        }
        // The next unit: this one again for its second pass (int4, blocks of
        // more than 8 rows), else the next step's; none after the last.
        const int g0 = kPassG * pass;
        const int ngp = ng - g0 < kPassG ? ng - g0 : kPassG;
        const bool again = g0 + kPassG < ng;
        const bool more = again || s + 1 < s1;
        unit_of(again ? s : s + 1, nxt);
        const uint32_t mask = more ? 0u : kOob;
        issue_scales(nxt, scn, mask);
        run_unit(g0, ngp, ring, cur, nxt, mask, bg, bu);
        if (again) {
            ++pass;
        } else {
            pass = 0;
            ++s;
        }
        cur = nxt;
    }
}

// One workgroup per compute unit.
static int resident_grid() {
    static int cus = 0;
    if (!cus) {
        int dev = 0, n = 0;
        cus = (hipGetDevice(&dev) == hipSuccess &&
               hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
                  ? n
                  : 256;
    }
    return cus;
}

// Every block is weighed by one thread, and a workgroup's run of steps
// spans a few blocks (the kernel reads the experts of up to 64). K up to
// 4096 (MXFP4) or 3584 (int4, whose scale rows take twice the LDS).
bool gemv_resident_eligible(const MoeGemmArgs& a) {
    const int kmax = a.fmt == kFmtMxfp4 ? 4096 : 3584;
    return (a.fmt == kFmtMxfp4 || a.fmt == kFmtInt4g32) && a.bm == 16 && a.cap / 16 <= kPxMaxBlocks &&
           resident_grid() >= 32 && resident_grid() <= 4096 && a.H <= kmax && a.I <= kmax && a.H % 512 == 0 && a.I % 512 == 0 &&
           (int64_t)a.T * a.topk * a.I * 2 < 0x7fff0000LL && (int64_t)a.T * a.H * 2 < 0x7fff0000LL;
}

template <int FMT, int NCH>
static void launch_px_nch(const MoeGemmArgs& a, int stage, dim3 grid, dim3 block, hipStream_t s) {
    if constexpr (FMT == kFmtInt4g32 && NCH > 7) {
        return;  // not eligible
    } else if (stage == 1) {
        if (a.w13_bias || a.swiglu_limit > 0.0f)
            hipLaunchKernelGGL((gemv_resident_kernel<FMT, 1, NCH, true>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((gemv_resident_kernel<FMT, 1, NCH, false>), grid, block, 0, s, a);
    } else {
        hipLaunchKernelGGL((gemv_resident_kernel<FMT, 2, NCH, false>), grid, block, 0, s, a);
    }
}

template <int NCH>
static void launch_px_nch(const MoeGemmArgs& a, int stage, dim3 grid, dim3 block, hipStream_t s) {
    if (a.fmt == kFmtMxfp4) launch_px_nch<kFmtMxfp4, NCH>(a, stage, grid, block, s);
    else launch_px_nch<kFmtInt4g32, NCH>(a, stage, grid, block, s);
}

hipError_t launch_gemv_resident_stage(const MoeGemmArgs& a, int stage, hipStream_t s) {
    const dim3 grid((unsigned)resident_grid()), block(kPxWaves * 64);
    const int nch = (stage == 1 ? a.H : a.I) / 512;  // 1..8
    switch (nch) {
        case 1: launch_px_nch<1>(a, stage, grid, block, s); break;
        case 2: launch_px_nch<2>(a, stage, grid, block, s); break;
        case 3: launch_px_nch<3>(a, stage, grid, block, s); break;
        case 4: launch_px_nch<4>(a, stage, grid, block, s); break;
        case 5: launch_px_nch<5>(a, stage, grid, block, s); break;
        case 6: launch_px_nch<6>(a, stage, grid, block, s); break;
        case 7: launch_px_nch<7>(a, stage, grid, block, s); break;
        default: launch_px_nch<8>(a, stage, grid, block, s); break;
    }
    return hipGetLastError();
}

}  // namespace moe

// Decode GEMMs for expert blocks of 2-16 token rows (MXFP4 or int4-g32
// weights) whose multiply-adds run on the matrix core:
// v_mfma_f32_4x4x4_16b_bf16, sixteen independent 4x4x4 products per
// instruction.
//
// The GEMV kernels (gemm_gemv.hip) dot every decoded weight with each token
// row on the VALU: 16 v_dot2 per 16 code bytes per row, so from about four
// rows per block the VALU, not HBM, sets their pace. Here lane 4b + r holds
// MX block b of weight row r (16 code bytes, one e8m0 scale) and the same K
// range of token row r; the sixteen 4x4 products of one MFMA are the sixteen
// K segments b of a 4-row x 4-token product, each over 4 K elements, so 8
// MFMAs consume one 16-byte code load for 4 tokens and the K segments are
// summed across lanes once per unit. The VALU keeps only the decode.
//
// A wave owns 16 weight rows (four sets of 4) over the whole K and 4 token
// rows (a token group) of one expert block; the activation fragments of a K
// chunk (16 MX blocks) feed all four row sets, so a chunk is 4 code loads +
// 4 activation loads of 1 KB. Chunks stream through a register ring of depth
// D (codes and activations of a chunk issued together; vector loads complete
// in order). The rows' scales (e8m0 bytes, or the int4 groups' bf16) go
// through wave-private LDS. A block of more than 4 rows takes its token
// groups one after another, each a further pass over the same weights. With
// int4-g32 weights a lane's 16 code bytes are one 32-group of its row, so the
// products of a chunk are folded per group (gm_int4_fold).
// Stage 1 takes gate columns i0 .. i0+7 and the matching up columns (row set
// s = gate 2s, gate 2s+1, up 2s, up 2s+1), so SwiGLU is formed in registers;
// stage 2 takes 16 consecutive rows of w2. h and y are stored by pair index,
// as on the GEMV path, and the combine kernel follows.
#include "gemv_mfma.hpp"

namespace moe {

constexpr int kGmWaves = 4;  // waves per workgroup: four units of one block

struct GmSlot {
    u32x4 w[kGmSets];  // 16 code bytes of this lane's row in each row set
    u32x4 x[4];        // 64 activation bytes of this lane's token
};

// One unit: 16 weight rows of one expert over K (nblk MX blocks or int4
// groups in NCH chunks of 16) against the token rows of x_off (kOob: no row),
// acc[s] += partial sums. w_off[s]: byte offset of this lane's row of set s in
// rw; lrow[s]: its row in the wave's LDS scale table (nblk scales per row).
// Fully unrolled over the chunks, without branches.
template <int FMT, int D, int NCH>
__device__ __forceinline__ void gm_k_loop(rsrc_t rw, rsrc_t rx, uint32_t (&w_off)[kGmSets], uint32_t x_off,
                                          const uint8_t* lds_scale, int (&lrow)[kGmSets], int nblk, int seg,
                                          f32x4 (&acc)[kGmSets]) {
    // Opaque to the optimizer from here: when a block's token groups run this
    // loop one after another, the per-chunk offsets are then recomputed in
    // each pass rather than kept live across passes (44 VGPRs).
#pragma unroll
    for (int s = 0; s < kGmSets; ++s) asm volatile("" : "+v"(w_off[s]), "+v"(lrow[s]));
    asm volatile("" : "+v"(seg));
    GmSlot ring[D];
    // Blocks past nblk (the last chunk's) load zeros without memory traffic:
    // an offset with bit 31 set is past every record.
    auto issue = [&](GmSlot& r, int c) {
        const uint32_t oob = (uint32_t)(16 * c + seg >= nblk) << 31;
#pragma unroll
        for (int s = 0; s < kGmSets; ++s) r.w[s] = bld16nt(rw, (w_off[s] + 256u * c) | oob);
        const uint32_t o = (x_off + 1024u * c) | oob;
#pragma unroll
        for (int q = 0; q < 4; ++q) r.x[q] = bld16(rx, o + 16u * q);
    };
    auto consume = [&](const GmSlot& r, int c) {
        const int blk = min(16 * c + seg, nblk - 1);
        if constexpr (FMT == kFmtMxfp4) {
            float sc[kGmSets];
#pragma unroll
            for (int s = 0; s < kGmSets; ++s) sc[s] = e8m0_scale_operand(lds_scale[lrow[s] * nblk + blk]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                bf16x8 wv[kGmSets];
#pragma unroll
                for (int s = 0; s < kGmSets; ++s) wv[s] = mxfp4x8_to_bf16(r.w[s][q], sc[s]);
                const bf16x8 xv = __builtin_bit_cast(bf16x8, r.x[q]);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const bf16x4_t xb = h ? __builtin_shufflevector(xv, xv, 4, 5, 6, 7)
                                          : __builtin_shufflevector(xv, xv, 0, 1, 2, 3);
#pragma unroll
                    for (int s = 0; s < kGmSets; ++s) {
                        const bf16x4_t wb = h ? __builtin_shufflevector(wv[s], wv[s], 4, 5, 6, 7)
                                              : __builtin_shufflevector(wv[s], wv[s], 0, 1, 2, 3);
                        acc[s] = mfma4x4(wb, xb, acc[s]);
                    }
                }
            }
        } else {
            const bf16x4_t ones = __builtin_bit_cast(bf16x4_t, u32x2{0x3F803F80u, 0x3F803F80u});
            f32x4 t[kGmSets], xs = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < kGmSets; ++s) t[s] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const bf16x8 xv = perm_x_int4(__builtin_bit_cast(bf16x8, r.x[q]));
                const bf16x4_t x0 = __builtin_shufflevector(xv, xv, 0, 1, 2, 3);
                const bf16x4_t x1 = __builtin_shufflevector(xv, xv, 4, 5, 6, 7);
                xs = mfma4x4(ones, x0, xs);
                xs = mfma4x4(ones, x1, xs);
#pragma unroll
                for (int s = 0; s < kGmSets; ++s) {
                    const bf16x8 wv = int4x8_to_bf16_biased(r.w[s][q]);
                    t[s] = mfma4x4(__builtin_shufflevector(wv, wv, 0, 1, 2, 3), x0, t[s]);
                    t[s] = mfma4x4(__builtin_shufflevector(wv, wv, 4, 5, 6, 7), x1, t[s]);
                }
            }
#pragma unroll
            for (int s = 0; s < kGmSets; ++s) {
                const uint16_t sb = *(const uint16_t*)(lds_scale + 2 * (lrow[s] * nblk + blk));
                gm_int4_fold(t[s], xs, bf16_bits_to_f32(sb), acc[s]);
            }
        }
    };
    // The scheduling barriers keep each chunk's loads where they are issued:
    // left free, the scheduler sinks them next to their first use (fewer live
    // registers, but one memory round trip per chunk).
#pragma unroll
    for (int c = 0; c < D && c < NCH; ++c) issue(ring[c], c);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        consume(ring[c % D], c);
        if (c + D < NCH) issue(ring[c % D], c + D);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// The rows' scales into wave-private LDS: run 0 (rows first0 ..
// first0 + n0 - 1) then run 1 (first1 ..), 16 rows in all, nblk scales of sb
// bytes each (e8m0: 1, bf16: 2), as 16-byte pieces (n0 * nblk * sb and
// 16 * nblk * sb multiples of 16).
__device__ __forceinline__ void gm_stage_scales(rsrc_t rs, int first0, int n0, int first1, int nblk, int sb,
                                                uint8_t* lds, int lane) {
    const int rb = nblk * sb, p0 = n0 * rb / 16, ptot = rb;  // 16 rows * rb / 16
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int p = lane + 64 * k;
        uint32_t so = kOob;
        if (p < p0)
            so = (uint32_t)first0 * rb + 16u * p;
        else if (p < ptot)
            so = (uint32_t)first1 * rb + 16u * (p - p0);
        const u32x4 v = bld16nt(rs, so);
        if (p < ptot) *(u32x4*)(lds + 16 * p) = v;
    }
    wave_lds_sync();
}

// This lane's block row 4 tg + (lane & 3): its pair, or -1. False when the
// token group holds no pair (rows are valid-first, so later groups neither).
__device__ __forceinline__ bool gm_rows(const MoeGemmArgs& a, int64_t row0, int tg, int r, int& pair) {
    const int P = a.T * a.topk;
    const int p = a.sorted_ids[row0 + 4 * tg + r];
    const bool ok = p >= 0 && p < P;
    pair = ok ? p : -1;
    return __builtin_amdgcn_ballot_w64(ok) != 0;
}

// Stage 1: unit u = (expert block b, gate columns i0 .. i0+7 and the matching
// up columns); the block's token groups one after another.
template <int FMT, int D, int NCH, bool EPI>
__global__ __launch_bounds__(kGmWaves * 64) __attribute__((amdgpu_waves_per_eu(FMT == kFmtMxfp4 ? 4 : 1))) void stage1_gemv_mfma_kernel(MoeGemmArgs a, int ngroups) {
    constexpr int SB = FMT == kFmtMxfp4 ? 1 : 2;  // scale bytes
    __shared__ __attribute__((aligned(16))) uint8_t lds_scale[kGmWaves][16 * 128 * SB];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int H = a.H, I = a.I, nblk = H / 32;
    const int upb = I / 8;
    const int64_t u = (int64_t)blockIdx.x * kGmWaves + wave;
    const int64_t b = u / upb;
    if (b >= a.cap / a.bm) return;
    const int64_t row0 = b * a.bm;
    if (row0 >= (int64_t)*a.num_post_pad) return;
    const int e = a.block_expert[b];
    if ((unsigned)e >= (unsigned)a.E) return;
    const int i0 = (int)(u % upb) * 8;
    const int seg = lane >> 2, r = lane & 3;
    const int64_t slab_rows = 2 * (int64_t)I;
    const rsrc_t rw = make_rsrc(a.w13 + e * slab_rows * (H / 2), (uint32_t)(slab_rows * (H / 2)));
    const rsrc_t rs = make_rsrc((const uint8_t*)a.w13_scale + e * slab_rows * nblk * SB, (uint32_t)(slab_rows * nblk * SB));
    const rsrc_t rx = make_rsrc(a.x, (uint32_t)((int64_t)a.T * H * 2));
    uint8_t* lds = lds_scale[wave];
    gm_stage_scales(rs, i0, 8, I + i0, nblk, SB, lds, lane);

    // Row slot r of set s: gate i0 + 2s + r (r < 2), up i0 + 2s + r - 2.
    uint32_t w_off[kGmSets];
    int lrow[kGmSets];
#pragma unroll
    for (int s = 0; s < kGmSets; ++s) {
        const int row = r < 2 ? i0 + 2 * s + r : I + i0 + 2 * s + (r - 2);
        w_off[s] = (uint32_t)row * (uint32_t)(H / 2) + 16u * seg;
        lrow[s] = r < 2 ? 2 * s + r : 8 + 2 * s + (r - 2);
    }
    // Lane 4c + j with c < 8 stores (token j, column i0 + 2 (c & 3) + (c >> 2)):
    // gate = row slot c >> 2, up = slot 2 + (c >> 2) of set c & 3.
    const int sel = seg & 3, half = (seg >> 2) & 1;
    const int col = i0 + 2 * sel + half;
    for (int tg = 0; tg < ngroups; ++tg) {
        int pair;
        if (!gm_rows(a, row0, tg, r, pair)) break;
        const uint32_t x_off = pair >= 0 ? (uint32_t)(pair / a.topk) * (uint32_t)(2 * H) + 64u * seg : kOob;
        f32x4 acc[kGmSets];
#pragma unroll
        for (int s = 0; s < kGmSets; ++s) acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
        gm_k_loop<FMT, D, NCH>(rw, rx, w_off, x_off, lds, lrow, nblk, seg, acc);
        gm_reduce(acc);
        float gv = 0.f, uv = 0.f;
#pragma unroll
        for (int s = 0; s < kGmSets; ++s) {
            gv = s == sel ? (half ? acc[s][1] : acc[s][0]) : gv;
            uv = s == sel ? (half ? acc[s][3] : acc[s][2]) : uv;
        }
        if (lane < 32 && pair >= 0) {
            if constexpr (EPI) {
                GluTerms glu;
                glu.load(a, e, col);
                glu.apply(gv, uv);
            }
            a.h[(int64_t)pair * I + col] = f32_to_bf16_bits(swiglu(gv, uv));
        }
    }
}

// Stage 2: unit u = (expert block b, output rows n0 .. n0+15); the block's
// token groups one after another; y by pair.
template <int FMT, int D, int NCH>
__global__ __launch_bounds__(kGmWaves * 64) __attribute__((amdgpu_waves_per_eu(FMT == kFmtMxfp4 ? 4 : 1))) void stage2_gemv_mfma_kernel(MoeGemmArgs a, int ngroups) {
    constexpr int SB = FMT == kFmtMxfp4 ? 1 : 2;  // scale bytes
    __shared__ __attribute__((aligned(16))) uint8_t lds_scale[kGmWaves][16 * 128 * SB];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int H = a.H, I = a.I, nblk = I / 32;
    const int upb = H / 16;
    const int64_t u = (int64_t)blockIdx.x * kGmWaves + wave;
    const int64_t b = u / upb;
    if (b >= a.cap / a.bm) return;
    const int64_t row0 = b * a.bm;
    if (row0 >= (int64_t)*a.num_post_pad) return;
    const int e = a.block_expert[b];
    if ((unsigned)e >= (unsigned)a.E) return;
    const int n0 = (int)(u % upb) * 16;
    const int seg = lane >> 2, r = lane & 3;
    const int P = a.T * a.topk;

    const rsrc_t rw = make_rsrc(a.w2 + (int64_t)e * H * (I / 2), (uint32_t)((int64_t)H * (I / 2)));
    const rsrc_t rs = make_rsrc((const uint8_t*)a.w2_scale + (int64_t)e * H * nblk * SB, (uint32_t)((int64_t)H * nblk * SB));
    const rsrc_t rx = make_rsrc(a.h, (uint32_t)((int64_t)P * I * 2));
    uint8_t* lds = lds_scale[wave];
    gm_stage_scales(rs, n0, 16, n0 + 16, nblk, SB, lds, lane);

    // Row slot r of set s: w2 row n0 + 4s + r.
    uint32_t w_off[kGmSets];
    int lrow[kGmSets];
#pragma unroll
    for (int s = 0; s < kGmSets; ++s) {
        w_off[s] = (uint32_t)(n0 + 4 * s + r) * (uint32_t)(I / 2) + 16u * seg;
        lrow[s] = 4 * s + r;
    }
    // Lane 4c + j stores (token j, row n0 + 4 (c & 3) + (c >> 2)).
    const int sel = seg & 3, slot = seg >> 2;
    for (int tg = 0; tg < ngroups; ++tg) {
        int pair;
        if (!gm_rows(a, row0, tg, r, pair)) break;
        const uint32_t x_off = pair >= 0 ? (uint32_t)pair * (uint32_t)(2 * I) + 64u * seg : kOob;
        f32x4 acc[kGmSets];
#pragma unroll
        for (int s = 0; s < kGmSets; ++s) acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
        gm_k_loop<FMT, D, NCH>(rw, rx, w_off, x_off, lds, lrow, nblk, seg, acc);
        gm_reduce(acc);
        float v = 0.f;
#pragma unroll
        for (int s = 0; s < kGmSets; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) v = (s == sel && i == slot) ? acc[s][i] : v;
        if (pair >= 0) a.y[(int64_t)pair * H + n0 + 4 * sel + slot] = v;
    }
}

// ---------------------------------------------------------------------------
// The same units with the block's activation rows shared by the workgroup
// (blocks of up to 16 rows: 13-16 tokens), MXFP4 or int4-g32. The four waves of a workgroup take
// four consecutive units of one block, so they need the same activations:
// each K chunk of the block's 16 rows (512 elements, 16 KB) is staged once in
// LDS by the whole workgroup (double-buffered, one barrier per chunk), and
// each wave reads its B operands from there, up to two token groups (8 rows)
// per pass over the weights. The weights keep the 4-row x 256-byte loads
// above: reading the same bytes as 16 rows x 64 bytes per instruction (the
// layout a 16x16x32 MFMA operand needs) took 230 against 177 us at 16 tokens.
constexpr int kGxRowBytes = 1024 + 16;  // one chunk of one activation row in LDS (padded)

struct GxSlot {
    u32x4 w[kGmSets];  // 16 code bytes of this lane's row in each row set
    u32x4 x[4];        // this thread's 64 bytes of the chunk's activation tile
};

// int4: held to three waves per SIMD (a few spilled registers); its own
// choice of 200 VGPRs and two waves was 4-15 % slower at 16 tokens.
template <int FMT, int STAGE, int NCH, bool EPI>
__global__ __launch_bounds__(kGmWaves * 64) __attribute__((amdgpu_waves_per_eu(FMT == kFmtMxfp4 ? 1 : 3))) void gemv_mfma_x_kernel(MoeGemmArgs a) {
    // Token groups per pass: two (MXFP4); one for int4, whose per-chunk group
    // sums take the registers of the second.
    constexpr int NTG = FMT == kFmtMxfp4 ? 2 : 1;
    constexpr int SB = FMT == kFmtMxfp4 ? 1 : 2;  // scale bytes
    __shared__ __attribute__((aligned(16))) uint8_t xs[2][16 * kGxRowBytes];
    __shared__ __attribute__((aligned(16))) uint8_t lds_scale[kGmWaves][16 * 128 * SB];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = a.H, I = a.I;
    const int K = STAGE == 1 ? H : I, nblk = K / 32;
    const int upb = STAGE == 1 ? I / 8 : H / 16;  // a multiple of kGmWaves: one block per workgroup
    const int64_t u = (int64_t)blockIdx.x * kGmWaves + wave;
    const int64_t b = u / upb;
    if (b >= a.cap / a.bm) return;  // everything below is uniform per workgroup
    const int64_t row0 = b * a.bm;
    if (row0 >= (int64_t)*a.num_post_pad) return;
    const int e = a.block_expert[b];
    if ((unsigned)e >= (unsigned)a.E) return;
    const int seg = lane >> 2, r = lane & 3;
    const int P = a.T * a.topk;
    // Rows of the block holding pairs (valid first).
    int nvalid;
    {
        const int p = a.sorted_ids[row0 + (lane & 15)];
        nvalid = __popcll(__builtin_amdgcn_ballot_w64(p >= 0 && p < P) & 0xFFFFull);
    }
    const int ngroups = (nvalid + 3) / 4;

    const int64_t slab_rows = STAGE == 1 ? 2 * (int64_t)I : (int64_t)H;
    const rsrc_t rw = make_rsrc((STAGE == 1 ? a.w13 : a.w2) + e * slab_rows * (K / 2), (uint32_t)(slab_rows * (K / 2)));
    const rsrc_t rs = make_rsrc((const uint8_t*)(STAGE == 1 ? a.w13_scale : a.w2_scale) + e * slab_rows * nblk * SB,
                                (uint32_t)(slab_rows * nblk * SB));
    const int c0 = (int)(u % upb) * (STAGE == 1 ? 8 : 16);  // stage 1: columns i0; stage 2: rows n0
    uint8_t* lds = lds_scale[wave];
    if (STAGE == 1) gm_stage_scales(rs, c0, 8, I + c0, nblk, SB, lds, lane);
    else gm_stage_scales(rs, c0, 16, c0 + 16, nblk, SB, lds, lane);
    uint32_t w_off[kGmSets];
    int lrow[kGmSets];
#pragma unroll
    for (int s = 0; s < kGmSets; ++s) {
        const int row = STAGE == 1 ? (r < 2 ? c0 + 2 * s + r : I + c0 + 2 * s + (r - 2)) : c0 + 4 * s + r;
        w_off[s] = (uint32_t)row * (uint32_t)(K / 2) + 16u * seg;
        lrow[s] = STAGE == 1 ? (r < 2 ? 2 * s + r : 8 + 2 * s + (r - 2)) : 4 * s + r;
    }
    // Activation staging: thread tid loads bytes 64 pc .. 64 pc + 63 of the
    // chunk's slice of block row mr.
    const int mr = tid >> 4, pc = tid & 15;
    uint32_t x_row = kOob;
    {
        const int p = a.sorted_ids[row0 + mr];
        if (p >= 0 && p < P) x_row = STAGE == 1 ? (uint32_t)(p / a.topk) * (uint32_t)(2 * H) : (uint32_t)p * (uint32_t)(2 * I);
    }
    const rsrc_t rx = STAGE == 1 ? make_rsrc(a.x, (uint32_t)((int64_t)a.T * H * 2))
                                 : make_rsrc(a.h, (uint32_t)((int64_t)P * I * 2));

    for (int tg0 = 0; tg0 < ngroups; tg0 += NTG) {
        GxSlot ring[2];
        // Loads of chunk c; blocks past nblk load zeros without memory traffic.
        auto issue = [&](GxSlot& sl, int c) {
            const uint32_t xo = (uint32_t)(512 * c + 32 * pc >= K) << 31;
            const uint32_t xa = (x_row + 1024u * c + 64u * pc) | xo;
#pragma unroll
            for (int k = 0; k < 4; ++k) sl.x[k] = bld16(rx, xa + 16u * k);
            const uint32_t wo = (uint32_t)(16 * c + seg >= nblk) << 31;
#pragma unroll
            for (int s = 0; s < kGmSets; ++s) sl.w[s] = bld16nt(rw, (w_off[s] + 256u * c) | wo);
        };
        f32x4 acc[NTG][kGmSets];
#pragma unroll
        for (int g = 0; g < NTG; ++g)
#pragma unroll
            for (int s = 0; s < kGmSets; ++s) acc[g][s] = f32x4{0.f, 0.f, 0.f, 0.f};
        const bool two = tg0 + 1 < ngroups;  // uniform: the pass's second token group holds rows
#pragma unroll
        for (int c = 0; c < 2 && c < NCH; ++c) issue(ring[c], c);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            GxSlot& sl = ring[c & 1];
            uint8_t* xb = xs[c & 1];
#pragma unroll
            for (int k = 0; k < 4; ++k) *(u32x4*)(xb + mr * kGxRowBytes + 64 * pc + 16 * k) = sl.x[k];
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            const int blk = min(16 * c + seg, nblk - 1);
            if constexpr (FMT == kFmtMxfp4) {
                float sc[kGmSets];
#pragma unroll
                for (int s = 0; s < kGmSets; ++s) sc[s] = e8m0_scale_operand(lds[lrow[s] * nblk + blk]);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    bf16x8 wv[kGmSets];
#pragma unroll
                    for (int s = 0; s < kGmSets; ++s) wv[s] = mxfp4x8_to_bf16(sl.w[s][q], sc[s]);
#pragma unroll
                    for (int g = 0; g < NTG; ++g) {
                        if (g == 1 && !two) break;
                        // Token 4 (tg0 + g) + r, elements 8q .. 8q + 7 of K segment seg.
                        const bf16x8 xv = *(const bf16x8*)(xb + (4 * (tg0 + g) + r) * kGxRowBytes + 64 * seg + 16 * q);
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const bf16x4_t xh = h ? __builtin_shufflevector(xv, xv, 4, 5, 6, 7)
                                                  : __builtin_shufflevector(xv, xv, 0, 1, 2, 3);
#pragma unroll
                            for (int s = 0; s < kGmSets; ++s) {
                                const bf16x4_t wb = h ? __builtin_shufflevector(wv[s], wv[s], 4, 5, 6, 7)
                                                      : __builtin_shufflevector(wv[s], wv[s], 0, 1, 2, 3);
                                acc[g][s] = mfma4x4(wb, xh, acc[g][s]);
                            }
                        }
                    }
                }
            } else {  // int4-g32, one token group: fold the chunk per group (gm_int4_fold)
                const bf16x4_t ones = __builtin_bit_cast(bf16x4_t, u32x2{0x3F803F80u, 0x3F803F80u});
                f32x4 t[kGmSets], xsum = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < kGmSets; ++s) t[s] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const bf16x8 xv =
                        perm_x_int4(*(const bf16x8*)(xb + (4 * tg0 + r) * kGxRowBytes + 64 * seg + 16 * q));
                    const bf16x4_t x0 = __builtin_shufflevector(xv, xv, 0, 1, 2, 3);
                    const bf16x4_t x1 = __builtin_shufflevector(xv, xv, 4, 5, 6, 7);
                    xsum = mfma4x4(ones, x0, xsum);
                    xsum = mfma4x4(ones, x1, xsum);
#pragma unroll
                    for (int s = 0; s < kGmSets; ++s) {
                        const bf16x8 wv = int4x8_to_bf16_biased(sl.w[s][q]);
                        t[s] = mfma4x4(__builtin_shufflevector(wv, wv, 0, 1, 2, 3), x0, t[s]);
                        t[s] = mfma4x4(__builtin_shufflevector(wv, wv, 4, 5, 6, 7), x1, t[s]);
                    }
                }
#pragma unroll
                for (int s = 0; s < kGmSets; ++s) {
                    const uint16_t sb = *(const uint16_t*)(lds + 2 * (lrow[s] * nblk + blk));
                    gm_int4_fold(t[s], xsum, bf16_bits_to_f32(sb), acc[0][s]);
                }
            }
            if (c + 2 < NCH) issue(sl, c + 2);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int g = 0; g < NTG; ++g) {
            if (g == 1 && !two) break;
            gm_reduce(acc[g]);
            const int m = 4 * (tg0 + g) + r;
            const int pr = a.sorted_ids[row0 + m];
            const bool ok = pr >= 0 && pr < P;
            if constexpr (STAGE == 1) {
                // Lane 4c + j with c < 8 stores (token j, column i0 + 2 (c & 3) + (c >> 2)).
                const int sel = seg & 3, half = (seg >> 2) & 1;
                const int col = c0 + 2 * sel + half;
                float gv = 0.f, uv = 0.f;
#pragma unroll
                for (int s = 0; s < kGmSets; ++s) {
                    gv = s == sel ? (half ? acc[g][s][1] : acc[g][s][0]) : gv;
                    uv = s == sel ? (half ? acc[g][s][3] : acc[g][s][2]) : uv;
                }
                if (lane < 32 && ok) {
                    if constexpr (EPI) {
                        GluTerms glu;
                        glu.load(a, e, col);
                        glu.apply(gv, uv);
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
                    for (int i = 0; i < 4; ++i) v = (s == sel && i == slot) ? acc[g][s][i] : v;
                if (ok) a.y[(int64_t)pr * H + c0 + 4 * sel + slot] = v;
            }
        }
        __syncthreads();  // the next pass rewrites both activation buffers
    }
}

bool gemv_mfma_eligible(const MoeGemmArgs& a) {
    return (a.fmt == kFmtMxfp4 || a.fmt == kFmtInt4g32) && a.bm == 16 && a.H <= 4096 && a.I <= 4096 && a.H % 64 == 0 &&
           a.I % 64 == 0 && (int64_t)a.T * a.topk * a.I * 2 < 0x7fff0000LL &&
           (int64_t)a.T * a.H * 2 < 0x7fff0000LL;
}

// Chunks in flight per wave: two, with four waves per SIMD (127 VGPRs, no
// spill). Three chunks with two waves per SIMD were 9-10 % slower at 4 tokens.
constexpr int kGmDepth = 2;

template <int FMT, int NCH>
static void launch_gm_nch(const MoeGemmArgs& a, int stage, int ngroups, dim3 grid, dim3 block, hipStream_t s) {
    const bool epi = a.w13_bias || a.swiglu_limit > 0.0f;
    if (stage == 1) {
        if (epi) hipLaunchKernelGGL((stage1_gemv_mfma_kernel<FMT, kGmDepth, NCH, true>), grid, block, 0, s, a, ngroups);
        else hipLaunchKernelGGL((stage1_gemv_mfma_kernel<FMT, kGmDepth, NCH, false>), grid, block, 0, s, a, ngroups);
    } else {
        hipLaunchKernelGGL((stage2_gemv_mfma_kernel<FMT, kGmDepth, NCH>), grid, block, 0, s, a, ngroups);
    }
}

template <int NCH>
static void launch_gm_nch(const MoeGemmArgs& a, int stage, int ngroups, dim3 grid, dim3 block, hipStream_t s) {
    if (a.fmt == kFmtMxfp4) launch_gm_nch<kFmtMxfp4, NCH>(a, stage, ngroups, grid, block, s);
    else launch_gm_nch<kFmtInt4g32, NCH>(a, stage, ngroups, grid, block, s);
}

template <int FMT, int NCH>
static void launch_gx_nch(const MoeGemmArgs& a, int stage, dim3 grid, dim3 block, hipStream_t s) {
    if (stage == 1) {
        if (a.w13_bias || a.swiglu_limit > 0.0f) hipLaunchKernelGGL((gemv_mfma_x_kernel<FMT, 1, NCH, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((gemv_mfma_x_kernel<FMT, 1, NCH, false>), grid, block, 0, s, a);
    } else {
        hipLaunchKernelGGL((gemv_mfma_x_kernel<FMT, 2, NCH, false>), grid, block, 0, s, a);
    }
}

template <int NCH>
static void launch_gx_nch(const MoeGemmArgs& a, int stage, dim3 grid, dim3 block, hipStream_t s) {
    if (a.fmt == kFmtMxfp4) launch_gx_nch<kFmtMxfp4, NCH>(a, stage, grid, block, s);
    else launch_gx_nch<kFmtInt4g32, NCH>(a, stage, grid, block, s);
}

hipError_t launch_gemv_mfma_x_stage(const MoeGemmArgs& a, int stage, hipStream_t s) {
    const int64_t nb = a.cap / a.bm;
    const int64_t units = nb * (stage == 1 ? a.I / 8 : a.H / 16);
    const dim3 grid((unsigned)(units / kGmWaves)), block(kGmWaves * 64);
    const int nch = ((stage == 1 ? a.H : a.I) / 32 + 15) / 16;  // 1..8 (K <= 4096)
    switch (nch) {
        case 1: launch_gx_nch<1>(a, stage, grid, block, s); break;
        case 2: launch_gx_nch<2>(a, stage, grid, block, s); break;
        case 3: launch_gx_nch<3>(a, stage, grid, block, s); break;
        case 4: launch_gx_nch<4>(a, stage, grid, block, s); break;
        case 5: launch_gx_nch<5>(a, stage, grid, block, s); break;
        case 6: launch_gx_nch<6>(a, stage, grid, block, s); break;
        case 7: launch_gx_nch<7>(a, stage, grid, block, s); break;
        default: launch_gx_nch<8>(a, stage, grid, block, s); break;
    }
    return hipGetLastError();
}

hipError_t launch_gemv_mfma_stage(const MoeGemmArgs& a, int stage, hipStream_t s) {
    const int64_t nb = a.cap / a.bm;
    const int64_t units = nb * (stage == 1 ? a.I / 8 : a.H / 16);
    const int rows = a.T < a.bm ? a.T : a.bm;
    const int ngroups = (rows + 3) / 4;  // 1..4 token groups of 4 rows
    const dim3 grid((unsigned)((units + kGmWaves - 1) / kGmWaves)), block(kGmWaves * 64);
    const int nch = ((stage == 1 ? a.H : a.I) / 32 + 15) / 16;  // 1..8 (K <= 4096)
    switch (nch) {
        case 1: launch_gm_nch<1>(a, stage, ngroups, grid, block, s); break;
        case 2: launch_gm_nch<2>(a, stage, ngroups, grid, block, s); break;
        case 3: launch_gm_nch<3>(a, stage, ngroups, grid, block, s); break;
        case 4: launch_gm_nch<4>(a, stage, ngroups, grid, block, s); break;
        case 5: launch_gm_nch<5>(a, stage, ngroups, grid, block, s); break;
        case 6: launch_gm_nch<6>(a, stage, ngroups, grid, block, s); break;
        case 7: launch_gm_nch<7>(a, stage, ngroups, grid, block, s); break;
        default: launch_gm_nch<8>(a, stage, ngroups, grid, block, s); break;
    }
    return hipGetLastError();
}

}  // namespace moe

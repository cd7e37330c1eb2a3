// Decode grouped GEMMs: one wave per output tile, weights streamed from HBM
// through a register ring.
//
// At decode token counts an expert block holds at most 32 rows, the layer
// reads every touched weight byte exactly once, and the kernels are HBM
// bound. The design follows from keeping enough bytes in flight:
//
//  * one wave owns one output tile over the whole K: stage 1 takes 16 gate
//    rows and the matching 16 up rows (so SwiGLU happens in registers), stage
//    2 takes 32 rows of w2. No LDS, no barriers, no cross-wave reduction, and
//    every wave of the grid streams independently;
//  * each lane loads 16 bytes of one weight row per step (32 e2m1 codes = one
//    MX block with one e8m0 byte); the four lane groups take four consecutive
//    blocks, so a wave reads 64 contiguous bytes of each of its rows per step;
//  * the activation fragments of a step are loaded together with its weights
//    into the same ring slot, D steps ahead. Vector-memory loads complete in
//    order, so an activation load issued later than the weight prefetches
//    would force waiting for all of them; issuing both together keeps D steps
//    of weights in flight per wave;
//  * decoding uses the gfx950 scaled fp4 -> bf16 converts (exact), and the
//    MFMA is v_mfma_f32_16x16x32_bf16 with the activations as the A operand
//    (row = lane % 16) and the weights as B. Inside one MFMA the K order is a
//    permutation shared by both operands: lane group g holds block 4s+g and
//    MFMA q takes elements 8q..8q+7 of it.
//
// int4-g32 weights: lane group g loads dword g of four consecutive 32-groups
// so that MFMA q spans exactly group q; its fp32 result is multiplied by the
// group's bf16 scale (exact, no bf16 rounding of code * scale). Codes enter
// as code + 136 (built from the nibbles with two bit operations) and
// 136 * sum(x over the group), from an MFMA against ones, is subtracted.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kUnitWaves = 4;        // waves (= units) per workgroup
constexpr int kRing = 4;             // K steps in flight per wave
constexpr uint32_t kOob = 0x80000000u;  // buffer offset past every record: loads 0, no traffic

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bld16(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// One wave's operands: two 16-row weight tiles of one expert (this lane's
// row in each), their scales, and up to MSUB activation rows. Offsets are
// bytes inside the buffer resources; kOob marks a row without data.
template <int MSUB>
struct UnitOperands {
    rsrc_t w, s, x;
    uint32_t w_off[2], s_off[2];
    uint32_t x_off[MSUB];
};

template <int FMT, int MSUB>
struct RingSlot {
    u32x4 w[2];              // two weight row-tiles (stage 1: gate, up)
    uint32_t s[2][2];        // MXFP4: e8m0 byte in s[t][0]; INT4: 4 bf16 scales
    u32x4 x[MSUB][4];        // activation fragments per 16-row sub-tile
};

// One wave: acc0/acc1[s] += A_s . B_t over all of K.
template <int FMT, int MSUB>
__device__ __forceinline__ void unit_k_loop(const UnitOperands<MSUB>& o, int nact, int K, int g,
                                            f32x4 (&acc0)[MSUB], f32x4 (&acc1)[MSUB]) {
    const int nblk = K / 32;
    const int niter = (nblk + 3) / 4;
    RingSlot<FMT, MSUB> ring[kRing];

    // Every load is unconditional; a row without data or a K block past the
    // end uses an out-of-range buffer offset and reads zeros without memory
    // traffic. No per-lane control flow reaches the loads, so the compiler
    // keeps the whole ring in flight.
    auto issue = [&](RingSlot<FMT, MSUB>& r, int it) {
        if constexpr (FMT == kFmtMxfp4) {
            const int blk = 4 * it + g;
            const bool ok = blk < nblk;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                r.w[t] = bld16(o.w, ok ? o.w_off[t] + 16u * blk : kOob);
                r.s[t][0] = __builtin_amdgcn_raw_buffer_load_b8(o.s, ok ? o.s_off[t] + blk : kOob, 0, 0);
            }
#pragma unroll
            for (int s = 0; s < MSUB; ++s) {
                const uint32_t xo = ok ? o.x_off[s] + 64u * blk : kOob;
#pragma unroll
                for (int q = 0; q < 4; ++q) r.x[s][q] = bld16(o.x, xo + 16u * q);
            }
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int grp = 4 * it + q;
                const bool ok = grp < nblk;
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    r.w[t][q] = __builtin_amdgcn_raw_buffer_load_b32(o.w, ok ? o.w_off[t] + 16u * grp + 4u * g : kOob, 0, 0);
                    const uint32_t sc = __builtin_amdgcn_raw_buffer_load_b16(o.s, ok ? o.s_off[t] + 2u * grp : kOob, 0, 0);
                    if (q & 1)
                        r.s[t][q >> 1] |= sc << 16;
                    else
                        r.s[t][q >> 1] = sc;
                }
#pragma unroll
                for (int s = 0; s < MSUB; ++s)
                    r.x[s][q] = bld16(o.x, ok ? o.x_off[s] + 64u * grp + 16u * g : kOob);
            }
        }
    };

    auto consume = [&](RingSlot<FMT, MSUB>& r) {
        if constexpr (FMT == kFmtMxfp4) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const float sc = e8m0_scale_operand(r.s[t][0]);
                bf16x8 bw[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) bw[q] = mxfp4x8_to_bf16(r.w[t][q], sc);
#pragma unroll
                for (int s = 0; s < MSUB; ++s) {
                    if (s >= nact) break;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const bf16x8 xa = __builtin_bit_cast(bf16x8, r.x[s][q]);
                        if (t == 0)
                            acc0[s] = mfma16x16x32(xa, bw[q], acc0[s]);
                        else
                            acc1[s] = mfma16x16x32(xa, bw[q], acc1[s]);
                    }
                }
            }
        } else {
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
#pragma unroll
            for (int s = 0; s < MSUB; ++s) {
                if (s >= nact) break;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const bf16x8 xa = perm_x_int4(__builtin_bit_cast(bf16x8, r.x[s][q]));
                    const f32x4 xs = mfma16x16x32(xa, ones, zero);
                    const f32x4 t0 = mfma16x16x32(xa, int4x8_to_bf16_biased(r.w[0][q]), zero);
                    const f32x4 t1 = mfma16x16x32(xa, int4x8_to_bf16_biased(r.w[1][q]), zero);
                    const float sc0 = bf16_bits_to_f32((r.s[0][q >> 1] >> (16 * (q & 1))) & 0xFFFFu);
                    const float sc1 = bf16_bits_to_f32((r.s[1][q >> 1] >> (16 * (q & 1))) & 0xFFFFu);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        acc0[s][j] = fmaf(fmaf(-136.0f, xs[j], t0[j]), sc0, acc0[s][j]);
                        acc1[s][j] = fmaf(fmaf(-136.0f, xs[j], t1[j]), sc1, acc1[s][j]);
                    }
                }
            }
        }
    };

    // Straight-line ring: each round consumes kRing steps and refills every
    // slot kRing steps ahead (steps past the end load zeros for free), so
    // the loop body has no branches and wait counts stay partial.
#pragma unroll
    for (int d = 0; d < kRing; ++d) issue(ring[d], d);
    for (int base = 0; base < niter; base += kRing) {
#pragma unroll
        for (int d = 0; d < kRing; ++d) {
            consume(ring[d]);
            issue(ring[d], base + d + kRing);
        }
    }
}

// Stage 1 (gate_up + SwiGLU). Unit u = (block b, 16-column slice of I).
template <int FMT, int MSUB>
__global__ __launch_bounds__(kUnitWaves * 64) void stage1_unit_kernel(MoeGemmArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int upb = a.I / 16;
    const int64_t u = (int64_t)blockIdx.x * kUnitWaves + wave;
    const int64_t b = u / upb;
    if (b >= a.cap / a.bm) return;
    const int bm = a.bm;
    const int64_t row0 = b * bm;
    if (row0 >= (int64_t)*a.num_post_pad) return;
    const int e = a.block_expert[b];
    if (e < 0 || e >= a.E) return;
    const int i0 = (int)(u % upb) * 16;
    const int nl = lane & 15, g = lane >> 4;
    const int H = a.H, I = a.I, P = a.T * a.topk;
    const int sb = FMT == kFmtMxfp4 ? 1 : 2;  // bytes per scale

    UnitOperands<MSUB> o;
    int valid[MSUB];
    int nact = 0;
#pragma unroll
    for (int s = 0; s < MSUB; ++s) {
        const int p = a.sorted_ids[row0 + 16 * s + nl];
        const bool ok = p >= 0 && p < P;
        o.x_off[s] = ok ? (uint32_t)(p / a.topk) * (uint32_t)(2 * H) : kOob;
        const uint64_t m = __ballot(ok) & 0xFFFFull;
        valid[s] = __popcll(m);
        if (m) nact = s + 1;
    }
    const int64_t slab_rows = 2 * (int64_t)I;  // w13 rows of one expert
    o.w = make_rsrc(a.w13 + e * slab_rows * (H / 2), (uint32_t)(slab_rows * (H / 2)));
    o.s = make_rsrc((const uint8_t*)a.w13_scale + e * slab_rows * (H / 32) * sb,
                    (uint32_t)(slab_rows * (H / 32) * sb));
    o.x = make_rsrc(a.x, (uint32_t)((int64_t)a.T * H * 2));
    o.w_off[0] = (uint32_t)(i0 + nl) * (uint32_t)(H / 2);
    o.w_off[1] = (uint32_t)(I + i0 + nl) * (uint32_t)(H / 2);
    o.s_off[0] = (uint32_t)(i0 + nl) * (uint32_t)(H / 32 * sb);
    o.s_off[1] = (uint32_t)(I + i0 + nl) * (uint32_t)(H / 32 * sb);

    f32x4 accg[MSUB], accu[MSUB];
#pragma unroll
    for (int s = 0; s < MSUB; ++s) accg[s] = accu[s] = f32x4{0.f, 0.f, 0.f, 0.f};
    unit_k_loop<FMT, MSUB>(o, nact, H, g, accg, accu);

    // C layout: this lane holds rows 4g + j, column nl.
#pragma unroll
    for (int s = 0; s < MSUB; ++s) {
        if (s >= nact) break;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = 4 * g + j;
            if (m < valid[s])
                a.h[(row0 + 16 * s + m) * I + i0 + nl] = f32_to_bf16_bits(swiglu(accg[s][j], accu[s][j]));
        }
    }
}

// Stage 2 (down). Unit u = (block b, 32-row slice of H).
template <int FMT, int MSUB>
__global__ __launch_bounds__(kUnitWaves * 64) void stage2_unit_kernel(MoeGemmArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int upb = a.H / 32;
    const int64_t u = (int64_t)blockIdx.x * kUnitWaves + wave;
    const int64_t b = u / upb;
    if (b >= a.cap / a.bm) return;
    const int bm = a.bm;
    const int64_t row0 = b * bm;
    if (row0 >= (int64_t)*a.num_post_pad) return;
    const int e = a.block_expert[b];
    if (e < 0 || e >= a.E) return;
    const int n0 = (int)(u % upb) * 32;
    const int nl = lane & 15, g = lane >> 4;
    const int H = a.H, I = a.I, P = a.T * a.topk;
    const int sb = FMT == kFmtMxfp4 ? 1 : 2;

    UnitOperands<MSUB> o;
    int nact = 0;
#pragma unroll
    for (int s = 0; s < MSUB; ++s) {
        const int64_t r = row0 + 16 * s + nl;
        const int p = a.sorted_ids[r];
        const bool ok = p >= 0 && p < P;
        o.x_off[s] = ok ? (uint32_t)r * (uint32_t)(2 * I) : kOob;
        if (__ballot(ok)) nact = s + 1;
    }
    o.w = make_rsrc(a.w2 + (int64_t)e * H * (I / 2), (uint32_t)((int64_t)H * (I / 2)));
    o.s = make_rsrc((const uint8_t*)a.w2_scale + (int64_t)e * H * (I / 32) * sb,
                    (uint32_t)((int64_t)H * (I / 32) * sb));
    o.x = make_rsrc(a.h, (uint32_t)(a.cap * I * 2));
    o.w_off[0] = (uint32_t)(n0 + nl) * (uint32_t)(I / 2);
    o.w_off[1] = (uint32_t)(n0 + 16 + nl) * (uint32_t)(I / 2);
    o.s_off[0] = (uint32_t)(n0 + nl) * (uint32_t)(I / 32 * sb);
    o.s_off[1] = (uint32_t)(n0 + 16 + nl) * (uint32_t)(I / 32 * sb);

    f32x4 acc0[MSUB], acc1[MSUB];
#pragma unroll
    for (int s = 0; s < MSUB; ++s) acc0[s] = acc1[s] = f32x4{0.f, 0.f, 0.f, 0.f};
    unit_k_loop<FMT, MSUB>(o, nact, I, g, acc0, acc1);

#pragma unroll
    for (int s = 0; s < MSUB; ++s) {
        if (s >= nact) break;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int p = a.sorted_ids[row0 + 16 * s + 4 * g + j];
            if (p >= 0 && p < P) {
                float* yr = a.y + (int64_t)p * H + n0 + nl;
                yr[0] = acc0[s][j];
                yr[16] = acc1[s][j];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// GEMV-shaped decode kernels for blocks with at most NR (<= 4) token rows.
//
// With one or a few activation rows per expert block, 15/16 of every MFMA
// would be idle and the MFMA operand layout (16 rows x 64 bytes per load)
// costs one memory instruction per 64 bytes of each row. Here a wave owns RPW
// weight rows over the whole K instead:
//  * each load instruction reads 1 KB contiguous of one row (lane l holds MX
//    block 64c + l of chunk c), and every weight load of the wave is issued
//    up front, so a wave is one memory round trip;
//  * the e8m0 scales of the wave's rows arrive with a few dword loads into
//    wave-private LDS (one byte per lane per row would cost as many memory
//    instructions as the weights themselves);
//  * a lane decodes its block with the scaled fp4 -> bf16 converts and
//    accumulates v_dot2_f32_bf16 against the matching 32 activations per
//    token row; row sums meet across the wave with permlane32/16 swaps and
//    DPP row rotations (no LDS, no shuffles through memory).
// Stage 1 takes RPW/2 gate rows and the RPW/2 matching up rows so SwiGLU is
// applied in registers after the reduction.
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float ror_add(float v) {
    return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of each DPP row; every lane of the row gets the sum.
__device__ __forceinline__ float row16_sum(float v) {
    v = ror_add<0x128>(v);  // row_ror:8
    v = ror_add<0x124>(v);  // row_ror:4
    v = ror_add<0x122>(v);  // row_ror:2
    v = ror_add<0x121>(v);  // row_ror:1
    return v;
}

// v_permlane32_swap a, b exchanges lanes 32..63 of a with lanes 0..31 of b
// (v_permlane16_swap: the odd 16-lane rows of a with the even rows of b).
// Issued as inline asm with both registers read-write: the compiler's
// two-result builtin lost its second result when both were summed. The
// s_nop covers the VALU-write -> permlane-read hazard.
__device__ __forceinline__ float swap32_add(float a, float b) {
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
    return a + b;
}
__device__ __forceinline__ float swap16_add(float a, float b) {
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
    return a + b;
}

// Reduce 8 per-lane partials v[0..7] over the wave. Afterwards, in q0 the
// 16-lane row rho holds the total of v[sig(rho)] and in q1 of v[4 + sig(rho)],
// sig = (0, 2, 1, 3).
__device__ __forceinline__ void reduce8(const float (&v)[8], float& q0, float& q1) {
    const float r01 = swap32_add(v[0], v[1]);
    const float r23 = swap32_add(v[2], v[3]);
    const float r45 = swap32_add(v[4], v[5]);
    const float r67 = swap32_add(v[6], v[7]);
    q0 = row16_sum(swap16_add(r01, r23));
    q1 = row16_sum(swap16_add(r45, r67));
}

template <int FMT, int NR, int RPW, int NCH>
struct GemvTile {
    static_assert(RPW == 8, "the reduction handles 8 rows per wave");
    // acc[r][m]: partial dot of weight row r with token row m.
    float acc[RPW][NR];

    __device__ __forceinline__ void run(rsrc_t rw, const uint32_t (&w_off)[RPW], rsrc_t rs,
                                        const uint32_t (&s_off)[RPW], rsrc_t rx,
                                        const uint32_t (&x_off)[NR], int nvalid, int K,
                                        uint8_t* lds_scale, int lane) {
        const int nblk = K / 32;
        // Activations first: they are the oldest loads, so waiting for them
        // never waits for the weight stream issued after.
        u32x4 xr[NR][NCH][4];
#pragma unroll
        for (int m = 0; m < NR; ++m)
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int blk = 64 * c + lane;
                const uint32_t o = (m < nvalid && blk < nblk) ? x_off[m] + 64u * blk : kOob;
#pragma unroll
                for (int q = 0; q < 4; ++q) xr[m][c][q] = bld16(rx, o + 16u * q);
            }
        // Scales of the RPW rows: rows r and r+1 are adjacent in memory for
        // the row sets used here (pairs of consecutive rows), so each row's
        // nblk bytes are fetched as dwords into wave-private LDS.
        uint32_t sv[RPW * ((NCH * 64 / 4 + 63) / 64)];
        constexpr int DW_PER_LANE = (NCH * 64 / 4 + 63) / 64;  // dwords per lane per row
#pragma unroll
        for (int r = 0; r < RPW; ++r)
#pragma unroll
            for (int j = 0; j < DW_PER_LANE; ++j) {
                const int dw = lane + 64 * j;
                sv[r * DW_PER_LANE + j] = __builtin_amdgcn_raw_buffer_load_b32(
                    rs, 4 * dw < nblk ? s_off[r] + 4u * dw : kOob, 0, 0);
            }
        // The weight stream: RPW x NCH loads of 1 KB each.
        u32x4 w[RPW][NCH];
#pragma unroll
        for (int r = 0; r < RPW; ++r)
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int blk = 64 * c + lane;
                w[r][c] = bld16(rw, blk < nblk ? w_off[r] + 16u * blk : kOob);
            }
        // Stage the scale bytes: row r occupies lds_scale[r * 64 * NCH ...].
#pragma unroll
        for (int r = 0; r < RPW; ++r)
#pragma unroll
            for (int j = 0; j < DW_PER_LANE; ++j) {
                const int dw = lane + 64 * j;
                if (4 * dw < 64 * NCH) *(uint32_t*)(lds_scale + r * 64 * NCH + 4 * dw) = sv[r * DW_PER_LANE + j];
            }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

#pragma unroll
        for (int r = 0; r < RPW; ++r)
#pragma unroll
            for (int m = 0; m < NR; ++m) acc[r][m] = 0.0f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int blk = 64 * c + lane;
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
                if constexpr (FMT == kFmtMxfp4) {
                    const uint32_t e = blk < nblk ? lds_scale[r * 64 * NCH + blk] : 127u;
                    const float sc = e8m0_scale_operand(e);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        // bf16 pairs are taken with shufflevector: going through
                        // a u32x4 bit_cast and an element index here was folded
                        // to element 0 by the compiler.
                        const bf16x8 wv = mxfp4x8_to_bf16(w[r][c][q], sc);
#pragma unroll
                        for (int m = 0; m < NR; ++m) {
                            if (m >= nvalid) break;
                            const bf16x8 xv = __builtin_bit_cast(bf16x8, xr[m][c][q]);
                            acc[r][m] = __builtin_amdgcn_fdot2_f32_bf16(
                                __builtin_shufflevector(wv, wv, 0, 1), __builtin_shufflevector(xv, xv, 0, 1),
                                acc[r][m], false);
                            acc[r][m] = __builtin_amdgcn_fdot2_f32_bf16(
                                __builtin_shufflevector(wv, wv, 2, 3), __builtin_shufflevector(xv, xv, 2, 3),
                                acc[r][m], false);
                            acc[r][m] = __builtin_amdgcn_fdot2_f32_bf16(
                                __builtin_shufflevector(wv, wv, 4, 5), __builtin_shufflevector(xv, xv, 4, 5),
                                acc[r][m], false);
                            acc[r][m] = __builtin_amdgcn_fdot2_f32_bf16(
                                __builtin_shufflevector(wv, wv, 6, 7), __builtin_shufflevector(xv, xv, 6, 7),
                                acc[r][m], false);
                        }
                    }
                }
            }
        }
    }
};

// Stage 1 GEMV: unit = (block b, 4 consecutive columns i0..i0+3 of I): the
// wave reads gate rows i0..i0+3 and up rows I+i0..I+i0+3.
template <int FMT, int NR, int NCH>
__global__ __launch_bounds__(kUnitWaves * 64) void stage1_gemv_kernel(MoeGemmArgs a) {
    constexpr int RPW = 8;
    __shared__ uint8_t lds_scale[kUnitWaves][RPW * 64 * NCH];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int upb = a.I / 4;
    const int64_t u = (int64_t)blockIdx.x * kUnitWaves + wave;
    const int64_t b = u / upb;
    if (b >= a.cap / a.bm) return;
    const int64_t row0 = b * a.bm;
    if (row0 >= (int64_t)*a.num_post_pad) return;
    const int e = a.block_expert[b];
    if (e < 0 || e >= a.E) return;
    const int i0 = (int)(u % upb) * 4;
    const int H = a.H, I = a.I, P = a.T * a.topk;

    // Token rows of the block (a prefix of at most NR valid rows).
    uint32_t x_off[NR];
    int nvalid = 0;
#pragma unroll
    for (int m = 0; m < NR; ++m) {
        const int p = a.sorted_ids[row0 + m];
        const bool ok = m < a.bm && p >= 0 && p < P;
        x_off[m] = ok ? (uint32_t)(p / a.topk) * (uint32_t)(2 * H) : kOob;
        nvalid += ok ? 1 : 0;
    }
    const int64_t slab_rows = 2 * (int64_t)I;
    const rsrc_t rw = make_rsrc(a.w13 + e * slab_rows * (H / 2), (uint32_t)(slab_rows * (H / 2)));
    const rsrc_t rs = make_rsrc((const uint8_t*)a.w13_scale + e * slab_rows * (H / 32),
                                (uint32_t)(slab_rows * (H / 32)));
    const rsrc_t rx = make_rsrc(a.x, (uint32_t)((int64_t)a.T * H * 2));
    uint32_t w_off[RPW], s_off[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        const int row = r < 4 ? i0 + r : I + i0 + (r - 4);
        w_off[r] = (uint32_t)row * (uint32_t)(H / 2);
        s_off[r] = (uint32_t)row * (uint32_t)(H / 32);
    }
    GemvTile<FMT, NR, RPW, NCH> t;
    t.run(rw, w_off, rs, s_off, rx, x_off, nvalid, H, lds_scale[wave], lane);

    // Rows 0..3 gate, 4..7 up: after reduce8, 16-lane row rho holds gate and
    // up of column i0 + sig(rho) in q0 / q1.
    const int rho = lane >> 4;
    const int col = i0 + ((rho == 1) ? 2 : (rho == 2) ? 1 : rho);
#pragma unroll
    for (int m = 0; m < NR; ++m) {
        if (m >= nvalid) break;
        float v[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) v[r] = t.acc[r][m];
        float gsum, usum;
        reduce8(v, gsum, usum);
        if ((lane & 15) == 0) a.h[(row0 + m) * I + col] = f32_to_bf16_bits(swiglu(gsum, usum));
    }
}

// Stage 2 GEMV: unit = (block b, 8 consecutive rows n0..n0+7 of w2).
template <int FMT, int NR, int NCH>
__global__ __launch_bounds__(kUnitWaves * 64) void stage2_gemv_kernel(MoeGemmArgs a) {
    constexpr int RPW = 8;
    __shared__ uint8_t lds_scale[kUnitWaves][RPW * 64 * NCH];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int upb = a.H / 8;
    const int64_t u = (int64_t)blockIdx.x * kUnitWaves + wave;
    const int64_t b = u / upb;
    if (b >= a.cap / a.bm) return;
    const int64_t row0 = b * a.bm;
    if (row0 >= (int64_t)*a.num_post_pad) return;
    const int e = a.block_expert[b];
    if (e < 0 || e >= a.E) return;
    const int n0 = (int)(u % upb) * 8;
    const int H = a.H, I = a.I, P = a.T * a.topk;

    uint32_t x_off[NR];
    int pair[NR];
    int nvalid = 0;
#pragma unroll
    for (int m = 0; m < NR; ++m) {
        const int p = a.sorted_ids[row0 + m];
        const bool ok = m < a.bm && p >= 0 && p < P;
        x_off[m] = ok ? (uint32_t)(row0 + m) * (uint32_t)(2 * I) : kOob;
        pair[m] = p;
        nvalid += ok ? 1 : 0;
    }
    const rsrc_t rw = make_rsrc(a.w2 + (int64_t)e * H * (I / 2), (uint32_t)((int64_t)H * (I / 2)));
    const rsrc_t rs = make_rsrc((const uint8_t*)a.w2_scale + (int64_t)e * H * (I / 32),
                                (uint32_t)((int64_t)H * (I / 32)));
    const rsrc_t rx = make_rsrc(a.h, (uint32_t)(a.cap * I * 2));
    uint32_t w_off[RPW], s_off[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        w_off[r] = (uint32_t)(n0 + r) * (uint32_t)(I / 2);
        s_off[r] = (uint32_t)(n0 + r) * (uint32_t)(I / 32);
    }
    GemvTile<FMT, NR, RPW, NCH> t;
    t.run(rw, w_off, rs, s_off, rx, x_off, nvalid, I, lds_scale[wave], lane);

    const int rho = lane >> 4;
    const int sig = (rho == 1) ? 2 : (rho == 2) ? 1 : rho;
#pragma unroll
    for (int m = 0; m < NR; ++m) {
        if (m >= nvalid) break;
        float v[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) v[r] = t.acc[r][m];
        float q0, q1;
        reduce8(v, q0, q1);
        if ((lane & 15) == 0) {
            float* yr = a.y + (int64_t)pair[m] * H + n0;
            yr[sig] = q0;
            yr[4 + sig] = q1;
        }
    }
}

// GEMV path: MXFP4 weights, blocks of at most 4 token rows, K up to 4096.
static bool gemv_eligible(const MoeGemmArgs& a) {
    const int max_rows = a.T < a.bm ? a.T : a.bm;
    return a.fmt == kFmtMxfp4 && max_rows <= 4 && a.H <= 4096 && a.I <= 4096 &&
           (a.H / 32) % 4 == 0 && (a.I / 32) % 4 == 0 && a.I % 4 == 0 && a.H % 8 == 0;
}

template <int NR>
static hipError_t launch_gemv_nr(const MoeGemmArgs& a, int stage, hipStream_t s) {
    const int64_t nb = a.cap / a.bm;
    const int64_t units = nb * (stage == 1 ? a.I / 4 : a.H / 8);
    const dim3 grid((unsigned)((units + kUnitWaves - 1) / kUnitWaves)), block(kUnitWaves * 64);
    const int K = stage == 1 ? a.H : a.I;
    const int nch = (K / 32 + 63) / 64;
    if (stage == 1) {
        if (nch == 1) hipLaunchKernelGGL((stage1_gemv_kernel<kFmtMxfp4, NR, 1>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((stage1_gemv_kernel<kFmtMxfp4, NR, 2>), grid, block, 0, s, a);
    } else {
        if (nch == 1) hipLaunchKernelGGL((stage2_gemv_kernel<kFmtMxfp4, NR, 1>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((stage2_gemv_kernel<kFmtMxfp4, NR, 2>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

template <int FMT>
static hipError_t launch_decode_fmt(const MoeGemmArgs& a, int stage, hipStream_t s) {
    const int64_t nb = a.cap / a.bm;
    const int64_t units = nb * (stage == 1 ? a.I / 16 : a.H / 32);
    const dim3 grid((unsigned)((units + kUnitWaves - 1) / kUnitWaves)), block(kUnitWaves * 64);
    if (stage == 1) {
        if (a.bm == 16) hipLaunchKernelGGL((stage1_unit_kernel<FMT, 1>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((stage1_unit_kernel<FMT, 2>), grid, block, 0, s, a);
    } else {
        if (a.bm == 16) hipLaunchKernelGGL((stage2_unit_kernel<FMT, 1>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((stage2_unit_kernel<FMT, 2>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_decode_stage(const MoeGemmArgs& a, int stage, hipStream_t s) {
    if (gemv_eligible(a)) {
        const int rows = a.T < a.bm ? a.T : a.bm;
        if (rows <= 1) return launch_gemv_nr<1>(a, stage, s);
        if (rows <= 2) return launch_gemv_nr<2>(a, stage, s);
        return launch_gemv_nr<4>(a, stage, s);
    }
    return a.fmt == kFmtMxfp4 ? launch_decode_fmt<kFmtMxfp4>(a, stage, s)
                              : launch_decode_fmt<kFmtInt4g32>(a, stage, s);
}

}  // namespace moe

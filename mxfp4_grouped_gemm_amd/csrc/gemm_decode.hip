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

constexpr int kUnitWaves = 4;        // waves (= units) per workgroup (one tile per wave)
constexpr int kRing = 4;             // K steps in flight per wave

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
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar addressing
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
    GluTerms glu;
    glu.load(a, e, i0 + nl);
#pragma unroll
    for (int s = 0; s < MSUB; ++s) {
        if (s >= nact) break;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = 4 * g + j;
            if (m < valid[s]) {
                float gv = accg[s][j], uv = accu[s][j];
                glu.apply(gv, uv);
                a.h[(row0 + 16 * s + m) * I + i0 + nl] = f32_to_bf16_bits(swiglu(gv, uv));
            }
        }
    }
}

// Stage 2 (down). Unit u = (block b, 32-row slice of H).
template <int FMT, int MSUB>
__global__ __launch_bounds__(kUnitWaves * 64) void stage2_unit_kernel(MoeGemmArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar addressing
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
    const int rows = a.T < a.bm ? a.T : a.bm;
    if (rows > 1 && gemv_resident_eligible(a)) return launch_gemv_resident_stage(a, stage, s);
    if (a.T > 12 && gemv_mfma_eligible(a)) return launch_gemv_mfma_x_stage(a, stage, s);
    if (rows > 1 && gemv_mfma_eligible(a)) return launch_gemv_mfma_stage(a, stage, s);
    if (gemv_eligible(a)) return launch_gemv_stage(a, stage, s);
    return a.fmt == kFmtMxfp4 ? launch_decode_fmt<kFmtMxfp4>(a, stage, s)
                              : launch_decode_fmt<kFmtInt4g32>(a, stage, s);
}

}  // namespace moe

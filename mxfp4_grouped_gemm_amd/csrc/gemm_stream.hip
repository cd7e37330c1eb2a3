// Weight-streaming grouped GEMMs for few rows per expert (decode).
//
// Stage 1 (gate_up + SwiGLU) and stage 2 (down) of the two-stage MoE. At
// decode token counts each expert block has at most a few dozen rows, so
// the layer streams its weights once from HBM and the kernel is built around
// that stream:
//
//  * a workgroup owns one expert block (<= 64 rows) and a 32-row slice of
//    the weight (stage 1: 16 gate rows + the matching 16 up rows, so the
//    SwiGLU pairs meet in one workgroup; stage 2: 32 output rows);
//  * its four waves split K, interleaved so that the workgroup reads 512
//    contiguous bytes of every weight row per step;
//  * each lane loads 16 bytes of one weight row -- 32 e2m1 codes, exactly one
//    MX block and one e8m0 byte -- and decodes them in registers with the
//    gfx950 scaled fp4 -> bf16 converts (exact: an e2m1 value times a power
//    of two fits bf16);
//  * the bf16 operands feed v_mfma_f32_16x16x32_bf16. The activation rows
//    form the A operand (row = lane % 16), the weights the B operand; the
//    K order inside an MFMA is a permutation shared by both operands, so
//    lane group g holds its own MX block and MFMA q takes elements 8q..8q+7
//    of it. Row sub-tiles of 16 with no valid row are skipped;
//  * partial sums of the four waves meet in LDS in a fixed order
//    (deterministic), then the epilogue applies SwiGLU (stage 1, h stored as
//    bf16) or writes fp32 y rows at the pair index (stage 2).
//
// int4-g32 weights use per-group MFMAs instead: lane group g loads dword g
// of four consecutive 32-groups, so one MFMA spans exactly one group and its
// fp32 result is scaled by that group's bf16 scale (exact, no bf16 rounding
// of code * scale). Codes enter the MFMA biased by +136 (cheap to build from
// the nibbles); the bias times the group's activation sum is subtracted.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kStreamThreads = 256;
constexpr int kStreamWaves = 4;

__device__ __forceinline__ u32x4 ld16(const void* p) { return *(const u32x4*)p; }

// One K pass over two weight row-slices (B0, B1; 16 rows each, rows selected
// per lane by the caller) against up to MSUB 16-row activation sub-tiles.
// arow[s]: this lane's activation row (A row = lane % 16) or nullptr.
template <int FMT, int MSUB>
__device__ __forceinline__ void stream_k_loop(const uint16_t* const (&arow)[MSUB], int nact,
                                              const uint8_t* b0, const uint8_t* b1,
                                              const void* s0v, const void* s1v, int K, int wave,
                                              int g, f32x4 (&acc0)[MSUB], f32x4 (&acc1)[MSUB]) {
    const int nblk = K / 32;
    if constexpr (FMT == kFmtMxfp4) {
        const uint8_t* s0 = (const uint8_t*)s0v;
        const uint8_t* s1 = (const uint8_t*)s1v;
        for (int base = 4 * wave; base < nblk; base += 4 * kStreamWaves) {
            const int blk = base + g;
            const bool ok = blk < nblk;
            u32x4 w0 = {0u, 0u, 0u, 0u}, w1 = {0u, 0u, 0u, 0u};
            uint32_t e0 = 127u, e1 = 127u;
            if (ok) {
                w0 = ld16(b0 + (int64_t)blk * 16);
                w1 = ld16(b1 + (int64_t)blk * 16);
                e0 = s0[blk];
                e1 = s1[blk];
            }
            const float sc0 = e8m0_scale_operand(e0), sc1 = e8m0_scale_operand(e1);
            bf16x8 q0[4], q1[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                q0[q] = mxfp4x8_to_bf16(w0[q], sc0);
                q1[q] = mxfp4x8_to_bf16(w1[q], sc1);
            }
#pragma unroll
            for (int s = 0; s < MSUB; ++s) {
                if (s >= nact) break;
                bf16x8 xa[4];
                if (ok && arow[s]) {
                    const u32x4* src = (const u32x4*)(arow[s] + (int64_t)blk * 32);
#pragma unroll
                    for (int q = 0; q < 4; ++q) xa[q] = __builtin_bit_cast(bf16x8, src[q]);
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q) xa[q] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc0[s] = mfma16x16x32(xa[q], q0[q], acc0[s]);
                    acc1[s] = mfma16x16x32(xa[q], q1[q], acc1[s]);
                }
            }
        }
    } else {
        const uint16_t* s0 = (const uint16_t*)s0v;
        const uint16_t* s1 = (const uint16_t*)s1v;
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
        for (int base = 4 * wave; base < nblk; base += 4 * kStreamWaves) {
            uint32_t d0[4], d1[4];
            float sc0[4], sc1[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int grp = base + q;
                const bool ok = grp < nblk;
                d0[q] = ok ? *(const uint32_t*)(b0 + (int64_t)grp * 16 + 4 * g) : 0u;
                d1[q] = ok ? *(const uint32_t*)(b1 + (int64_t)grp * 16 + 4 * g) : 0u;
                sc0[q] = ok ? bf16_bits_to_f32(s0[grp]) : 0.0f;
                sc1[q] = ok ? bf16_bits_to_f32(s1[grp]) : 0.0f;
            }
#pragma unroll
            for (int s = 0; s < MSUB; ++s) {
                if (s >= nact) break;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int grp = base + q;
                    bf16x8 xa = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
                    if (grp < nblk && arow[s])
                        xa = perm_x_int4(__builtin_bit_cast(
                            bf16x8, ld16(arow[s] + (int64_t)grp * 32 + 8 * g)));
                    const f32x4 t0 = mfma16x16x32(xa, int4x8_to_bf16_biased(d0[q]), zero);
                    const f32x4 t1 = mfma16x16x32(xa, int4x8_to_bf16_biased(d1[q]), zero);
                    const f32x4 xs = mfma16x16x32(xa, ones, zero);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        acc0[s][j] = fmaf(fmaf(-136.0f, xs[j], t0[j]), sc0[q], acc0[s][j]);
                        acc1[s][j] = fmaf(fmaf(-136.0f, xs[j], t1[j]), sc1[q], acc1[s][j]);
                    }
                }
            }
        }
    }
}

// Stage 1. grid = (I / 16, cap / bm). h[r, i] = silu(gate) * up for valid rows.
template <int FMT, int MSUB>
__global__ __launch_bounds__(kStreamThreads) void stage1_stream_kernel(MoeGemmArgs a) {
    __shared__ float red[kStreamWaves][MSUB][2][16][17];
    const int b = blockIdx.y;
    const int bm = a.bm;
    if ((int64_t)b * bm >= (int64_t)*a.num_post_pad) return;
    const int e = a.block_expert[b];
    if (e < 0 || e >= a.E) return;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nl = lane & 15, g = lane >> 4;
    const int H = a.H, I = a.I, P = a.T * a.topk;
    const int i0 = blockIdx.x * 16;
    const int64_t row0 = (int64_t)b * bm;

    const uint16_t* arow[MSUB];
    int nact = 0;
#pragma unroll
    for (int s = 0; s < MSUB; ++s) {
        arow[s] = nullptr;
        if (16 * s < bm) {
            const int p = a.sorted_ids[row0 + 16 * s + nl];
            if (p >= 0 && p < P) arow[s] = a.x + (int64_t)(p / a.topk) * H;
        }
        if (__ballot(arow[s] != nullptr)) nact = s + 1;
    }

    const int64_t gate_row = (int64_t)e * 2 * I + i0 + nl;
    const int64_t up_row = gate_row + I;
    const int64_t sstride = H / 32;
    const void *sg, *su;
    if constexpr (FMT == kFmtMxfp4) {
        sg = (const uint8_t*)a.w13_scale + gate_row * sstride;
        su = (const uint8_t*)a.w13_scale + up_row * sstride;
    } else {
        sg = (const uint16_t*)a.w13_scale + gate_row * sstride;
        su = (const uint16_t*)a.w13_scale + up_row * sstride;
    }

    f32x4 accg[MSUB], accu[MSUB];
#pragma unroll
    for (int s = 0; s < MSUB; ++s) accg[s] = accu[s] = f32x4{0.f, 0.f, 0.f, 0.f};
    stream_k_loop<FMT, MSUB>(arow, nact, a.w13 + gate_row * (H / 2), a.w13 + up_row * (H / 2), sg,
                             su, H, wave, g, accg, accu);

#pragma unroll
    for (int s = 0; s < MSUB; ++s) {
        if (s >= nact) break;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            red[wave][s][0][4 * g + j][nl] = accg[s][j];
            red[wave][s][1][4 * g + j][nl] = accu[s][j];
        }
    }
    __syncthreads();
    const int row = tid >> 4, col = tid & 15;
    GluTerms glu;
    glu.load(a, e, i0 + col);
    for (int s = 0; s < nact; ++s) {
        const int64_t r = row0 + 16 * s + row;
        const int p = a.sorted_ids[r];
        if (p < 0 || p >= P) continue;
        float gs = 0.f, us = 0.f;
#pragma unroll
        for (int w = 0; w < kStreamWaves; ++w) {
            gs += red[w][s][0][row][col];
            us += red[w][s][1][row][col];
        }
        glu.apply(gs, us);
        a.h[r * I + i0 + col] = f32_to_bf16_bits(swiglu(gs, us));
    }
}

// Stage 2. grid = (H / 32, cap / bm). y[p, n] = W2[e][n] . h[r] for valid rows.
template <int FMT, int MSUB>
__global__ __launch_bounds__(kStreamThreads) void stage2_stream_kernel(MoeGemmArgs a) {
    __shared__ float red[kStreamWaves][MSUB][2][16][17];
    const int b = blockIdx.y;
    const int bm = a.bm;
    if ((int64_t)b * bm >= (int64_t)*a.num_post_pad) return;
    const int e = a.block_expert[b];
    if (e < 0 || e >= a.E) return;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nl = lane & 15, g = lane >> 4;
    const int H = a.H, I = a.I, P = a.T * a.topk;
    const int n0 = blockIdx.x * 32;
    const int64_t row0 = (int64_t)b * bm;

    const uint16_t* arow[MSUB];
    int nact = 0;
#pragma unroll
    for (int s = 0; s < MSUB; ++s) {
        arow[s] = nullptr;
        if (16 * s < bm) {
            const int64_t r = row0 + 16 * s + nl;
            const int p = a.sorted_ids[r];
            if (p >= 0 && p < P) arow[s] = a.h + r * I;
        }
        if (__ballot(arow[s] != nullptr)) nact = s + 1;
    }

    const int64_t wrow0 = (int64_t)e * H + n0 + nl;
    const int64_t wrow1 = wrow0 + 16;
    const int64_t sstride = I / 32;
    const void *s0, *s1;
    if constexpr (FMT == kFmtMxfp4) {
        s0 = (const uint8_t*)a.w2_scale + wrow0 * sstride;
        s1 = (const uint8_t*)a.w2_scale + wrow1 * sstride;
    } else {
        s0 = (const uint16_t*)a.w2_scale + wrow0 * sstride;
        s1 = (const uint16_t*)a.w2_scale + wrow1 * sstride;
    }

    f32x4 acc0[MSUB], acc1[MSUB];
#pragma unroll
    for (int s = 0; s < MSUB; ++s) acc0[s] = acc1[s] = f32x4{0.f, 0.f, 0.f, 0.f};
    stream_k_loop<FMT, MSUB>(arow, nact, a.w2 + wrow0 * (I / 2), a.w2 + wrow1 * (I / 2), s0, s1, I,
                             wave, g, acc0, acc1);

#pragma unroll
    for (int s = 0; s < MSUB; ++s) {
        if (s >= nact) break;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            red[wave][s][0][4 * g + j][nl] = acc0[s][j];
            red[wave][s][1][4 * g + j][nl] = acc1[s][j];
        }
    }
    __syncthreads();
    const int row = tid >> 4, col = tid & 15;
    for (int s = 0; s < nact; ++s) {
        const int64_t r = row0 + 16 * s + row;
        const int p = a.sorted_ids[r];
        if (p < 0 || p >= P) continue;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            float sum = 0.f;
#pragma unroll
            for (int w = 0; w < kStreamWaves; ++w) sum += red[w][s][t][row][col];
            a.y[(int64_t)p * H + n0 + 16 * t + col] = sum;
        }
    }
}

template <int FMT>
static hipError_t launch_stage1_fmt(const MoeGemmArgs& a, hipStream_t s) {
    const dim3 grid(a.I / 16, (unsigned)(a.cap / a.bm)), block(kStreamThreads);
    switch (a.bm) {
        case 16: hipLaunchKernelGGL((stage1_stream_kernel<FMT, 1>), grid, block, 0, s, a); break;
        case 32: hipLaunchKernelGGL((stage1_stream_kernel<FMT, 2>), grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL((stage1_stream_kernel<FMT, 4>), grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

template <int FMT>
static hipError_t launch_stage2_fmt(const MoeGemmArgs& a, hipStream_t s) {
    const dim3 grid(a.H / 32, (unsigned)(a.cap / a.bm)), block(kStreamThreads);
    switch (a.bm) {
        case 16: hipLaunchKernelGGL((stage2_stream_kernel<FMT, 1>), grid, block, 0, s, a); break;
        case 32: hipLaunchKernelGGL((stage2_stream_kernel<FMT, 2>), grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL((stage2_stream_kernel<FMT, 4>), grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_stage1(const MoeGemmArgs& a, hipStream_t s) {
    return a.fmt == kFmtMxfp4 ? launch_stage1_fmt<kFmtMxfp4>(a, s) : launch_stage1_fmt<kFmtInt4g32>(a, s);
}

hipError_t launch_stage2(const MoeGemmArgs& a, hipStream_t s) {
    return a.fmt == kFmtMxfp4 ? launch_stage2_fmt<kFmtMxfp4>(a, s) : launch_stage2_fmt<kFmtInt4g32>(a, s);
}

}  // namespace moe

// GEMV-shaped decode kernels for expert blocks of at most 8 token rows
// (MXFP4 weights; H a multiple of 256 and I a multiple of 128, both up to
// 4096, so that each wave's scale bytes arrive as whole 16-byte pieces).
//
// With one or a few activation rows per expert block, 15/16 of every MFMA
// would idle and the MFMA operand layout (16 rows x 64 bytes per load) costs a
// memory instruction per 64 bytes of each row. Here a wave owns 4 weight
// rows over the whole K instead:
//  * each load instruction reads 1 KB contiguous of one row (lane l holds MX
//    block 64c + l of chunk c), and every load of the wave is issued up
//    front, so a wave is one memory round trip;
//  * the e8m0 scales of the 4 rows arrive as one 16-byte load per lane into
//    wave-private LDS (a byte per lane per row would cost as many memory
//    instructions as the weights);
//  * a lane decodes its block with the scaled fp4 -> bf16 converts and
//    accumulates v_dot2_f32_bf16 against the matching 32 activations; row
//    sums meet with permlane32/16 swaps and DPP row rotations.
//
// Both stages are block-major (one expert block; its <= 8 token rows share
// the weight stream, dotted one after another against the same registers).
// Stage 1 stores h by pair index, stage 2 stores fp32 y by pair index, and
// the combine kernel sums the slots of each token.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kGemvWaves1 = 4;            // stage 1: waves per workgroup (independent tiles)
constexpr int kDownWaves = 4;             // stage 2: waves per workgroup
constexpr int kDownRows = 4 * kDownWaves; // stage 2: output rows per workgroup

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
// two-result builtin lost its second result when both were used. The
// compiler cannot see inside the asm, so the asm carries its own wait states
// for the VALU-write -> permlane-read hazard: 3 cover the slowest producer
// here (v_dot2c_f32_bf16; other VALU ops need 2). With 2, the last dot of
// the lanes moved across was read stale.
__device__ __forceinline__ void permlane32_swap(float& a, float& b) {
    asm volatile("s_nop 2\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void permlane16_swap(float& a, float& b) {
    asm volatile("s_nop 2\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float swap32_add(float a, float b) {
    permlane32_swap(a, b);
    return a + b;
}
__device__ __forceinline__ float swap16_add(float a, float b) {
    permlane16_swap(a, b);
    return a + b;
}
// Reduce 4 per-lane partials over the wave: 16-lane row rho of the result
// holds the total of v[sig(rho)], sig = (0, 2, 1, 3).
__device__ __forceinline__ float reduce4(const float (&v)[4]) {
    return row16_sum(swap16_add(swap32_add(v[0], v[1]), swap32_add(v[2], v[3])));
}

// Four weight rows as up to two runs of consecutive rows (run 0 -> slots
// 0..n0-1, run 1 -> the rest).
struct GemvRows {
    int first0, n0, first1;
    __device__ __forceinline__ int row(int r) const { return r < n0 ? first0 + r : first1 + (r - n0); }
};

// Loads of one wave for 4 weight rows over NCH chunks of 64 MX blocks.
template <int NCH>
struct GemvWeights {
    u32x4 w[4][NCH];
    u32x4 sc;  // this lane's 16-byte piece of the rows' scale bytes

    __device__ __forceinline__ void issue(rsrc_t rw, rsrc_t rs, const GemvRows& rows, int nblk, int lane) {
        const int p0 = rows.n0 * nblk / 16, ptot = 4 * nblk / 16;
        uint32_t so = kOob;
        if (lane < p0)
            so = (uint32_t)rows.first0 * nblk + 16u * lane;
        else if (lane < ptot)
            so = (uint32_t)rows.first1 * nblk + 16u * (lane - p0);
        sc = bld16nt(rs, so);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int blk = 64 * c + lane;
                w[r][c] = bld16nt(rw, blk < nblk ? (uint32_t)rows.row(r) * (uint32_t)(nblk * 16) + 16u * blk : kOob);
            }
    }
    // Scale bytes into wave-private LDS: row slot r at [r * nblk, +nblk).
    __device__ __forceinline__ void stage_scales(uint8_t* lds, int nblk, int lane) const {
        if (lane < 4 * nblk / 16) *(u32x4*)(lds + 16 * lane) = sc;
    }
};

template <int NCH>
__device__ __forceinline__ void issue_x(u32x4 (&x)[NCH][4], rsrc_t rx, uint32_t x_off, int nblk, int lane) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int blk = 64 * c + lane;
        const uint32_t o = (x_off != kOob && blk < nblk) ? x_off + 64u * blk : kOob;
#pragma unroll
        for (int q = 0; q < 4; ++q) x[c][q] = bld16(rx, o + 16u * q);
    }
}

// acc[r] += dot(weight row r, activation row) over this lane's blocks.
template <int NCH>
__device__ __forceinline__ void gemv_dot(const GemvWeights<NCH>& W, const uint8_t* lds_scale,
                                         const u32x4 (&x)[NCH][4], int nblk, int lane,
                                         float (&acc)[4]) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int blk = 64 * c + lane;
        const int sblk = blk < nblk ? blk : nblk - 1;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float sc = e8m0_scale_operand(lds_scale[r * nblk + sblk]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                // bf16 pairs via shufflevector: element access through a u32x4
                // bit_cast was folded to element 0 by the compiler.
                const bf16x8 wv = mxfp4x8_to_bf16(W.w[r][c][q], sc);
                const bf16x8 xv = __builtin_bit_cast(bf16x8, x[c][q]);
                acc[r] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(wv, wv, 0, 1),
                                                         __builtin_shufflevector(xv, xv, 0, 1), acc[r], false);
                acc[r] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(wv, wv, 2, 3),
                                                         __builtin_shufflevector(xv, xv, 2, 3), acc[r], false);
                acc[r] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(wv, wv, 4, 5),
                                                         __builtin_shufflevector(xv, xv, 4, 5), acc[r], false);
                acc[r] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(wv, wv, 6, 7),
                                                         __builtin_shufflevector(xv, xv, 6, 7), acc[r], false);
            }
        }
    }
}

// Stage 1: unit = (expert block b, columns i0, i0+1 of I): gate rows i0,
// i0+1 and up rows I+i0, I+i0+1, against the block's <= NRMAX token rows.
// The activations of the first NR rows are loaded with the weights; further
// rows (rare at decode sizes) reuse those registers one row at a time, so
// the register footprint -- and the occupancy -- is that of NR rows.
// One token row per block (T = 1) fits 79 VGPRs without spilling: six waves
// per SIMD keep about 1.5x more weight bytes in flight per CU than the
// compiler's default of four (35 -> 32 us at the production decode shape).
// With rows reloaded in sequence the default allocation is faster.
// EPI: with the optional expert bias / clamp epilogue (instances launched
// without them are built without it, so their registers are untouched).
template <int NR, int NRMAX, int NCH, bool EPI>
__global__ __launch_bounds__(kGemvWaves1 * 64) __attribute__((amdgpu_waves_per_eu(NRMAX == 1 ? 6 : 1)))
void stage1_gemv_kernel(MoeGemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t lds_scale[kGemvWaves1][4 * 64 * NCH];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar addressing
    const int upb = a.I / 2;
    const int64_t u = (int64_t)blockIdx.x * kGemvWaves1 + wave;
    const int64_t b = u / upb;
    if (b >= a.cap / a.bm) return;
    // One round trip: the block's expert (-1 past the used blocks) and rows.
    const int64_t row0 = b * a.bm;
    const int e = a.block_expert[b];
    const int P = a.T * a.topk;
    int pair[NRMAX], nvalid = 0;
#pragma unroll
    for (int m = 0; m < NRMAX; ++m) {
        pair[m] = a.sorted_ids[row0 + m];
        nvalid += (pair[m] >= 0 && pair[m] < P) ? 1 : 0;
    }
    if (e < 0 || e >= a.E) return;
    const int i0 = (int)(u % upb) * 2;
    const int H = a.H, I = a.I, nblk = H / 32;
    // The unit's gate and up biases (columns i0, i0 + 1: one aligned dword
    // each), read with wave-uniform loads before anything is stored, so they
    // sit in scalar registers and cost the weight stream no VGPRs.
    uint32_t bgate = 0u, bup = 0u;
    if (EPI && a.w13_bias) {
        const uint16_t* bb = a.w13_bias + (int64_t)e * 2 * I + i0;
        bgate = __builtin_amdgcn_readfirstlane(*(const uint32_t*)bb);
        bup = __builtin_amdgcn_readfirstlane(*(const uint32_t*)(bb + I));
    }

    const int64_t slab_rows = 2 * (int64_t)I;
    const rsrc_t rw = make_rsrc(a.w13 + e * slab_rows * (H / 2), (uint32_t)(slab_rows * (H / 2)));
    const rsrc_t rs = make_rsrc((const uint8_t*)a.w13_scale + e * slab_rows * nblk, (uint32_t)(slab_rows * nblk));
    const rsrc_t rx = make_rsrc(a.x, (uint32_t)((int64_t)a.T * H * 2));
    auto x_off = [&](int m) -> uint32_t {
        return m < nvalid ? (uint32_t)(pair[m] / a.topk) * (uint32_t)(2 * H) : kOob;
    };
    // Activations first: the oldest loads, so waiting for them never waits
    // for the weight stream issued after them.
    u32x4 x[NR][NCH][4];
#pragma unroll
    for (int m = 0; m < NR; ++m) issue_x<NCH>(x[m], rx, x_off(m), nblk, lane);
    GemvWeights<NCH> W;
    W.issue(rw, rs, GemvRows{i0, 2, I + i0}, nblk, lane);
    W.stage_scales(lds_scale[wave], nblk, lane);
    wave_lds_sync();

#pragma unroll
    for (int m = 0; m < NRMAX; ++m) {
        if (m >= nvalid) break;
        if (m >= NR) issue_x<NCH>(x[m % NR], rx, x_off(m), nblk, lane);
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        gemv_dot<NCH>(W, lds_scale[wave], x[m % NR], nblk, lane, acc);
        // acc: gate i0, gate i0+1, up i0, up i0+1. With v = (g0, u0, g1, u1)
        // the rows after reduce4 hold (g0, g1, u0, u1); a permlane32 swap of
        // the sum with itself puts (g0, u0) in lanes 0..15, (g1, u1) in 16..31.
        float v[4] = {acc[0], acc[2], acc[1], acc[3]};
        float gs = reduce4(v), us = gs;
        permlane32_swap(gs, us);
        if ((lane & 15) == 0 && lane < 32) {
            if constexpr (EPI) {
                if (a.w13_bias) {  // lane 0 takes column i0 (low halves), lane 16 column i0 + 1
                    gs += __uint_as_float(lane ? (bgate & 0xffff0000u) : (bgate << 16));
                    us += __uint_as_float(lane ? (bup & 0xffff0000u) : (bup << 16));
                }
                const float lim = a.swiglu_limit;
                if (lim > 0.0f) {
                    gs = fminf(fmaxf(gs, -lim), lim);
                    us = fminf(fmaxf(us, -lim), lim);
                }
            }
            a.h[(int64_t)pair[m] * I + i0 + (lane >> 4)] = f32_to_bf16_bits(swiglu(gs, us));
        }
    }
}

// Four weight rows in half-block units: lane l holds half-block 64c + l
// (16 K elements, 8 code bytes) of each row, so K = 16 * nhb fills the lanes
// evenly whenever nhb is a multiple of 64 (I = 3072: three chunks, no idle
// lane). Rows first .. first + nv - 1 (nv <= 4) of one expert; further row
// slots load nothing.
template <int NHC>
struct HalfRows {
    u32x2 w[4][NHC];
    u32x4 sc;  // this lane's 16-byte piece of the rows' scale bytes

    __device__ __forceinline__ void issue_run(rsrc_t rw, rsrc_t rs, int first, int nv, int nhb, int lane) {
        const int nblk = nhb / 2, ptot = nv * nblk / 16;
        sc = bld16nt(rs, lane < ptot ? (uint32_t)first * nblk + 16u * lane : kOob);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < NHC; ++c) {
                const int hb = 64 * c + lane;
                w[r][c] = bld8nt(rw, (r < nv && hb < nhb) ? (uint32_t)(first + r) * (uint32_t)(nhb * 8) + 8u * hb
                                                        : kOob);
            }
    }
    __device__ __forceinline__ void stage_scales(uint8_t* lds, int nhb, int lane) const {
        if (lane < 4 * (nhb / 2) / 16) *(u32x4*)(lds + 16 * lane) = sc;
    }
};

template <int NHC>
__device__ __forceinline__ void issue_xh(u32x4 (&x)[NHC][2], rsrc_t rx, uint32_t x_off, int nhb, int lane) {
#pragma unroll
    for (int c = 0; c < NHC; ++c) {
        const int hb = 64 * c + lane;
        const uint32_t o = (x_off != kOob && hb < nhb) ? x_off + 32u * hb : kOob;
        x[c][0] = bld16(rx, o);
        x[c][1] = bld16(rx, o + 16u);
    }
}

template <int NHC>
__device__ __forceinline__ void half_dot(const HalfRows<NHC>& W, const uint8_t* lds_scale,
                                         const u32x4 (&x)[NHC][2], int nhb, int lane, float (&acc)[4]) {
    const int nblk = nhb / 2;
#pragma unroll
    for (int c = 0; c < NHC; ++c) {
        const int hb = 64 * c + lane;
        const int sblk = (hb < nhb ? hb : nhb - 1) >> 1;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float sc = e8m0_scale_operand(lds_scale[r * nblk + sblk]);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const bf16x8 wv = mxfp4x8_to_bf16(W.w[r][c][q], sc);
                const bf16x8 xv = __builtin_bit_cast(bf16x8, x[c][q]);
                acc[r] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(wv, wv, 0, 1),
                                                         __builtin_shufflevector(xv, xv, 0, 1), acc[r], false);
                acc[r] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(wv, wv, 2, 3),
                                                         __builtin_shufflevector(xv, xv, 2, 3), acc[r], false);
                acc[r] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(wv, wv, 4, 5),
                                                         __builtin_shufflevector(xv, xv, 4, 5), acc[r], false);
                acc[r] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(wv, wv, 6, 7),
                                                         __builtin_shufflevector(xv, xv, 6, 7), acc[r], false);
            }
        }
    }
}

// Stage 2, block-major like stage 1: unit = (expert block b, output rows
// n0..n0+3); a wave reads those 4 rows of the block's expert once (6 KB at
// I = 3072, one memory round trip in half-block loads) and dots them with the
// block's <= NRMAX h rows one after another, storing fp32 y[pair][n]; the
// combine kernel follows. A workgroup covers kDownRows consecutive rows of one
// block, so its loads are one contiguous run of the expert's rows.
template <int NHC, int NRMAX>
__global__ __launch_bounds__(kDownWaves * 64) void stage2_gemv_blk_kernel(MoeGemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t lds_scale[kDownWaves][4 * 32 * NHC];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar addressing
    const int H = a.H, I = a.I, nblk = I / 32, nhb = I / 16;
    const int gpb = H / kDownRows;  // row groups per block
    const int64_t b = blockIdx.x / gpb;
    const int g = (int)(blockIdx.x % gpb);
    const int nused = *a.num_post_pad / a.bm;  // blocks holding pairs
    if (b >= nused) return;
    const int64_t row0 = b * a.bm;
    const int e = a.block_expert[b];
    const int P = a.T * a.topk;
    int pair[NRMAX], nvalid = 0;
#pragma unroll
    for (int m = 0; m < NRMAX; ++m) {
        pair[m] = a.sorted_ids[row0 + m];
        nvalid += (pair[m] >= 0 && pair[m] < P) ? 1 : 0;
    }
    const int n0 = g * kDownRows + 4 * wave;
    if ((unsigned)e >= (unsigned)a.E) return;
    const rsrc_t rw = make_rsrc(a.w2 + (int64_t)e * H * (I / 2), (uint32_t)((int64_t)H * (I / 2)));
    const rsrc_t rs = make_rsrc((const uint8_t*)a.w2_scale + (int64_t)e * H * nblk, (uint32_t)((int64_t)H * nblk));
    const rsrc_t rx = make_rsrc(a.h, (uint32_t)((int64_t)P * I * 2));
    u32x4 x[NHC][2];
    issue_xh<NHC>(x, rx, nvalid > 0 ? (uint32_t)pair[0] * (uint32_t)(2 * I) : kOob, nhb, lane);
    HalfRows<NHC> W;
    W.issue_run(rw, rs, n0, 4, nhb, lane);
    W.stage_scales(lds_scale[wave], nhb, lane);
    wave_lds_sync();
    const int rho = lane >> 4;
    const int r = (rho == 1) ? 2 : (rho == 2) ? 1 : rho;  // rows after reduce4: (0, 2, 1, 3)
#pragma unroll
    for (int m = 0; m < NRMAX; ++m) {
        if (m >= nvalid) break;
        if (m > 0) issue_xh<NHC>(x, rx, (uint32_t)pair[m] * (uint32_t)(2 * I), nhb, lane);
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        half_dot<NHC>(W, lds_scale[wave], x, nhb, lane, acc);
        const float q = reduce4(acc);
        if ((lane & 15) == 0) a.y[(int64_t)pair[m] * H + n0 + r] = q;
    }
}

bool gemv_eligible(const MoeGemmArgs& a) {
    const int max_rows = a.T < a.bm ? a.T : a.bm;
    return a.fmt == kFmtMxfp4 && max_rows <= 8 &&
           a.H <= 4096 && a.I <= 4096 && a.H % 256 == 0 && a.I % 128 == 0 &&
           (int64_t)a.T * a.topk * a.I * 2 < 0x7fff0000LL;
}

template <int NRMAX>
static void launch_stage1_nr(const MoeGemmArgs& a, int nch, hipStream_t s) {
    const int64_t units = (a.cap / a.bm) * (a.I / 2);
    const dim3 grid((unsigned)((units + kGemvWaves1 - 1) / kGemvWaves1)), block(kGemvWaves1 * 64);
    const bool epi = a.w13_bias || a.swiglu_limit > 0.0f;
    if (nch == 1) {
        if (epi) hipLaunchKernelGGL((stage1_gemv_kernel<1, NRMAX, 1, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((stage1_gemv_kernel<1, NRMAX, 1, false>), grid, block, 0, s, a);
    } else {
        if (epi) hipLaunchKernelGGL((stage1_gemv_kernel<1, NRMAX, 2, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((stage1_gemv_kernel<1, NRMAX, 2, false>), grid, block, 0, s, a);
    }
}

template <int NHC>
static void launch_down_blk(const MoeGemmArgs& a, int rows, hipStream_t s) {
    const dim3 grid((unsigned)((a.cap / a.bm) * (a.H / kDownRows))), block(kDownWaves * 64);
    if (rows <= 1) hipLaunchKernelGGL((stage2_gemv_blk_kernel<NHC, 1>), grid, block, 0, s, a);
    else if (rows <= 2) hipLaunchKernelGGL((stage2_gemv_blk_kernel<NHC, 2>), grid, block, 0, s, a);
    else if (rows <= 4) hipLaunchKernelGGL((stage2_gemv_blk_kernel<NHC, 4>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((stage2_gemv_blk_kernel<NHC, 8>), grid, block, 0, s, a);
}

hipError_t launch_gemv_stage(const MoeGemmArgs& a, int stage, hipStream_t s) {
    if (stage == 1) {
        const int nch = (a.H / 32 + 63) / 64;
        const int rows = a.T < a.bm ? a.T : a.bm;
        if (rows <= 1) launch_stage1_nr<1>(a, nch, s);
        else if (rows <= 2) launch_stage1_nr<2>(a, nch, s);
        else if (rows <= 4) launch_stage1_nr<4>(a, nch, s);
        else launch_stage1_nr<8>(a, nch, s);
    } else {
        const int nhc = (a.I / 16 + 63) / 64;
        const int rows = a.T < a.bm ? a.T : a.bm;
        if (nhc == 1) launch_down_blk<1>(a, rows, s);
        else if (nhc == 2) launch_down_blk<2>(a, rows, s);
        else if (nhc == 3) launch_down_blk<3>(a, rows, s);
        else launch_down_blk<4>(a, rows, s);
    }
    return hipGetLastError();
}

}  // namespace moe

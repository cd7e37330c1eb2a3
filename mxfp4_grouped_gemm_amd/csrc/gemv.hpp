// GEMV building blocks of the decode kernels (blocks of at most 8 token
// rows, MXFP4 weights): one wave owns 4 weight rows over the whole K, reads
// each row in 1 KB runs (one MX block, or half of one, per lane), issues all
// of its loads up front (one memory round trip), decodes with the gfx950
// scaled fp4 -> bf16 converts and accumulates with v_dot2_f32_bf16; the 4 row
// sums meet through permlane swaps and DPP row rotations.
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace moe {

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

// ROWS (<= 4) weight rows in half-block units: lane l holds half-block
// 64c + l (16 K elements, 8 code bytes) of each row, so K = 16 * nhb fills
// the lanes evenly whenever nhb is a multiple of 64 (I = 3072: three chunks,
// no idle lane). Rows first .. first + nv - 1 (nv <= ROWS) of one expert;
// further row slots load nothing. The rows' scale bytes arrive as 16-byte
// pieces, so ROWS * nhb / 2 must be a multiple of 16.
template <int NHC, int ROWS = 4>
struct HalfRows {
    u32x2 w[ROWS][NHC];
    u32x4 sc;  // this lane's 16-byte piece of the rows' scale bytes

    __device__ __forceinline__ void issue_run(rsrc_t rw, rsrc_t rs, int first, int nv, int nhb, int lane) {
        const int nblk = nhb / 2, ptot = nv * nblk / 16;
        sc = bld16nt(rs, lane < ptot ? (uint32_t)first * nblk + 16u * lane : kOob);
#pragma unroll
        for (int r = 0; r < ROWS; ++r)
#pragma unroll
            for (int c = 0; c < NHC; ++c) {
                const int hb = 64 * c + lane;
                w[r][c] = bld8nt(rw, (r < nv && hb < nhb) ? (uint32_t)(first + r) * (uint32_t)(nhb * 8) + 8u * hb
                                                        : kOob);
            }
    }
    __device__ __forceinline__ void stage_scales(uint8_t* lds, int nhb, int lane) const {
        if (lane < ROWS * (nhb / 2) / 16) *(u32x4*)(lds + 16 * lane) = sc;
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

template <int NHC, int ROWS>
__device__ __forceinline__ void half_dot(const HalfRows<NHC, ROWS>& W, const uint8_t* lds_scale,
                                         const u32x4 (&x)[NHC][2], int nhb, int lane, float (&acc)[4]) {
    const int nblk = nhb / 2;
#pragma unroll
    for (int c = 0; c < NHC; ++c) {
        const int hb = 64 * c + lane;
        const int sblk = (hb < nhb ? hb : nhb - 1) >> 1;
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
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

// The gate_up unit of one wave: expert e, columns i0, i0 + 1 (gate rows i0,
// i0 + 1 and up rows I + i0, I + i0 + 1 of w13[e]), against the token rows
// of pairs pair[0 .. nvalid) (nvalid <= NRMAX; x row = pair / topk); h is
// stored by pair. The activations of the first NR rows are loaded with the
// weights; further rows (rare at decode sizes) reuse those registers one row
// at a time, so the register footprint -- and the occupancy -- is that of NR
// rows. lds_scale: this wave's 4 * 64 * NCH bytes of LDS.
// EPI: with the optional expert bias / clamp epilogue (instances launched
// without them are built without it, so their registers are untouched).
template <int NR, int NRMAX, int NCH, bool EPI>
__device__ __forceinline__ void gemv_gate_up_unit(const MoeGemmArgs& a, int e, int i0, const int (&pair)[NRMAX],
                                                  int nvalid, uint8_t* lds_scale, int lane) {
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
    W.stage_scales(lds_scale, nblk, lane);
    wave_lds_sync();

#pragma unroll
    for (int m = 0; m < NRMAX; ++m) {
        if (m >= nvalid) break;
        if (m >= NR) issue_x<NCH>(x[m % NR], rx, x_off(m), nblk, lane);
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        gemv_dot<NCH>(W, lds_scale, x[m % NR], nblk, lane, acc);
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

}  // namespace moe

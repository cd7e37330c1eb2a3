// GEMV-shaped decode kernels for expert blocks of at most 8 token rows
// (MXFP4 weights; H a multiple of 256 and I a multiple of 128, both up to
// 4096, so that each wave's scale bytes arrive as whole 16-byte pieces).
//
// With one or a few activation rows per expert block, 15/16 of every MFMA
// would idle and the MFMA operand layout (16 rows x 64 bytes per load) costs a
// memory instruction per 64 bytes of each row. Here a wave owns 4 weight
// rows over the whole K instead (the down kernel at one token row: two sets
// of 4):
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
#include "gemv.hpp"

namespace moe {

constexpr int kGemvWaves1 = 4;            // stage 1: waves per workgroup (independent tiles)
constexpr int kDownWaves = 4;             // stage 2: waves per workgroup
constexpr int kDownRows = 4 * kDownWaves; // stage 2: output rows per workgroup

// Stage 1: unit = (expert block b, columns i0, i0+1 of I): gate rows i0,
// i0+1 and up rows I+i0, I+i0+1, against the block's <= NRMAX token rows.
// One token row per block (T = 1) fits 79 VGPRs without spilling: six waves
// per SIMD keep about 1.5x more weight bytes in flight per CU than the
// compiler's default of four (35 -> 32 us at the production decode shape).
// With rows reloaded in sequence the default allocation is faster.
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
    gemv_gate_up_unit<NR, NRMAX, NCH, EPI>(a, e, i0, pair, nvalid, lds_scale[wave], lane);
}

// Stage 2, block-major like stage 1: unit = (expert block b, output rows
// n0..n0+4NS-1); a wave reads those rows of the block's expert once (NS sets
// of 4 rows, 6 KB each at I = 3072, one memory round trip in half-block
// loads) and dots them with the block's <= NRMAX h rows one after another,
// storing fp32 y[pair][n]; the combine kernel follows. A workgroup covers
// 4 NS kDownWaves consecutive rows of one block, so its loads are one
// contiguous run of the expert's rows. Two sets per wave (90 VGPRs at one
// token row, five waves per SIMD) put twice the weight bytes in flight per
// h row loaded (graph-replayed step, three alternating runs on one box: 58.2
// -> 57.1 us at one token, 29.5 -> 28.9 us on the 8-way shard; blocks of up
// to 4 and 8 rows at the production shape, forced onto this kernel: 58.4 ->
// 53.9 us at 4 tokens, 87.5 -> 84.7 us at 7); four sets (145 VGPRs) were
// slower.
template <int NHC, int NRMAX, int NS>
__global__ __launch_bounds__(kDownWaves * 64) void stage2_gemv_blk_kernel(MoeGemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t lds_scale[kDownWaves][NS][4 * 32 * NHC];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar addressing
    const int H = a.H, I = a.I, nblk = I / 32, nhb = I / 16;
    const int gpb = H / (NS * kDownRows);  // row groups per block
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
    const int n0 = g * NS * kDownRows + 4 * NS * wave;
    if ((unsigned)e >= (unsigned)a.E) return;
    const rsrc_t rw = make_rsrc(a.w2 + (int64_t)e * H * (I / 2), (uint32_t)((int64_t)H * (I / 2)));
    const rsrc_t rs = make_rsrc((const uint8_t*)a.w2_scale + (int64_t)e * H * nblk, (uint32_t)((int64_t)H * nblk));
    const rsrc_t rx = make_rsrc(a.h, (uint32_t)((int64_t)P * I * 2));
    u32x4 x[NHC][2];
    issue_xh<NHC>(x, rx, nvalid > 0 ? (uint32_t)pair[0] * (uint32_t)(2 * I) : kOob, nhb, lane);
    HalfRows<NHC> W[NS];
#pragma unroll
    for (int k = 0; k < NS; ++k) W[k].issue_run(rw, rs, n0 + 4 * k, 4, nhb, lane);
#pragma unroll
    for (int k = 0; k < NS; ++k) W[k].stage_scales(lds_scale[wave][k], nhb, lane);
    wave_lds_sync();
    const int rho = lane >> 4;
    const int r = (rho == 1) ? 2 : (rho == 2) ? 1 : rho;  // rows after reduce4: (0, 2, 1, 3)
#pragma unroll
    for (int m = 0; m < NRMAX; ++m) {
        if (m >= nvalid) break;
        if (m > 0) issue_xh<NHC>(x, rx, (uint32_t)pair[m] * (uint32_t)(2 * I), nhb, lane);
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            float acc[4] = {0.f, 0.f, 0.f, 0.f};
            half_dot<NHC>(W[k], lds_scale[wave][k], x, nhb, lane, acc);
            const float q = reduce4(acc);
            if ((lane & 15) == 0) a.y[(int64_t)pair[m] * H + n0 + 4 * k + r] = q;
        }
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

// Two sets of 4 rows per wave: H is a multiple of 256 on this path, so a
// workgroup's 32 rows divide it.
template <int NHC>
static void launch_down_blk(const MoeGemmArgs& a, int rows, hipStream_t s) {
    const dim3 grid((unsigned)((a.cap / a.bm) * (a.H / (2 * kDownRows)))), block(kDownWaves * 64);
    if (rows <= 1) hipLaunchKernelGGL((stage2_gemv_blk_kernel<NHC, 1, 2>), grid, block, 0, s, a);
    else if (rows <= 2) hipLaunchKernelGGL((stage2_gemv_blk_kernel<NHC, 2, 2>), grid, block, 0, s, a);
    else if (rows <= 4) hipLaunchKernelGGL((stage2_gemv_blk_kernel<NHC, 4, 2>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((stage2_gemv_blk_kernel<NHC, 8, 2>), grid, block, 0, s, a);
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

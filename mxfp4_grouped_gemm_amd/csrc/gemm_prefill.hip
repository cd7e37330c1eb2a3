// Prefill-sized grouped GEMMs (bf16 MFMA over MXFP4 or int4-g32 weights):
// the super-block pass, the 4-wave kernels, the launcher and (through it) the
// MXFP4 single-wave kernels. The tile design is described in
// prefill_tile.hpp; the int4 single-wave kernels are built in
// gemm_prefill_int4.hip.
#include "prefill_tile.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// Super-blocks: runs of consecutive blocks with the same expert, cut every
// maxb blocks. One 1024-thread workgroup; list[i] = {expert, first row, blocks}.
// Robust to any block order (a run is what it is, wherever it sits).
__global__ __launch_bounds__(1024) void superblock_kernel(const int32_t* __restrict__ block_expert,
                                                         int nblocks, int E, int maxb, int4* __restrict__ list,
                                                         int* __restrict__ count) {
    __shared__ int wred[16];
    __shared__ int carry_run, carry_cnt;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    if (tid == 0) {
        carry_run = 0;
        carry_cnt = 0;
    }
    __syncthreads();
    for (int base = 0; base < nblocks; base += 1024) {
        const int b = base + tid;
        const int e = b < nblocks ? block_expert[b] : -1;
        const bool run_start = b < nblocks && (b == 0 || block_expert[b - 1] != e);
        // Inclusive max-scan of run starts: the first block of b's run.
        int v = run_start ? b : -1;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int o = __shfl_up(v, off);
            if (lane >= off) v = max(v, o);
        }
        if (lane == 63) wred[wv] = v;
        __syncthreads();
        int rs = carry_run;
        for (int w = 0; w < wv; ++w) rs = max(rs, wred[w]);
        rs = max(rs, v);
        const bool start = (unsigned)e < (unsigned)E && ((b - rs) % maxb) == 0;
        // Inclusive count scan of super-block starts.
        int c = start ? 1 : 0;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int o = __shfl_up(c, off);
            if (lane >= off) c += o;
        }
        __syncthreads();
        if (lane == 63) wred[wv] = c;
        __syncthreads();
        int cb = carry_cnt;
        for (int w = 0; w < wv; ++w) cb += wred[w];
        if (start) {
            int nb = 1;
            while (nb < maxb && b + nb < nblocks && block_expert[b + nb] == e) ++nb;
            list[cb + c - 1] = make_int4(e, b * kPfBlockRows, nb, 0);
        }
        __syncthreads();
        if (tid == 1023) {
            carry_run = rs;
            carry_cnt = cb + c;
        }
        __syncthreads();
    }
    if (tid == 0) *count = carry_cnt;
}

// EPI: stage 1 with the optional expert-bias / clamp epilogue.
template <int STAGE, int FMT, int NBMAX, bool EPI>
__global__ __launch_bounds__(kPfThreads, NBMAX <= 2 ? 2 : 1) void prefill_kernel(MoeGemmArgs a,
                                                                               const int4* __restrict__ list,
                                                                               const int* __restrict__ count,
                                                                               int ntiles) {
    __shared__ PfShared<NBMAX> sh;
    // Workgroup id -> (super-block, N tile): ids go round-robin over the 8
    // XCDs, so super-block s lives on XCD s % 8 with all of its N tiles.
    const int b = blockIdx.x;
    const int xcd = b & 7, j = b >> 3;
    const int s = 8 * (j / ntiles) + xcd;
    const int nt = j % ntiles;
    if (s >= *count) return;
    const int4 sb = list[s];
    const int e = sb.x, row0 = sb.y, nb = sb.z;
    for (int r = threadIdx.x; r < NBMAX * kPfBlockRows; r += kPfThreads)
        sh.rows[r] = r < nb * kPfBlockRows ? a.sorted_ids[row0 + r] : -1;
    __syncthreads();
    const int n0 = nt * (STAGE == 1 ? 128 : 256);
    if constexpr (NBMAX <= 2) {
        if (nb == 1) pf_tile<STAGE, FMT, 1, false, PfShared<NBMAX>, EPI>(a, sh, e, row0, n0);
        else pf_tile<STAGE, FMT, 2, false, PfShared<NBMAX>, EPI>(a, sh, e, row0, n0);
    } else {
        switch (nb) {
            case 1: pf_tile<STAGE, FMT, 1, false, PfShared<NBMAX>, EPI>(a, sh, e, row0, n0); break;
            case 2: pf_tile<STAGE, FMT, 2, false, PfShared<NBMAX>, EPI>(a, sh, e, row0, n0); break;
            case 3: pf_tile<STAGE, FMT, 3, false, PfShared<NBMAX>, EPI>(a, sh, e, row0, n0); break;
            case 4: pf_tile<STAGE, FMT, 4, false, PfShared<NBMAX>, EPI>(a, sh, e, row0, n0); break;
            case 5: pf_tile<STAGE, FMT, 5, false, PfShared<NBMAX>, EPI>(a, sh, e, row0, n0); break;
            case 6: pf_tile<STAGE, FMT, 6, false, PfShared<NBMAX>, EPI>(a, sh, e, row0, n0); break;
            case 7: pf_tile<STAGE, FMT, 7, false, PfShared<NBMAX>, EPI>(a, sh, e, row0, n0); break;
            default: pf_tile<STAGE, FMT, 8, false, PfShared<NBMAX>, EPI>(a, sh, e, row0, n0); break;
        }
    }
}

bool prefill_eligible(const MoeGemmArgs& a) {
    return (a.fmt == kFmtMxfp4 || a.fmt == kFmtInt4g32) && a.bm == kPfBlockRows && a.H % 256 == 0 &&
           a.I % 256 == 0 && (int64_t)2 * a.I * (a.H / 32) * 2 < 0x7fff0000LL &&
           (int64_t)a.T * a.topk * a.H * 4 < 0x7fff0000LL &&
           a.cap * a.I * 2 < 0x7fff0000LL && (int64_t)a.T * a.H * 2 < 0x7fff0000LL &&
           (int64_t)2 * a.I * (a.H / 2) < 0x7fff0000LL;
}

int64_t prefill_list_bytes(int64_t cap) { return (cap / kPfBlockRows + 1) * 16 + 256; }

hipError_t launch_prefill(const MoeGemmArgs& a, int stage, void* list_ws, hipStream_t s) {
    int4* list = (int4*)list_ws;
    const int64_t nblocks = a.cap / kPfBlockRows;
    const int direct_max = stage == 2 ? kPfDirectMaxTokens2
                           : a.fmt == kFmtMxfp4 ? kPfDirectMaxTokens1 : kPfDirectMaxTokens1Int4;
    if (a.T <= direct_max) {
        const int ntiles = stage == 1 ? a.I / 32 : a.H / 64;
        const dim3 grid((unsigned)(8 * ((nblocks + 7) / 8) * ntiles)), block(64);
        if (a.fmt == kFmtMxfp4) {
            if (stage == 1) hipLaunchKernelGGL((prefill_direct_kernel<1, kFmtMxfp4>), grid, block, 0, s, a, (int)nblocks, ntiles);
            else hipLaunchKernelGGL((prefill_direct_kernel<2, kFmtMxfp4>), grid, block, 0, s, a, (int)nblocks, ntiles);
        } else {
            return launch_prefill_direct_int4(a, stage, grid, (int)nblocks, ntiles, s);
        }
        return hipGetLastError();
    }
    int* count = (int*)(list + nblocks);
    // Few rows per expert (decode batches): 64-row super-blocks and a small
    // LDS footprint, so two workgroups share a CU and keep more weight bytes
    // in flight. Both stages take the same choice from the same sizes.
    const int64_t P = (int64_t)a.T * a.topk;
    const int64_t touched = P < a.E ? P : a.E;
    const int maxb = P <= 48 * touched ? kPfMaxBlocksSmall : kPfMaxBlocks;
    if (stage == 1)
        hipLaunchKernelGGL(superblock_kernel, dim3(1), dim3(1024), 0, s, a.block_expert, (int)nblocks, a.E,
                           maxb, list, count);
    // Super-blocks: sum over experts of ceil(rows / (32 maxb)) <= P / (32 maxb) + min(E, P) + 1.
    int64_t sbound = P / (maxb * kPfBlockRows) + touched + 1;
    if (sbound > nblocks) sbound = nblocks;
    const int ntiles = stage == 1 ? a.I / 128 : a.H / 256;
    const int64_t grid = 8 * ((sbound + 7) / 8) * ntiles;
    const bool epi = stage == 1 && (a.w13_bias || a.swiglu_limit > 0.0f);
#define MOE_PF_LAUNCH(ST, F, NBM, EP) \
    hipLaunchKernelGGL((prefill_kernel<ST, F, NBM, EP>), dim3((unsigned)grid), dim3(kPfThreads), 0, s, a, list, count, ntiles)
#define MOE_PF_LAUNCH_F(ST, NBM, EP)                                   \
    do {                                                               \
        if (a.fmt == kFmtMxfp4) MOE_PF_LAUNCH(ST, kFmtMxfp4, NBM, EP); \
        else MOE_PF_LAUNCH(ST, kFmtInt4g32, NBM, EP);                 \
    } while (0)
    if (maxb == kPfMaxBlocksSmall) {
        if (stage == 2) MOE_PF_LAUNCH_F(2, kPfMaxBlocksSmall, false);
        else if (epi) MOE_PF_LAUNCH_F(1, kPfMaxBlocksSmall, true);
        else MOE_PF_LAUNCH_F(1, kPfMaxBlocksSmall, false);
    } else {
        if (stage == 2) MOE_PF_LAUNCH_F(2, kPfMaxBlocks, false);
        else if (epi) MOE_PF_LAUNCH_F(1, kPfMaxBlocks, true);
        else MOE_PF_LAUNCH_F(1, kPfMaxBlocks, false);
    }
#undef MOE_PF_LAUNCH_F
#undef MOE_PF_LAUNCH
    return hipGetLastError();
}

}  // namespace moe

// Single-wave int4-g32 tiles (prefill_direct_kernel<., INT4G32>, decode
// batches of 9-32 tokens over requantized weights).
//
// This file is built with -mllvm -amdgpu-mfma-vgpr-form=1: the group-scaled
// k-loop reads every MFMA result back (acc += s * (group sum - 136 * row
// sum), once per 32-group), and with the results in AGPRs each of those reads
// was a v_accvgpr_read (192 of 656 VALU operations per stage). With the
// results in VGPRs they disappear; the kernel stays at 256 registers, two
// waves per SIMD. The option is per file because the 4-wave kernels, whose
// accumulators are only read in the epilogue, need AGPRs for their 256
// accumulator registers.
#include "prefill_tile.hpp"

namespace moe {

hipError_t launch_prefill_direct_int4(const MoeGemmArgs& a, int stage, dim3 grid, int nblocks, int ntiles,
                                      hipStream_t s) {
    if (stage == 1) hipLaunchKernelGGL((prefill_direct_kernel<1, kFmtInt4g32>), grid, dim3(64), 0, s, a, nblocks, ntiles);
    else hipLaunchKernelGGL((prefill_direct_kernel<2, kFmtInt4g32>), grid, dim3(64), 0, s, a, nblocks, ntiles);
    return hipGetLastError();
}

}  // namespace moe

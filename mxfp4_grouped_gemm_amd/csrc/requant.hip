// MXFP4 -> int4 per-group-32 requantization (load time, opt-in).
//
// convert() in Mxfp4MoEMethod._setup_kernel_k3_situ_gfx942 (vLLM mxfp4 API
// page) decodes the packed e2m1 weight to float, multiplies each 32-block by
// its e8m0 scale, casts to bf16 and quantizes every 1x32 group to int4 with
// one bf16 scale; the pull request converts eight experts per call to bound
// the memory that a whole-tensor unpack (8x the packed size) would take.
// Here one thread owns one 32-group: a 16-byte load of 32 codes, the gfx950
// scaled fp4 -> bf16 converts, amax, scale = bf16(amax / 7) from an IEEE
// fp32 divide, codes = clamp(rint(v / scale), -8, 7) (ties to even), and a
// 16-byte store of the packed codes. Nothing is staged: the only memory
// touched is the source range and the preallocated outputs.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

__global__ __launch_bounds__(256) void requant_kernel(const uint8_t* __restrict__ w,
                                                      const uint8_t* __restrict__ scale, int64_t g0,
                                                      int64_t ngroups, uint8_t* __restrict__ q,
                                                      uint16_t* __restrict__ qs) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < ngroups;
         i += (int64_t)gridDim.x * 256) {
        const int64_t gi = g0 + i;
        const u32x4 d = *(const u32x4*)(w + gi * 16);
        const float sc = e8m0_scale_operand(scale[gi]);
        float v[32];
        float amax = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const bf16x8 b = mxfp4x8_to_bf16(d[k], sc);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                v[8 * k + j] = (float)b[j];
                amax = fmaxf(amax, fabsf(v[8 * k + j]));
            }
        }
        const uint16_t sbits = f32_to_bf16_bits(amax / 7.0f);
        const float sf = bf16_bits_to_f32(sbits);
        u32x4 packed = {0u, 0u, 0u, 0u};
        if (sf != 0.0f) {
#pragma unroll
            for (int k = 0; k < 32; ++k) {
                float r = rintf(v[k] / sf);
                r = fminf(fmaxf(r, -8.0f), 7.0f);
                const uint32_t nib = (uint32_t)((int)r) & 0xFu;
                packed[k >> 3] |= nib << (4 * (k & 7));
            }
        }
        *(u32x4*)(q + gi * 16) = packed;
        qs[gi] = sbits;
    }
}

hipError_t launch_requant(const uint8_t* w, const uint8_t* scale, int N, int K, int lo, int hi,
                          uint8_t* q, uint16_t* qs, hipStream_t s) {
    const int64_t gpr = K / 32;
    const int64_t g0 = (int64_t)lo * N * gpr;
    const int64_t n = (int64_t)(hi - lo) * N * gpr;
    if (n == 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 256 * 32) blocks = 256 * 32;
    hipLaunchKernelGGL(requant_kernel, dim3((unsigned)blocks), dim3(256), 0, s, w, scale, g0, n, q, qs);
    return hipGetLastError();
}

}  // namespace moe

// MXFP4 -> int4 per-group-32 requantization (load time, opt-in).
//
// convert() in Mxfp4MoEMethod._setup_kernel_k3_situ_gfx942 (vLLM mxfp4 API
// page) decodes the packed e2m1 weight to float, multiplies each 32-block by
// its e8m0 scale, casts to bf16 and quantizes every 1x32 group to int4 with
// one bf16 scale; the pull request converts eight experts per call to bound
// the memory that a whole-tensor unpack (8x the packed size) would take.
// Here one thread owns one 32-group: a 16-byte load of 32 codes, scale =
// bf16(amax / 7) from an IEEE fp32 divide, codes = clamp(rint(v / scale),
// -8, 7) (ties to even) -- through the table below where the exponent allows,
// else from the decoded values with a divide per element -- and a 16-byte
// store of the packed codes. Nothing is staged: the only memory touched is
// the source range and the preallocated outputs.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

// In the normal exponent range the group's power of two cancels: with
// v = m * 2^a and amax = M * 2^a (m, M e2m1 magnitudes, a = s - 127), the
// fp32 quotient amax / 7 and its bf16 rounding are those of M / 7 times 2^a,
// and v / scale is exactly m / bf16(M / 7). So a code depends only on its
// nibble and on the group's largest magnitude code: an 8 x 16 table, built
// at compile time from the same rule (IEEE fp32 divide, bf16 RNE, rint ties
// to even, clamp to [-8, 7]), looked up four codes at a time with byte
// permutes. That holds for e8m0 bytes 5..252 (M / 7 * 2^a
// stays a normal float, m * 2^a stays finite); other bytes take the divide.
namespace rq {
constexpr float kMag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
constexpr float bf16_rne(float f) {  // finite f
    const uint32_t u = __builtin_bit_cast(uint32_t, f);
    return __builtin_bit_cast(float, (u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u);
}
constexpr float rint_even(float x) {  // |x| < 2^31
    long long t = (long long)x;  // toward zero
    const float fr = x - (float)t;
    if (fr > 0.5f) ++t;
    else if (fr < -0.5f) --t;
    else if (fr == 0.5f) t += (t & 1);
    else if (fr == -0.5f) t -= (t & 1);
    return (float)t;
}
constexpr uint64_t row(int mi) {
    const float s0 = bf16_rne(kMag[mi] / 7.0f);
    uint64_t r = 0;
    if (s0 == 0.0f) return 0;
    for (int n = 0; n < 16; ++n) {
        const float v = (n & 8) ? -kMag[n & 7] : kMag[n & 7];
        float q = rint_even(v / s0);
        q = q < -8.0f ? -8.0f : q > 7.0f ? 7.0f : q;
        r |= (uint64_t)((uint32_t)(int)q & 0xFu) << (4 * n);
    }
    return r;
}
// Byte tables for v_perm_b32: entry mi holds the codes (low nibble of each
// byte) of magnitudes 0..7 for positive nibbles (words 0-1) and negative
// nibbles (words 2-3).
constexpr uint32_t word(int mi, int neg, int half) {
    const uint64_t r = row(mi);
    uint32_t w = 0;
    for (int b = 0; b < 4; ++b) w |= (uint32_t)((r >> (4 * (8 * neg + 4 * half + b))) & 0xFu) << (8 * b);
    return w;
}
struct Lut {
    uint32_t w[8][4];
};
constexpr Lut make_lut() {
    Lut l{};
    for (int mi = 0; mi < 8; ++mi)
        for (int k = 0; k < 4; ++k) l.w[mi][k] = word(mi, k >> 1, k & 1);
    return l;
}
constexpr Lut kLut = make_lut();
}  // namespace rq

// Largest magnitude code (0..7) over the 32 nibbles of a group, bit by bit:
// keep the nibbles that have the highest bit any of them has.
__device__ __forceinline__ uint32_t max_mag(const u32x4& d) {
    uint32_t m[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) m[k] = d[k] & 0x77777777u;
    uint32_t mi = 0;
#pragma unroll
    for (int bit = 2; bit >= 0; --bit) {
        const uint32_t sel = 0x11111111u << bit;
        const uint32_t any = (m[0] | m[1] | m[2] | m[3]) & sel;
        if (any) {
            mi |= 1u << bit;
#pragma unroll
            for (int k = 0; k < 4; ++k) m[k] &= ((m[k] & sel) >> bit) * 0xFu;  // nibbles with the bit
        }
    }
    return mi;
}

__global__ __launch_bounds__(256) void requant_kernel(const uint8_t* __restrict__ w,
                                                      const uint8_t* __restrict__ scale, int64_t g0,
                                                      int64_t ngroups, uint8_t* __restrict__ q,
                                                      uint16_t* __restrict__ qs) {
    __shared__ u32x4 lut[8];
    if (threadIdx.x < 8)
        lut[threadIdx.x] = u32x4{rq::kLut.w[threadIdx.x][0], rq::kLut.w[threadIdx.x][1],
                                 rq::kLut.w[threadIdx.x][2], rq::kLut.w[threadIdx.x][3]};
    __syncthreads();
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < ngroups;
         i += (int64_t)gridDim.x * 256) {
        const int64_t gi = g0 + i;
        // Every byte is read and written once: streaming (nt) accesses.
        const u32x4 d = __builtin_nontemporal_load((const u32x4*)(w + gi * 16));
        const uint32_t sb = __builtin_nontemporal_load(scale + gi);
        u32x4 packed = {0u, 0u, 0u, 0u};
        uint16_t sbits;
        if (sb >= 5u && sb <= 252u) {
            const uint32_t mi = max_mag(d);
            const u32x4 t = lut[mi];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                // even nibbles in the low half of each byte, odd in the high
                const uint32_t se = d[k] & 0x07070707u, so = (d[k] >> 4) & 0x07070707u;
                const uint32_t ne = ((d[k] >> 3) & 0x01010101u) * 0xFFu;  // negative even nibbles
                const uint32_t no = ((d[k] >> 7) & 0x01010101u) * 0xFFu;
                const uint32_t ce = (__builtin_amdgcn_perm(t[3], t[2], se) & ne) |
                                    (__builtin_amdgcn_perm(t[1], t[0], se) & ~ne);
                const uint32_t co = (__builtin_amdgcn_perm(t[3], t[2], so) & no) |
                                    (__builtin_amdgcn_perm(t[1], t[0], so) & ~no);
                packed[k] = (ce & 0x0F0F0F0Fu) | ((co & 0x0F0F0F0Fu) << 4);
            }
            // amax = M * 2^a exactly (M: the e2m1 magnitude of code mi)
            const float mag = mi == 7 ? 6.0f : mi == 6 ? 4.0f : mi == 5 ? 3.0f : 0.5f * (float)mi;
            sbits = f32_to_bf16_bits(__builtin_amdgcn_ldexpf(mag, (int)sb - 127) / 7.0f);
        } else {
            const float sc = e8m0_scale_operand(sb);
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
            sbits = f32_to_bf16_bits(amax / 7.0f);
            const float sf = bf16_bits_to_f32(sbits);
            if (sf != 0.0f) {
#pragma unroll
                for (int k = 0; k < 32; ++k) {
                    float r = rintf(v[k] / sf);
                    r = fminf(fmaxf(r, -8.0f), 7.0f);
                    const uint32_t nib = (uint32_t)((int)r) & 0xFu;
                    packed[k >> 3] |= nib << (4 * (k & 7));
                }
            }
        }
        __builtin_nontemporal_store(packed, (u32x4*)(q + gi * 16));
        __builtin_nontemporal_store(sbits, qs + gi);
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

// Shared device-side types and helpers for the gfx950 (CDNA4) kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Weight formats (values match moe_wfmt).
constexpr int kFmtMxfp4 = 0;
constexpr int kFmtInt4g32 = 1;

// The e8m0 block scale 2^(s-127) as the float operand of the gfx950 scaled
// fp4 converts. Those instructions use only the exponent of that operand,
// so the scale is applied exactly; s == 0 needs the subnormal 2^-127.
__device__ __forceinline__ float e8m0_scale_operand(uint32_t s) {
    return __uint_as_float(s ? (s << 23) : 0x00400000u);
}

// Eight e2m1 values packed in one dword (element 2b in the low nibble of
// byte b) -> eight bf16 in k order, each multiplied by the block scale.
// v_cvt_scalef32_pk_bf16_fp4 converts one byte (low nibble first).
__device__ __forceinline__ bf16x8 mxfp4x8_to_bf16(uint32_t d, float scale) {
    bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 0);
    bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 1);
    bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 2);
    bf16x2 e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 3);
    bf16x4 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3);
    bf16x4 ce = __builtin_shufflevector(c, e, 0, 1, 2, 3);
    return __builtin_shufflevector(ab, ce, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Eight two's-complement int4 codes packed in one dword -> eight bf16
// holding (code + 136), i.e. 128 + (code ^ 8), exactly. The nibble lands in
// the low mantissa bits of 128.0 (bf16 0x4300, ulp 1). Output element
// order: nibbles {0, 4, 1, 5, 2, 6, 3, 7} -- the activation operand must use
// the same permutation (see perm_x_int4).
//
// One v_bitop3 per output dword (after a shift): with s = d >> 4i, bit p of
// the result is 1 where 0x4300 has ones, NOT s[p] at the nibble's top bit
// (code ^ 8), s[p] at its three low bits and 0 elsewhere. The two constant
// operands mark these four kinds of positions (B: "1" or "not s", C: "1" or
// "s"), and the truth table 0xAC selects: B C = 00 -> 0, 01 -> s, 10 -> !s,
// 11 -> 1 (table index = 4 s + 2 B + C).
__device__ __forceinline__ bf16x8 int4x8_to_bf16_biased(uint32_t d) {
    constexpr uint32_t kB = 0x43084308u, kC = 0x43074307u;
    u32x4 r;
    r[0] = __builtin_amdgcn_bitop3_b32(d, kB, kC, 0xAC);
    r[1] = __builtin_amdgcn_bitop3_b32(d >> 4, kB, kC, 0xAC);
    r[2] = __builtin_amdgcn_bitop3_b32(d >> 8, kB, kC, 0xAC);
    r[3] = __builtin_amdgcn_bitop3_b32(d >> 12, kB, kC, 0xAC);
    return __builtin_bit_cast(bf16x8, r);
}

// Reorder eight bf16 activations (k order 0..7) into the nibble order that
// int4x8_to_bf16_biased produces: {0, 4, 1, 5, 2, 6, 3, 7}.
__device__ __forceinline__ bf16x8 perm_x_int4(bf16x8 v) {
    return __builtin_shufflevector(v, v, 0, 4, 1, 5, 2, 6, 3, 7);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    __bf16 h = (__bf16)f;
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

// Eight two's-complement int4 codes (element e in nibble e, low nibble
// first) times a bf16 group scale, split exactly into two bf16 vectors:
// q * s is exact in fp32 but can need 11 significant bits; hi = bf16(q*s)
// (RNE) and lo = q*s - hi (at most 3 significant bits, exact in bf16), so a
// bf16 MFMA over hi and then lo sees the exact weight.
__device__ __forceinline__ void int4x8_to_bf16_hilo(uint32_t d, float s, bf16x8& hi, bf16x8& lo) {
    u32x4 h, l;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float f0 = (float)((int)(d << (28 - 8 * k)) >> 28) * s;
        const float f1 = (float)((int)(d << (24 - 8 * k)) >> 28) * s;
        const uint32_t hp = pack_bf16x2(f0, f1);
        h[k] = hp;
        l[k] = pack_bf16x2(f0 - __uint_as_float(hp << 16), f1 - __uint_as_float(hp & 0xffff0000u));
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Raw buffer resources. A load whose offset is past the record count returns
// zeros without touching memory, which gives masked loads without control
// flow; kOob is past every record used here (records stay below 2^31).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOob = 0x80000000u;
constexpr int kNt = 2;  // cache-policy operand of a buffer load: the nt bit

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bld16(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ u32x2 bld8(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
// Streaming loads (nt): for bytes read once per launch (weight codes and
// scales), so they do not displace the activations that every wave re-reads
// from L2. A plain read of 175 MB streams about 7 % faster this way, and so
// do the GEMV kernels, whose loads are 1 KB runs of one row; the MFMA tiles,
// which read 128-byte pieces of 64 rows, were 5-20 % slower with nt.
__device__ __forceinline__ u32x4 bld16nt(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNt));
}
__device__ __forceinline__ u32x2 bld8nt(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kNt));
}
// The same with a wave-uniform part of the offset in the scalar operand
// (no per-lane address arithmetic). Only the vector part is checked against
// the record count, so callers keep every access inside the buffer (the
// scalar part is clamped) and put kOob in the vector part to mask a lane.
__device__ __forceinline__ u32x4 bld16s(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ u32x2 bld8s(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}

__device__ __forceinline__ u32x4 bld16snt(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kNt));
}

// Orders one wave's LDS writes before its later LDS reads (LDS executes a
// wave's operations in order; this keeps the compiler from reordering them).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// silu(g) * u in fp32. For very negative g, expf(-g) overflows to +inf and
// the quotient is -0 (never NaN).
__device__ __forceinline__ float swiglu(float g, float u) {
    return g / (1.0f + expf(-g)) * u;
}

// The same with the hardware exp2 and reciprocal (about 1 ulp each): for
// epilogues with many outputs per lane. Very negative g: exp overflows to
// +inf, the reciprocal is 0 and the result -0.
__device__ __forceinline__ float swiglu_fast(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

}  // namespace moe

// common.hpp -- device-side building blocks for the gfx950 kernels of libwqmoe:
// vector types, MFMA wrappers, in-register dequantisation of the packed int4 /
// int8 weights, 16-bit float conversions.
//
// MFMA operand layouts on gfx950 (verified on the hardware with known inputs):
//   v_mfma_f32_16x16x32_{f16,bf16}: lane l holds A[row l%16][k 8*(l/16)+v],
//     B[k 8*(l/16)+v][col l%16] for v < 8; D[row 4*(l/16)+r][col l%16], r < 4.
//   v_mfma_f32_32x32x16_{f16,bf16}: lane l holds A[row l%32][k 8*(l/32)+v],
//     B[k 8*(l/32)+v][col l%32]; D[row 8*(r/4)+4*(l/32)+r%4][col l%32], r < 16.
//   v_smfmac_f32_16x16x64_f16 (A 2:4 sparse): lane l holds the 8 kept A values
//     of row l%16 for dense k in [16*(l/16), +16), two per group of 4 in
//     ascending position; B[k][col l%16] with k = 8*(l/16)+v for v < 8 and
//     32+8*(l/16)+(v-8) for v >= 8; the index operand carries, per group g of
//     the lane's four, the first kept position in bits [4g+1:4g] and the second
//     in [4g+3:4g+2] (low 16 bits with ABID 0, high 16 bits with ABID 1).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace wq {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// MFMA wrappers: operands are 8 packed 16-bit values in 4 dwords.
// ---------------------------------------------------------------------------
template <bool BF16>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                       0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                      0, 0);
}

template <bool BF16>
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                       0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                      0, 0);
}

// 2:4-sparse A (8 kept fp16 values) x dense B (16 fp16 values), index half ABID
template <int ABID>
__device__ __forceinline__ f32x4 smfmac16x16x64(u32x4 a, u32x8 b, int idx, f32x4 c) {
    return __builtin_amdgcn_smfmac_f32_16x16x64_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x16, b), c,
                                                    idx, 0, ABID);
}

// ---------------------------------------------------------------------------
// 16-bit float conversions (round to nearest even)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float f16_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ uint16_t f32_to_f16(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));  // inf / nan
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
template <bool BF16>
__device__ __forceinline__ float act_to_f32(uint16_t h) {
    if constexpr (BF16) return bf16_to_f32(h);
    else return f16_to_f32(h);
}
template <bool BF16>
__device__ __forceinline__ uint16_t f32_to_act(float f) {
    if constexpr (BF16) return f32_to_bf16(f);
    else return f32_to_f16(f);
}

// ---------------------------------------------------------------------------
// int4 codes -> fp16.  A packed dword holds 8 offset-binary nibbles u = q + 8
// for consecutive input channels j = 0..7, nibble j at bit 4*(j>>1)+16*(j&1),
// so that d & 0x000F000F isolates channels (0, 1) as the low bits of the two
// halves and d & 0x00F000F0 channels (2, 3) as bits 4..7 (and d >> 8 the same
// for channels 4..7).  OR-ing the exponent of 1024 (0x6400) gives 1024 + u, or
// 1024 + 16u for the upper nibble of a byte, exactly; 1024 + u - 1032 = q and
// (1024 + 16u) / 16 - 72 = q are exact in fp16.  9 VALU ops per 8 codes.
// This is the published fast integer-to-half conversion with an interleaved
// nibble order (Kim et al., "Who Says Elephants Can't Run: Bringing Large
// Scale MoE Models into Cloud Scale Production", 2022), the conversion the
// Marlin kernels also use; the mask and bias constants follow from the fp16
// encoding of 1024 + u and are fixed by the method.
// ---------------------------------------------------------------------------
// (16-bit float arithmetic on a dword holding two halves; only scalars are
// bit-cast: a bit-cast of an ext-vector element reads the vector's first dword)
__device__ __forceinline__ uint32_t f16x2_sub(uint32_t v, f16x2 b) {
    const f16x2 h = __builtin_bit_cast(f16x2, v);
    return __builtin_bit_cast(uint32_t, h - b);
}
__device__ __forceinline__ uint32_t f16x2_mul(uint32_t v, f16x2 b) {
    const f16x2 h = __builtin_bit_cast(f16x2, v);
    return __builtin_bit_cast(uint32_t, h * b);
}
__device__ __forceinline__ uint32_t f16x2_fma(uint32_t v, f16x2 a, f16x2 b) {
    const f16x2 h = __builtin_bit_cast(f16x2, v);
    return __builtin_bit_cast(uint32_t, h * a + b);
}

// (a & m) | c in one v_and_or_b32.  A gfx9 VOP3 instruction takes no literal
// constant, so the compiler splits the expression into v_and_b32 + v_or_b32
// with literals; with the constants in VGPRs it is one instruction.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(c));
    return r;
}

__device__ __forceinline__ u32x4 dequant_w4_f16(uint32_t d) {
    const uint32_t magic = 0x64006400u;
    const f16x2 bias = {(_Float16)1032.0f, (_Float16)1032.0f};
    const f16x2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const f16x2 bias16 = {(_Float16)-72.0f, (_Float16)-72.0f};
    const uint32_t h = d >> 8;
    const uint32_t p0 = and_or(d, 0x000F000Fu, magic);  // 1024 + u, channels 0, 1
    const uint32_t p1 = and_or(d, 0x00F000F0u, magic);  // 1024 + 16u, channels 2, 3
    const uint32_t p2 = and_or(h, 0x000F000Fu, magic);
    const uint32_t p3 = and_or(h, 0x00F000F0u, magic);
    return u32x4{f16x2_sub(p0, bias), f16x2_fma(p1, sixteenth, bias16), f16x2_sub(p2, bias),
                 f16x2_fma(p3, sixteenth, bias16)};
}

// same, times one fp16 scale (q * s rounded once to fp16)
__device__ __forceinline__ u32x4 dequant_w4_f16_scaled(uint32_t d, f16x2 s2) {
    const u32x4 r = dequant_w4_f16(d);
    const uint32_t r0 = r[0], r1 = r[1], r2 = r[2], r3 = r[3];
    return u32x4{f16x2_mul(r0, s2), f16x2_mul(r1, s2), f16x2_mul(r2, s2), f16x2_mul(r3, s2)};
}

// ---------------------------------------------------------------------------
// int8 codes -> 16-bit floats.  Bytes are the two's-complement codes q,
// consecutive input channels in consecutive bytes.
//  bf16: q converts to float exactly in one instruction (a sign-extending
//        byte-select of the source operand feeds the int->float convert); q
//        has at most 8 significant bits, so the upper half of its float32
//        pattern is q in bf16 exactly.
//  f16:  with u = q ^ 0x80 = q + 128, the half with bits 0x64uu is 1024 + u
//        exactly; minus 1152 gives q.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t pack_hi16(float lo, float hi) {
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

__device__ __forceinline__ u32x2 dequant_w8x4_bf16(uint32_t d) {
    const float f0 = (float)(signed char)(d & 0xffu);
    const float f1 = (float)(signed char)((d >> 8) & 0xffu);
    const float f2 = (float)(signed char)((d >> 16) & 0xffu);
    const float f3 = (float)((int)d >> 24);
    u32x2 r;
    r[0] = pack_hi16(f0, f1);
    r[1] = pack_hi16(f2, f3);
    return r;
}

__device__ __forceinline__ u32x2 dequant_w8x4_f16(uint32_t d) {
    const f16x2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
    const uint32_t u = d ^ 0x80808080u;
    const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, u, 0x05010400u);  // bytes [u0, 64, u1, 64]
    const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, u, 0x05030402u);  // bytes [u2, 64, u3, 64]
    return u32x2{f16x2_sub(lo, bias), f16x2_sub(hi, bias)};
}

template <bool BF16>
__device__ __forceinline__ u32x4 dequant_w8x8(uint32_t d0, uint32_t d1) {
    u32x2 a, b;
    if constexpr (BF16) {
        a = dequant_w8x4_bf16(d0);
        b = dequant_w8x4_bf16(d1);
    } else {
        a = dequant_w8x4_f16(d0);
        b = dequant_w8x4_f16(d1);
    }
    u32x4 r;
    r[0] = a[0];
    r[1] = a[1];
    r[2] = b[0];
    r[3] = b[1];
    return r;
}

// ---------------------------------------------------------------------------
// misc
// ---------------------------------------------------------------------------
// calls f(std::integral_constant<int, i>) for i in [B, E), unrolled
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

__device__ __forceinline__ u32x4 ldg128(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x4 ldg128_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ float silu_f32(float a) { return a / (1.0f + __expf(-a)); }

// first index in [lo, hi) with v[idx] >= key (v non-decreasing on [lo, hi))
__device__ __forceinline__ int lower_bound_i32(const int32_t* v, int lo, int hi, int key) {
    while (lo < hi) {
        int mid = (lo + hi) >> 1;
        if (v[mid] < key) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

}  // namespace wq

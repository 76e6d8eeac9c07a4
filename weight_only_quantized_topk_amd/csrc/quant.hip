// quant.hip -- ExpertsInt8 load-time quantization of 16-bit expert weights.
//
// "[Kernel] W8A16 Int8 inside FusedMoE" (vLLM PR 7415), opening description:
// symmetric per-column, per-expert int8 weights whose scales are extracted
// when the model loads ("How to convert models to ExpertsInt8?": quantization
// on the fly).  Per row of k weights (one expert's output column):
//   s32 = max |w| / 127 (float32, correctly rounded division)
//   s   = s32 rounded to the 16-bit type, nearest-even   (the stored scale)
//   q   = w / s rounded half-to-even, clamped to +-127   (float32 division)
// and q = 0 where s = 0, so q * s is the nearest int8 multiple of the stored
// scale.  One wave per row: the row's 128-bit loads all issued at once into
// registers (rows up to 16384 weights), the absolute maximum reduced across
// the wave by lane shuffles, then the codes from the same registers, 64-bit
// stores.  HBM-bound: 2k bytes read and k + 2 written per row.
#include "common.hpp"
#include "launch.hpp"

namespace wq {

template <bool BF16>
__device__ __forceinline__ uint32_t quant_code(uint16_t h, float sv) {
    if (sv == 0.0f) return 0u;
    float t = rintf(act_to_f32<BF16>(h) / sv);
    t = fminf(fmaxf(t, -127.0f), 127.0f);
    return (uint32_t)(int32_t)t & 0xffu;
}

template <bool BF16>
__device__ __forceinline__ u32x2 quant_piece(u32x4 v, float sv) {
    u32x2 out;
#pragma unroll
    for (int d = 0; d < 2; ++d) {
        const uint32_t a = v[2 * d], b = v[2 * d + 1];
        out[d] = quant_code<BF16>((uint16_t)(a & 0xffffu), sv) | (quant_code<BF16>((uint16_t)(a >> 16), sv) << 8) |
                 (quant_code<BF16>((uint16_t)(b & 0xffffu), sv) << 16) |
                 (quant_code<BF16>((uint16_t)(b >> 16), sv) << 24);
    }
    return out;
}

template <bool BF16>
__device__ __forceinline__ float abs_max8(u32x4 v, float mx) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t u = v[d];
        mx = fmaxf(mx, fabsf(act_to_f32<BF16>((uint16_t)(u & 0xffffu))));
        mx = fmaxf(mx, fabsf(act_to_f32<BF16>((uint16_t)(u >> 16))));
    }
    return mx;
}

// wave-wide max, then the stored scale and its float value
template <bool BF16>
__device__ __forceinline__ float row_scale(float mx, uint16_t* s, int64_t r, int lane) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    const uint16_t sbits = f32_to_act<BF16>(mx / 127.0f);
    if (lane == 0) s[r] = sbits;
    return act_to_f32<BF16>(sbits);
}

// NCH > 0: rows of at most NCH * 512 weights held in registers, every load of
// the row in flight at once (indices past the row clamp to its last piece, whose
// duplicate codes are not stored); NCH == 0: any length, the code pass rereads
// the row from the cache
template <bool BF16, int NCH>
__global__ __launch_bounds__(256) void quant_w8_kernel(const uint16_t* __restrict__ w, int64_t rows, int k,
                                                       int8_t* __restrict__ q, uint16_t* __restrict__ s) {
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows) return;  // a whole wave
    const uint16_t* wr = w + r * k;
    int8_t* qr = q + r * k;
    float mx = 0.0f;
    if constexpr (NCH > 0) {
        const int last = k - 8;  // first channel of the row's last 8-channel piece
        u32x4 v[NCH];
#pragma unroll
        for (int c = 0; c < NCH; ++c) v[c] = ldg128(wr + min(8 * lane + 512 * c, last));
#pragma unroll
        for (int c = 0; c < NCH; ++c) mx = abs_max8<BF16>(v[c], mx);
        const float sv = row_scale<BF16>(mx, s, r, lane);
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int i = 8 * lane + 512 * c;
            if (i < k) *reinterpret_cast<u32x2*>(qr + i) = quant_piece<BF16>(v[c], sv);
        }
    } else {
        for (int i = 8 * lane; i < k; i += 512) mx = abs_max8<BF16>(ldg128(wr + i), mx);
        const float sv = row_scale<BF16>(mx, s, r, lane);
        for (int i = 8 * lane; i < k; i += 512) *reinterpret_cast<u32x2*>(qr + i) = quant_piece<BF16>(ldg128(wr + i), sv);
    }
}

template <bool BF16>
static void launch_quant(const uint16_t* w, int64_t rows, int k, int8_t* q, uint16_t* s, hipStream_t st) {
    const dim3 grid((unsigned)((rows + 3) / 4));
    if (k <= 4096) hipLaunchKernelGGL((quant_w8_kernel<BF16, 8>), grid, dim3(256), 0, st, w, rows, k, q, s);
    else if (k <= 16384) hipLaunchKernelGGL((quant_w8_kernel<BF16, 32>), grid, dim3(256), 0, st, w, rows, k, q, s);
    else hipLaunchKernelGGL((quant_w8_kernel<BF16, 0>), grid, dim3(256), 0, st, w, rows, k, q, s);
}

void launch_quant_w8(const uint16_t* w, int64_t rows, int k, bool bf16, int8_t* q, uint16_t* s, hipStream_t st) {
    if (bf16) launch_quant<true>(w, rows, k, q, s, st);
    else launch_quant<false>(w, rows, k, q, s, st);
}

}  // namespace wq

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
// scale.  One wave per row: a max pass, a wave reduction by lane shuffles, and
// a code pass that rereads the row (8 KiB at k = 4096, still in cache);
// 128-bit loads, 64-bit stores.  HBM-bound: 2k bytes read and k + 2 written
// per row.
#include "common.hpp"
#include "launch.hpp"

namespace wq {

template <bool BF16>
__global__ __launch_bounds__(256) void quant_w8_kernel(const uint16_t* __restrict__ w, int64_t rows, int k,
                                                       int8_t* __restrict__ q, uint16_t* __restrict__ s) {
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows) return;  // a whole wave
    const uint16_t* wr = w + r * k;

    float mx = 0.0f;
    for (int i = 8 * lane; i < k; i += 512) {
        const u32x4 v = ldg128(wr + i);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t u = v[d];
            mx = fmaxf(mx, fabsf(act_to_f32<BF16>((uint16_t)(u & 0xffffu))));
            mx = fmaxf(mx, fabsf(act_to_f32<BF16>((uint16_t)(u >> 16))));
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    const uint16_t sbits = f32_to_act<BF16>(mx / 127.0f);
    const float sv = act_to_f32<BF16>(sbits);
    if (lane == 0) s[r] = sbits;

    auto code = [&](uint16_t h) -> uint32_t {
        if (sv == 0.0f) return 0u;
        float t = rintf(act_to_f32<BF16>(h) / sv);
        t = fminf(fmaxf(t, -127.0f), 127.0f);
        return (uint32_t)(int32_t)t & 0xffu;
    };
    for (int i = 8 * lane; i < k; i += 512) {
        const u32x4 v = ldg128(wr + i);
        u32x2 out;
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const uint32_t a = v[2 * d], b = v[2 * d + 1];
            out[d] = code((uint16_t)(a & 0xffffu)) | (code((uint16_t)(a >> 16)) << 8) |
                     (code((uint16_t)(b & 0xffffu)) << 16) | (code((uint16_t)(b >> 16)) << 24);
        }
        *reinterpret_cast<u32x2*>(q + r * k + i) = out;
    }
}

void launch_quant_w8(const uint16_t* w, int64_t rows, int k, bool bf16, int8_t* q, uint16_t* s, hipStream_t st) {
    const dim3 grid((unsigned)((rows + 3) / 4));
    if (bf16) hipLaunchKernelGGL(quant_w8_kernel<true>, grid, dim3(256), 0, st, w, rows, k, q, s);
    else hipLaunchKernelGGL(quant_w8_kernel<false>, grid, dim3(256), 0, st, w, rows, k, q, s);
}

}  // namespace wq

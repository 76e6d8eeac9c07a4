// dense_decode.hip -- the dense single-expert linear layer at small batches.
//
// y[m, n] = sum_k x[m, k] W[n, k] for at most 4 token rows (the GEMV end of the
// batch-size dispatch of "[WIP] AWQ Faster Kernels", vLLM issue 3289).  The
// weights are the packed layout of the grouped GEMM with one expert: a 1 KiB
// chunk of a 16-row tile gives every lane the A operand of 2 (int8) or 4
// (int4) v_mfma_f32_16x16x32 steps.  One workgroup per 16-row tile; its NW
// waves split the tile's chunks (wave w takes chunks w, w + NW, ...), each
// keeping DEPTH chunks in flight.  The M token rows are staged in LDS once,
// before the chunk loop (rows padded by 16 bytes: the 16 column lanes of the B
// operand hit distinct banks; columns at or beyond M read row M - 1), so the
// loop's only global loads are the weight stream.  Numerics as the grouped
// small-batch kernel: int4 codes exact in fp16, the group scale applied to the
// fp32 partial sum of each 128-channel chunk; int8 exact, the per-column scale
// in the fp32 epilogue.  The NW partial sums are added in LDS in wave order and
// rounded once to the activation type.
#include "common.hpp"
#include "launch.hpp"

namespace wq {

template <int WBITS, bool BF16, int NW, int DEPTH>
__global__ __launch_bounds__(NW * 64) void dense_decode_kernel(const uint16_t* __restrict__ x, int M, int K, int N,
                                                               const uint8_t* __restrict__ w,
                                                               const uint16_t* __restrict__ s, int groups,
                                                               uint16_t* __restrict__ y) {
    constexpr int KCHUNK = WFmt<WBITS>::KCHUNK;
    constexpr int KSTEPS = KCHUNK / 32;
    extern __shared__ __attribute__((aligned(16))) uint8_t xs_dyn[];
    __shared__ f32x4 red[NW][64];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int t = blockIdx.x;
    const int C = K / KCHUNK;
    const int xrow_b = 2 * K + 16;
    const int rowq = 4 * (lane >> 4);  // first of this lane's 4 output rows in the tile

    // chunks wave + NW * i, i < nw; indices clamp to the wave's last chunk
    // (chunk C - 1 for a wave without chunks, whose loads are then never used)
    const int nw = wave < C ? (C - 1 - wave) / NW + 1 : 0;
    const int clast = wave < C ? wave + (nw - 1) * NW : C - 1;
    const uint8_t* wt = w + (size_t)t * C * CHUNK_BYTES + lane * 16;
    const uint16_t* st = s + (size_t)t * TILE_ROWS + rowq;
    u32x4 wv[DEPTH];
    u32x2 sv[DEPTH];
    auto wload = [&](int i, int slot) {
        const int c = min(wave + NW * i, clast);
        wv[slot] = ldg128_stream(wt + (size_t)c * CHUNK_BYTES);
        if constexpr (WBITS == 4)
            sv[slot] = *reinterpret_cast<const u32x2*>(st + (size_t)(groups > 1 ? c : 0) * N);
    };
#pragma unroll
    for (int p = 0; p < DEPTH; ++p) wload(p, p);

    const int pieces = M * (K / 8);  // 16-byte token pieces
    for (int q = tid; q < pieces; q += NW * 64) {
        const int row = q / (K / 8), pc = q - row * (K / 8);
        *reinterpret_cast<u32x4*>(xs_dyn + row * xrow_b + 16 * pc) = ldg128(x + (size_t)row * K + 8 * pc);
    }
    __syncthreads();

    const uint8_t* xl = xs_dyn + min(lane & 15, M - 1) * xrow_b + 16 * (lane >> 4);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    auto body = [&](int i, auto U) {
        constexpr int u = decltype(U)::value;
        const uint8_t* xc = xl + (size_t)min(wave + NW * i, clast) * (2 * KCHUNK);
        if constexpr (WBITS == 4) {
            f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                const u32x4 a = dequant_w4_f16(wv[u][ks]);
                const u32x4 b = *reinterpret_cast<const u32x4*>(xc + 64 * ks);
                part = mfma16x16x32<false>(a, b, part);
            }
            const uint32_t lo = sv[u][0], hi = sv[u][1];
            acc[0] += part[0] * f16_to_f32((uint16_t)(lo & 0xffffu));
            acc[1] += part[1] * f16_to_f32((uint16_t)(lo >> 16));
            acc[2] += part[2] * f16_to_f32((uint16_t)(hi & 0xffffu));
            acc[3] += part[3] * f16_to_f32((uint16_t)(hi >> 16));
        } else {
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                const u32x4 a = dequant_w8x8<BF16>(wv[u][2 * ks], wv[u][2 * ks + 1]);
                const u32x4 b = *reinterpret_cast<const u32x4*>(xc + 64 * ks);
                acc = mfma16x16x32<BF16>(a, b, acc);
            }
        }
        wload(i + DEPTH, u);
    };
    int i0 = 0;
    for (; i0 + DEPTH <= nw; i0 += DEPTH) static_for<0, DEPTH>([&](auto U) { body(i0 + decltype(U)::value, U); });
    static_for<0, DEPTH - 1>([&](auto U) {
        if (i0 + decltype(U)::value < nw) body(i0 + decltype(U)::value, U);
    });

    red[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int q = 1; q < NW; ++q) acc += red[q][lane];
        const int m = lane & 15;
        if (m < M) {
            const int n0 = t * TILE_ROWS + rowq;
            float o[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                o[r] = acc[r];
                if constexpr (WBITS == 8) o[r] *= act_to_f32<BF16>(s[n0 + r]);
            }
            u32x2 stv;
            stv[0] = (uint32_t)f32_to_act<BF16>(o[0]) | ((uint32_t)f32_to_act<BF16>(o[1]) << 16);
            stv[1] = (uint32_t)f32_to_act<BF16>(o[2]) | ((uint32_t)f32_to_act<BF16>(o[3]) << 16);
            *reinterpret_cast<u32x2*>(y + (size_t)m * N + n0) = stv;
        }
    }
}

size_t dense_decode_lds(int M, int K) { return (size_t)M * (2 * (size_t)K + 16); }

bool dense_decode_supported(int M, int K) { return M >= 1 && M <= 4 && dense_decode_lds(M, K) <= 96 * 1024; }

template <int WBITS, bool BF16>
static void launch_dd(const uint16_t* x, int M, int K, int N, const uint8_t* w, const uint16_t* s, int groups,
                      uint16_t* y, hipStream_t st) {
    constexpr int NW = 4, DEPTH = 4;
    const size_t lds = dense_decode_lds(M, K);
    auto kern = dense_decode_kernel<WBITS, BF16, NW, DEPTH>;
    if (lds + sizeof(f32x4) * 64 * NW > 65536)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)lds);
    hipLaunchKernelGGL(kern, dim3(N / TILE_ROWS), dim3(NW * 64), lds, st, x, M, K, N, w, s, groups, y);
}

void launch_dense_decode(int wbits, bool bf16, const uint16_t* x, int M, int K, int N, const uint8_t* w,
                         const uint16_t* s, int groups, uint16_t* y, hipStream_t st) {
    if (wbits == 4) launch_dd<4, false>(x, M, K, N, w, s, groups, y, st);
    else if (bf16) launch_dd<8, true>(x, M, K, N, w, s, groups, y, st);
    else launch_dd<8, false>(x, M, K, N, w, s, groups, y, st);
}

}  // namespace wq

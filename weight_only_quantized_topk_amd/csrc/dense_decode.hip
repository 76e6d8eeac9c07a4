// dense_decode.hip -- the dense single-expert linear layer at small batches.
//
// y[m, n] = sum_k x[m, k] W[n, k] for 1 or 2 token rows (the GEMV end of the
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

// ----------------------------------------------------------------------------
// 3..128 token rows (R 16-row token tiles per workgroup, grid y over groups
// of 16 R rows): one workgroup per NWV 16-row weight tiles, one tile per
// wave, every wave walking all of K.  The tokens of one K chunk (16 R rows x
// KCHUNK channels) are staged once in LDS and shared by the NWV waves
// (double-buffered, one barrier per chunk): a workgroup covering many weight
// rows stages the token rows few times, where a workgroup per tile would read
// them from L2 once per tile; each chunk's weights are converted once per wave
// for all R token tiles.  Each wave keeps PF chunks of its weights in flight;
// token rows at or beyond M read row M - 1 and their outputs are dropped.
// Same numerics as the kernel above; no reduction across waves, the output is
// rounded once to the activation type.  Yi-34B shape int4 (K = 7168, N =
// 20480), against the grouped large-batch path it replaces above 16 rows:
// M = 32 50.9 -> 34.4 us, M = 64 66.6 -> 47.5 us, M = 128 90.7 -> 79.7 us
// (4 token tiles on 8 waves; 8 token tiles or 4 waves were slower).
constexpr int DS_ROWB = 2 * 128 + 16;  // LDS bytes per token row of one chunk (int4 chunk + pad)
#ifndef DS_NW1
#define DS_NW1 8
#define DS_PF1 6
#endif
#ifndef DS_NW2
#define DS_NW2 8
#define DS_NW4 8
#define DS_PF4 4
#define DS_R4 4
#endif

template <int WBITS, bool BF16, int NWV, int PF, int R>
__global__ __launch_bounds__(NWV * 64) void dense_stream_kernel(const uint16_t* __restrict__ x, int M, int K, int N,
                                                                const uint8_t* __restrict__ w,
                                                                const uint16_t* __restrict__ s, int groups,
                                                                uint16_t* __restrict__ y) {
    constexpr int KCHUNK = WFmt<WBITS>::KCHUNK;
    constexpr int KSTEPS = KCHUNK / 32;
    constexpr int NT = NWV * 64;
    constexpr int ROWS = 16 * R;                  // token rows of the workgroup
    constexpr int PIECES = ROWS * KCHUNK / 8;     // 16-byte token pieces per chunk
    constexpr int XP = (PIECES + NT - 1) / NT;    // per thread
    static_assert(PF % 2 == 0, "chunk parity = slot parity: the token buffers alternate with it");
    __shared__ __attribute__((aligned(16))) uint8_t xs[2][ROWS * DS_ROWB];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ntiles = N / TILE_ROWS;
    const int t_raw = NWV * blockIdx.x + wave;
    const bool tvalid = t_raw < ntiles;
    const int t = tvalid ? t_raw : ntiles - 1;  // surplus waves stream the last tile and store nothing
    const int m0 = blockIdx.y * ROWS;
    const int C = K / KCHUNK;
    const int rowq = 4 * (lane >> 4);

    const uint8_t* wt = w + (size_t)t * C * CHUNK_BYTES + lane * 16;
    const uint16_t* st = s + (size_t)t * TILE_ROWS + rowq;
    u32x4 wv[PF];
    u32x2 sv[PF];
    auto wload = [&](int c, int slot) {
        wv[slot] = ldg128_stream(wt + (size_t)c * CHUNK_BYTES);
        if constexpr (WBITS == 4)
            sv[slot] = *reinterpret_cast<const u32x2*>(st + (size_t)(groups > 1 ? c : 0) * N);
    };
    // token pieces of this thread (threads past PIECES reload the last piece;
    // rows at or beyond M read row M - 1)
    const uint16_t* xsrc[XP];
    int xoff[XP];
#pragma unroll
    for (int i = 0; i < XP; ++i) {
        const int q = min(tid + NT * i, PIECES - 1);
        const int xr = q / (KCHUNK / 8), xp = q % (KCHUNK / 8);
        xsrc[i] = x + (size_t)min(m0 + xr, M - 1) * K + 8 * xp;
        xoff[i] = xr * DS_ROWB + 16 * xp;
    }
    u32x4 xv[2][XP];
    auto xload = [&](int c, int slot) {
#pragma unroll
        for (int i = 0; i < XP; ++i) xv[slot][i] = ldg128(xsrc[i] + (size_t)c * KCHUNK);
    };
    auto xstore = [&](int slot, int buf) {
#pragma unroll
        for (int i = 0; i < XP; ++i) *reinterpret_cast<u32x4*>(&xs[buf][xoff[i]]) = xv[slot][i];
    };

    f32x4 acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int slot, int buf) {
        if constexpr (WBITS == 4) {
            u32x4 a[KSTEPS];
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) a[ks] = dequant_w4_f16(wv[slot][ks]);
            const uint32_t lo = sv[slot][0], hi = sv[slot][1];
            const float s0 = f16_to_f32((uint16_t)(lo & 0xffffu)), s1 = f16_to_f32((uint16_t)(lo >> 16));
            const float s2 = f16_to_f32((uint16_t)(hi & 0xffffu)), s3 = f16_to_f32((uint16_t)(hi >> 16));
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint8_t* xb = &xs[buf][(16 * r + (lane & 15)) * DS_ROWB + 16 * (lane >> 4)];
                f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks)
                    part = mfma16x16x32<false>(a[ks], *reinterpret_cast<const u32x4*>(xb + 64 * ks), part);
                acc[r][0] += part[0] * s0;
                acc[r][1] += part[1] * s1;
                acc[r][2] += part[2] * s2;
                acc[r][3] += part[3] * s3;
            }
        } else {
            u32x4 a[KSTEPS];
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) a[ks] = dequant_w8x8<BF16>(wv[slot][2 * ks], wv[slot][2 * ks + 1]);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint8_t* xb = &xs[buf][(16 * r + (lane & 15)) * DS_ROWB + 16 * (lane >> 4)];
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks)
                    acc[r] = mfma16x16x32<BF16>(a[ks], *reinterpret_cast<const u32x4*>(xb + 64 * ks), acc[r]);
            }
        }
    };
    // chunk c: store its tokens (loaded one chunk earlier), load chunk c + 2's
    // tokens, barrier, multiply, refill the weight slot with chunk c + PF.
    // Every load is unconditional (indices clamp to the last chunk).
    auto body = [&](int c, auto U) {
        constexpr int u = decltype(U)::value;
        xstore(u & 1, u & 1);
        xload(min(c + 2, C - 1), u & 1);
        __syncthreads();
        compute(u, u & 1);
        wload(min(c + PF, C - 1), u);
    };
#pragma unroll
    for (int p = 0; p < PF; ++p) wload(min(p, C - 1), p);
    xload(0, 0);
    xload(min(1, C - 1), 1);
    int c0 = 0;
    for (; c0 + PF <= C; c0 += PF) static_for<0, PF>([&](auto U) { body(c0 + decltype(U)::value, U); });
    static_for<0, PF - 1>([&](auto U) {  // tail of fewer than PF chunks (uniform guard)
        if (c0 + decltype(U)::value < C) body(c0 + decltype(U)::value, U);
    });

    if (tvalid) {
        const int n0 = t * TILE_ROWS + rowq;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int m = m0 + 16 * r + (lane & 15);
            if (m < M) {
                float o[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    o[i] = acc[r][i];
                    if constexpr (WBITS == 8) o[i] *= act_to_f32<BF16>(s[n0 + i]);
                }
                u32x2 stv;
                stv[0] = (uint32_t)f32_to_act<BF16>(o[0]) | ((uint32_t)f32_to_act<BF16>(o[1]) << 16);
                stv[1] = (uint32_t)f32_to_act<BF16>(o[2]) | ((uint32_t)f32_to_act<BF16>(o[3]) << 16);
                *reinterpret_cast<u32x2*>(y + (size_t)m * N + n0) = stv;
            }
        }
    }
}

size_t dense_decode_lds(int M, int K) { return (size_t)M * (2 * (size_t)K + 16); }

// rows staged whole for 1 or 2 rows; from 3 rows the chunk-streaming kernel
// is the faster one (Yi-34B shape int4: M = 1 19.6 / 28.3 us, M = 2 23.6 /
// 28.7 us, M = 4 34.0 / 29.1 us whole-row / chunk-streaming)
static bool dense_rows_in_lds(int M, int K) { return M >= 1 && M <= 2 && dense_decode_lds(M, K) <= 96 * 1024; }

#ifndef DS_MAX_ROWS
#define DS_MAX_ROWS 128
#endif
bool dense_decode_supported(int M, int K) { return dense_rows_in_lds(M, K) || (M >= 1 && M <= DS_MAX_ROWS); }

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

template <int WBITS, bool BF16, int NWV, int PF, int R>
static void launch_ds_r(const uint16_t* x, int M, int K, int N, const uint8_t* w, const uint16_t* s, int groups,
                        uint16_t* y, hipStream_t st) {
    const dim3 grid((N / TILE_ROWS + NWV - 1) / NWV, (M + 16 * R - 1) / (16 * R));
    hipLaunchKernelGGL((dense_stream_kernel<WBITS, BF16, NWV, PF, R>), grid, dim3(NWV * 64), 0, st, x, M, K, N, w, s,
                       groups, y);
}

template <int WBITS, bool BF16>
static void launch_ds(const uint16_t* x, int M, int K, int N, const uint8_t* w, const uint16_t* s, int groups,
                      uint16_t* y, hipStream_t st) {
    if (M <= 16) launch_ds_r<WBITS, BF16, DS_NW1, DS_PF1, 1>(x, M, K, N, w, s, groups, y, st);
    else if (M <= 32) launch_ds_r<WBITS, BF16, DS_NW2, 6, 2>(x, M, K, N, w, s, groups, y, st);
    else launch_ds_r<WBITS, BF16, DS_NW4, DS_PF4, DS_R4>(x, M, K, N, w, s, groups, y, st);
}

void launch_dense_decode(int wbits, bool bf16, const uint16_t* x, int M, int K, int N, const uint8_t* w,
                         const uint16_t* s, int groups, uint16_t* y, hipStream_t st) {
    if (dense_rows_in_lds(M, K)) {
        if (wbits == 4) launch_dd<4, false>(x, M, K, N, w, s, groups, y, st);
        else if (bf16) launch_dd<8, true>(x, M, K, N, w, s, groups, y, st);
        else launch_dd<8, false>(x, M, K, N, w, s, groups, y, st);
    } else {
        if (wbits == 4) launch_ds<4, false>(x, M, K, N, w, s, groups, y, st);
        else if (bf16) launch_ds<8, true>(x, M, K, N, w, s, groups, y, st);
        else launch_ds<8, false>(x, M, K, N, w, s, groups, y, st);
    }
}

}  // namespace wq

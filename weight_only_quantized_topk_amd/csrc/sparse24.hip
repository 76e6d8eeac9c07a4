// sparse24.hip -- 2:4-structured-sparse W4A16 linear layer y = x W^T.
//
// W [N, K] keeps 2 of every 4 input channels ("Add GPTQ Marlin 2:4 sparse
// structured support", vLLM PR 4790, opening description: 2:4 sparsity, 4-bit
// values, group size 128).  On gfx950 the sparse operand of
// v_smfmac_f32_16x16x64_f16 is A, so the weights are A (16 output rows x 64
// dense input channels per instruction, 8 kept values per lane) and the
// activations B.  The packer stores, per 16-row tile and 256 dense channels,
// one 16-byte piece of kept int4 codes per lane (4 instructions' worth, nibble
// order of the dense int4 format) and one 8-byte piece of 2-bit position
// metadata per lane, already in the instruction's index format, so the
// metadata decode is a register move: two instructions share one index dword
// through ABID 0/1.  Group scales are folded in fp32 per 128 dense channels.
//
// One workgroup: 16 output rows x up to 64 tokens, the 4 waves split K and
// meet in LDS.
#include "common.hpp"
#include "launch.hpp"

namespace wq {

constexpr int SP_WAVES = 4;
constexpr int SP_THREADS = 64 * SP_WAVES;
constexpr int SP_KCHUNK = 256;  // dense input channels per packed piece
constexpr int SP_RMAX = 4;      // 16-row token blocks per workgroup

__global__ __launch_bounds__(SP_THREADS) void sparse24_kernel(const uint16_t* __restrict__ x, int M, int K, int N,
                                                              const uint8_t* __restrict__ vals,
                                                              const uint8_t* __restrict__ meta,
                                                              const uint16_t* __restrict__ scales,
                                                              uint16_t* __restrict__ y) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int tile = blockIdx.x;
    const int tok0 = blockIdx.y * 16 * SP_RMAX;
    const int R = min(SP_RMAX, (M - tok0 + 15) / 16);
    const int C = K / SP_KCHUNK;
    const int rowq = 4 * (lane >> 4);

    const uint8_t* vt = vals + (size_t)tile * C * 1024 + lane * 16;
    const uint8_t* mt = meta + (size_t)tile * C * 512 + lane * 8;
    const uint16_t* st = scales + tile * 16 + rowq;

    const uint16_t* xr[SP_RMAX];
    bool xv_ok[SP_RMAX];
#pragma unroll
    for (int r = 0; r < SP_RMAX; ++r) {
        const int m = tok0 + 16 * r + (lane & 15);
        xv_ok[r] = (r < R) && (m < M);
        xr[r] = x + (size_t)(xv_ok[r] ? m : 0) * K + 8 * (lane >> 4);
    }

    f32x4 acc[SP_RMAX];
#pragma unroll
    for (int r = 0; r < SP_RMAX; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int c = wave; c < C; c += SP_WAVES) {
        const u32x4 v = ldg128_stream(vt + (size_t)c * 1024);
        const u32x2 md = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(mt + (size_t)c * 512));
        u32x8 b[SP_RMAX][4];
#pragma unroll
        for (int r = 0; r < SP_RMAX; ++r)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
                if (xv_ok[r]) {
                    lo = ldg128(xr[r] + c * SP_KCHUNK + 64 * s);
                    hi = ldg128(xr[r] + c * SP_KCHUNK + 64 * s + 32);
                }
                b[r][s] = u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
        const u32x2 s01 = *reinterpret_cast<const u32x2*>(st + (size_t)(2 * c) * N);
        const u32x2 s23 = *reinterpret_cast<const u32x2*>(st + (size_t)(2 * c + 1) * N);
#pragma unroll
        for (int grp = 0; grp < 2; ++grp) {
            f32x4 part[SP_RMAX];
#pragma unroll
            for (int r = 0; r < SP_RMAX; ++r) part[r] = f32x4{0.f, 0.f, 0.f, 0.f};
            const u32x4 a0 = dequant_w4_f16(v[2 * grp]);
            const u32x4 a1 = dequant_w4_f16(v[2 * grp + 1]);
            const int idx = (int)md[grp];
#pragma unroll
            for (int r = 0; r < SP_RMAX; ++r) {
                if (r < R) {
                    part[r] = smfmac16x16x64<0>(a0, b[r][2 * grp], idx, part[r]);
                    part[r] = smfmac16x16x64<1>(a1, b[r][2 * grp + 1], idx, part[r]);
                }
            }
            const u32x2 sp = grp ? s23 : s01;
            const float f0 = f16_to_f32((uint16_t)(sp[0] & 0xffffu));
            const float f1 = f16_to_f32((uint16_t)(sp[0] >> 16));
            const float f2 = f16_to_f32((uint16_t)(sp[1] & 0xffffu));
            const float f3 = f16_to_f32((uint16_t)(sp[1] >> 16));
#pragma unroll
            for (int r = 0; r < SP_RMAX; ++r) {
                acc[r][0] += part[r][0] * f0;
                acc[r][1] += part[r][1] * f1;
                acc[r][2] += part[r][2] * f2;
                acc[r][3] += part[r][3] * f3;
            }
        }
    }

    __shared__ f32x4 red[SP_WAVES][SP_RMAX][64];
#pragma unroll
    for (int r = 0; r < SP_RMAX; ++r) red[wave][r][lane] = acc[r];
    __syncthreads();
    if (wave < R) {
        const int r = wave;
        f32x4 o = red[0][r][lane];
#pragma unroll
        for (int w = 1; w < SP_WAVES; ++w) o += red[w][r][lane];
        const int m = tok0 + 16 * r + (lane & 15);
        if (m < M) {
            u32x2 stv;
            stv[0] = (uint32_t)f32_to_f16(o[0]) | ((uint32_t)f32_to_f16(o[1]) << 16);
            stv[1] = (uint32_t)f32_to_f16(o[2]) | ((uint32_t)f32_to_f16(o[3]) << 16);
            *reinterpret_cast<u32x2*>(y + (size_t)m * N + tile * 16 + rowq) = stv;
        }
    }
}

void launch_sparse24(const uint16_t* x, int M, int K, int N, const uint8_t* vals, const uint8_t* meta,
                     const uint16_t* scales, uint16_t* y, hipStream_t s) {
    const dim3 grid(N / 16, (M + 16 * SP_RMAX - 1) / (16 * SP_RMAX));
    hipLaunchKernelGGL(sparse24_kernel, grid, dim3(SP_THREADS), 0, s, x, M, K, N, vals, meta, scales, y);
}

}  // namespace wq

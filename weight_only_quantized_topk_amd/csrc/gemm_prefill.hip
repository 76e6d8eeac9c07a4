// gemm_prefill.hip -- large-batch grouped GEMM of the quantized MoE layer.
//
// Requires block_size % 128 == 0, so every 128-row slice of the sorted token
// order belongs to one expert.  One workgroup computes a 128 (weight rows) x
// 128 (sorted token rows) tile:
//  - per K step the packed weight tile (8 row-tiles x 1 KiB) is loaded with
//    128-bit loads, dequantized once per workgroup (int4: q * group scale,
//    rounded once to fp16; int8: exact) and stored to LDS; the token rows
//    (gathered through sorted_token_ids, or read directly for H and the
//    act-order-permuted activations) go to LDS unchanged;
//  - LDS rows are split in 16-byte chunks stored at chunk ^ (row & 7), so the
//    32 rows read by an MFMA operand fetch hit distinct banks;
//  - 4 waves in a 2 x 2 grid, each 64 x 64 = 2 x 2 v_mfma_f32_32x32x16 tiles
//    with fp32 accumulators; the next K step's global loads are in flight
//    while the current one is multiplied.
// The MFMA A operand is the weight tile (rows = output channels), B the
// tokens, so with the gate/up interleave of the packer a 32-row A tile holds 16
// gate rows and the matching 16 up rows and SiLU(gate)*up is lane-local
// (accumulator registers r and r + 8).
#include "common.hpp"
#include "launch.hpp"

namespace wq {

constexpr int PF_BM = 128;  // sorted token rows per tile
constexpr int PF_BN = 128;  // weight rows per tile
constexpr int PF_THREADS = 256;

template <int WBITS, bool BF16, int STAGE>
__global__ __launch_bounds__(PF_THREADS, 2) void gemm_prefill_kernel(GemmArgs g) {
    constexpr int BK = WFmt<WBITS>::KCHUNK;  // input channels per K step
    constexpr int CPR = BK / 8;              // 16-byte chunks per LDS row
    constexpr int ROWB = BK * 2;             // LDS row bytes
    constexpr int TOK_PIECES = PF_BM * CPR / PF_THREADS;
    __shared__ __attribute__((aligned(16))) uint8_t As[PF_BN * ROWB];
    __shared__ __attribute__((aligned(16))) uint8_t Bs[PF_BM * ROWB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wn = wave & 1, wm = wave >> 1;
    const int ntile = blockIdx.x;
    const int mtile = blockIdx.y;
    const int T = g.M * g.topk;
    const int row0 = mtile * PF_BM;
    if (row0 >= *g.ntpp) return;
    const int e = g.expert_ids[row0 / g.block_size];

    if (g.sorted[row0] >= T) {  // a slice of pad rows only (blocks larger than 128)
        if constexpr (STAGE == STAGE_GATE_UP) {
            const int N = g.n_out / 2;
            for (int k = tid; k < PF_BM * (PF_BN / 2); k += PF_THREADS)
                static_cast<uint16_t*>(g.out)[(size_t)(row0 + k / (PF_BN / 2)) * N + ntile * (PF_BN / 2) +
                                              k % (PF_BN / 2)] = 0;
        }
        return;
    }

    const int C = g.k_in / BK;
    const size_t expert_bytes = (size_t)(g.n_out / TILE_ROWS) * C * CHUNK_BYTES;
    const uint8_t* we = g.w + (size_t)e * expert_bytes;
    const uint16_t* se = g.s + (size_t)e * g.groups * g.n_out;

    // weight pieces of this thread: row-tiles (tid/64) and (tid/64 + 4), lane-equivalent tid%64
    const int wl = tid & 63;
    const int wtile0 = ntile * (PF_BN / TILE_ROWS) + (tid >> 6);
    const uint8_t* wsrc0 = we + (size_t)wtile0 * C * CHUNK_BYTES + wl * 16;
    const uint8_t* wsrc1 = wsrc0 + (size_t)4 * C * CHUNK_BYTES;
    const int wrow0 = (tid >> 6) * TILE_ROWS + (wl & 15);  // tile-local weight row of piece 0
    const int wrow1 = wrow0 + 4 * TILE_ROWS;

    // token pieces: fixed rows, one 16-byte chunk each per K step
    const uint16_t* tsrc[TOK_PIECES];
    bool tval[TOK_PIECES];
#pragma unroll
    for (int i = 0; i < TOK_PIECES; ++i) {
        const int id = tid + PF_THREADS * i;
        const int r = id / CPR, ch = id % CPR;
        const int p = row0 + r;
        const int pair = g.sorted[p];
        tval[i] = pair < T;
        const int src = g.a_direct ? p : (tval[i] ? pair / g.topk : 0);
        tsrc[i] = g.a + (size_t)src * g.k_in + ch * 8;
    }

    u32x4 wv0, wv1;
    u32x4 tv[TOK_PIECES];
    uint32_t sc0 = 0, sc1 = 0;

    auto gload = [&](int c) {
        wv0 = ldg128_stream(wsrc0 + (size_t)c * CHUNK_BYTES);
        wv1 = ldg128_stream(wsrc1 + (size_t)c * CHUNK_BYTES);
        if constexpr (WBITS == 4) {
            const int grp = g.groups > 1 ? c : 0;
            sc0 = se[(size_t)grp * g.n_out + ntile * PF_BN + wrow0];
            sc1 = se[(size_t)grp * g.n_out + ntile * PF_BN + wrow1];
        }
#pragma unroll
        for (int i = 0; i < TOK_PIECES; ++i) tv[i] = tval[i] ? ldg128(tsrc[i] + c * BK) : u32x4{0u, 0u, 0u, 0u};
    };

    auto lds_store = [&]() {
        // weights
        if constexpr (WBITS == 4) {
            const f16x2 s0 = __builtin_bit_cast(f16x2, sc0 | (sc0 << 16));
            const f16x2 s1 = __builtin_bit_cast(f16x2, sc1 | (sc1 << 16));
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int ch = 4 * s + (wl >> 4);
                *reinterpret_cast<u32x4*>(As + wrow0 * ROWB + ((ch ^ (wrow0 & 7)) * 16)) =
                    dequant_w4_f16_scaled(wv0[s], s0);
                *reinterpret_cast<u32x4*>(As + wrow1 * ROWB + ((ch ^ (wrow1 & 7)) * 16)) =
                    dequant_w4_f16_scaled(wv1[s], s1);
            }
        } else {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int ch = 4 * s + (wl >> 4);
                *reinterpret_cast<u32x4*>(As + wrow0 * ROWB + ((ch ^ (wrow0 & 7)) * 16)) =
                    dequant_w8x8<BF16>(wv0[2 * s], wv0[2 * s + 1]);
                *reinterpret_cast<u32x4*>(As + wrow1 * ROWB + ((ch ^ (wrow1 & 7)) * 16)) =
                    dequant_w8x8<BF16>(wv1[2 * s], wv1[2 * s + 1]);
            }
        }
        // tokens
#pragma unroll
        for (int i = 0; i < TOK_PIECES; ++i) {
            const int id = tid + PF_THREADS * i;
            const int r = id / CPR, ch = id % CPR;
            *reinterpret_cast<u32x4*>(Bs + r * ROWB + ((ch ^ (r & 7)) * 16)) = tv[i];
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    gload(0);
    lds_store();
    __syncthreads();
    for (int c = 0; c < C; ++c) {
        if (c + 1 < C) gload(c + 1);
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int ch = 2 * kk + (lane >> 5);
            u32x4 a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int ra = 64 * wn + 32 * i + (lane & 31);
                a[i] = *reinterpret_cast<const u32x4*>(As + ra * ROWB + ((ch ^ (ra & 7)) * 16));
                const int rb = 64 * wm + 32 * i + (lane & 31);
                b[i] = *reinterpret_cast<const u32x4*>(Bs + rb * ROWB + ((ch ^ (rb & 7)) * 16));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16<BF16>(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
        if (c + 1 < C) {
            lds_store();
            __syncthreads();
        }
    }

    // epilogue
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int p = row0 + 64 * wm + 32 * j + (lane & 31);
        const int pair = g.sorted[p];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int wbase = ntile * PF_BN + 64 * wn + 32 * i;  // first packed weight row of the 32-row tile
            if constexpr (STAGE == STAGE_GATE_UP) {
                const int N = g.n_out / 2;
                const int hbase = wbase / 2;
#pragma unroll
                for (int half = 0; half < 2; ++half) {  // regs 4*half .. 4*half+3
                    float h[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int r = 4 * half + q;
                        const int rho = 8 * half + 4 * (lane >> 5) + q;  // gate row within the 16
                        float gt = acc[i][j][r], up = acc[i][j][r + 8];
                        if constexpr (WBITS == 8) {
                            gt *= act_to_f32<BF16>(se[wbase + rho]);
                            up *= act_to_f32<BF16>(se[wbase + 16 + rho]);
                        }
                        h[q] = silu_f32(gt) * up;
                    }
                    u32x2 st;
                    st[0] = (uint32_t)f32_to_act<BF16>(h[0]) | ((uint32_t)f32_to_act<BF16>(h[1]) << 16);
                    st[1] = (uint32_t)f32_to_act<BF16>(h[2]) | ((uint32_t)f32_to_act<BF16>(h[3]) << 16);
                    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(g.out) + (size_t)p * N + hbase + 8 * half +
                                              4 * (lane >> 5)) = st;
                }
            } else {
                if (pair < T) {
                    const float rw = (STAGE == STAGE_DOWN) ? g.topk_w[pair] : 1.0f;
#pragma unroll
                    for (int grp = 0; grp < 4; ++grp) {
                        const int rr = 8 * grp + 4 * (lane >> 5);
                        f32x4 o;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            float v = acc[i][j][4 * grp + q];
                            if constexpr (WBITS == 8) v *= act_to_f32<BF16>(se[wbase + rr + q]);
                            o[q] = v * rw;
                        }
                        *reinterpret_cast<f32x4*>(static_cast<float*>(g.out) + (size_t)pair * g.n_out + wbase + rr) =
                            o;
                    }
                }
            }
        }
    }
}

template <int WBITS, bool BF16>
static void launch_prefill_s(int stage, const GemmArgs& g, hipStream_t s) {
    const dim3 grid(g.n_out / PF_BN, g.cap / PF_BM);
    if (stage == STAGE_GATE_UP)
        hipLaunchKernelGGL((gemm_prefill_kernel<WBITS, BF16, STAGE_GATE_UP>), grid, dim3(PF_THREADS), 0, s, g);
    else if (stage == STAGE_DOWN)
        hipLaunchKernelGGL((gemm_prefill_kernel<WBITS, BF16, STAGE_DOWN>), grid, dim3(PF_THREADS), 0, s, g);
    else
        hipLaunchKernelGGL((gemm_prefill_kernel<WBITS, BF16, STAGE_RAW>), grid, dim3(PF_THREADS), 0, s, g);
}

void launch_gemm_prefill(int wbits, bool bf16, int stage, const GemmArgs& g, hipStream_t s) {
    if (wbits == 4) launch_prefill_s<4, false>(stage, g, s);
    else if (bf16) launch_prefill_s<8, true>(stage, g, s);
    else launch_prefill_s<8, false>(stage, g, s);
}

}  // namespace wq

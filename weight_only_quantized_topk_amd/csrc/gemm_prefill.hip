// gemm_prefill.hip -- large-batch grouped GEMM of the quantized MoE layer.
//
// Works on blocks of 64 or a multiple of 128 sorted token rows, so every
// BM-row slice (BM = 64 or 128) of the sorted order belongs to one expert.
// One workgroup of 4 waves computes BN (128 or 256) weight rows x BM rows:
//  - the packed weight tile (16 rows x 64 input channels per 1 KiB of int8,
//    per 512 B of int4) and the token rows (gathered through
//    sorted_token_ids, or read directly for H and the act-order-permuted
//    activations) are loaded with vector loads two K steps ahead into
//    registers, the weights are dequantized once per workgroup (int4: q *
//    group scale rounded once to fp16; int8: exact) and both tiles stored to
//    LDS;
//  - LDS holds two K steps: while the MFMAs of step k read one buffer, the
//    same waves dequantize and store step k+1 into the other (independent
//    instruction streams that the SIMD co-issues), one barrier per K step;
//  - each wave owns a 64 x 64 (or 64 x 32) slice of the outputs as 32 x 32
//    v_mfma_f32_32x32x16 tiles with fp32 accumulators;
//  - 128-byte LDS rows are split in 16-byte chunks stored at
//    chunk ^ ((row ^ (row >> 3)) & 7), measured free of bank conflicts on
//    gfx950 for the operand reads and both tile writes.
// The MFMA A operand is the weight tile (rows = output channels), B the
// tokens, so with the gate/up interleave of the packer a 32-row A tile holds 16
// gate rows and the matching 16 up rows and SiLU(gate)*up is lane-local
// (accumulator registers r and r + 8).
#include "common.hpp"
#include "launch.hpp"

#include <type_traits>

namespace wq {

constexpr int PF_BK = 64;  // input channels per K step
constexpr int PF_ROWB = PF_BK * 2;
constexpr int PF_THREADS = 256;

// 16-byte chunk swizzle of a 128-byte LDS row: measured on gfx950 to be free of
// bank conflicts for the MFMA operand reads (lane -> row l%32), the weight
// writes (lane -> row l%16) and the token writes (8 lanes per row)
__device__ __forceinline__ int lds_swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int row, int ch) { return row * PF_ROWB + ((ch ^ lds_swz(row)) << 4); }

// BN weight rows x BM token rows per workgroup; WN waves along the weight
// rows, 4 / WN along the tokens
template <int WBITS, bool BF16, int STAGE, int BN, int BM, int WN>
__global__ __launch_bounds__(PF_THREADS, 2) void gemm_prefill_kernel(GemmArgs g) {
    constexpr int WM = 4 / WN;
    constexpr int TI = BN / WN / 32;                              // 32-row weight tiles per wave
    constexpr int TJ = BM / WM / 32;                              // 32-row token tiles per wave
    constexpr int WPIECES = (BN / TILE_ROWS) * 64 / PF_THREADS;  // weight pieces per thread
    constexpr int TPIECES = BM * (PF_BK / 8) / PF_THREADS;       // token pieces per thread
    constexpr int A_BYTES = BN * PF_ROWB, B_BYTES = BM * PF_ROWB;
    static_assert(TI >= 1 && TJ >= 1 && WPIECES >= 1 && TPIECES >= 1, "tile shape");
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * (A_BYTES + B_BYTES)];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int ntile = blockIdx.x;
    const int mtile = blockIdx.y;
    const int T = g.M * g.topk;
    const int row0 = mtile * BM;
    if (row0 >= *g.ntpp) return;
    const int e = g.expert_ids[row0 / g.block_size];

    if (g.sorted[row0] >= T) {  // a slice of pad rows only (blocks larger than 128)
        if constexpr (STAGE == STAGE_GATE_UP) {
            const int N = g.n_out / 2;
            for (int k = tid; k < BM * (BN / 2); k += PF_THREADS)
                static_cast<uint16_t*>(g.out)[(size_t)(row0 + k / (BN / 2)) * N + ntile * (BN / 2) + k % (BN / 2)] = 0;
        }
        return;
    }

    constexpr int KCHUNK = WFmt<WBITS>::KCHUNK;
    const int C = g.k_in / KCHUNK;  // packed chunks per 16-row tile
    const int STEPS = g.k_in / PF_BK;
    const size_t expert_bytes = (size_t)(g.n_out / TILE_ROWS) * C * CHUNK_BYTES;
    const uint16_t* se = g.s + (size_t)e * g.groups * g.n_out;

    // ----------------------------------------------------------- loaders
    const uint8_t* we = g.w + (size_t)e * expert_bytes;
    const uint8_t* wsrc[WPIECES];
    int wrow[WPIECES];
#pragma unroll
    for (int i = 0; i < WPIECES; ++i) {
        const int piece = tid + PF_THREADS * i;
        const int rt = piece >> 6, l = piece & 63;
        wsrc[i] = we + (size_t)(ntile * (BN / TILE_ROWS) + rt) * C * CHUNK_BYTES + l * 16;
        wrow[i] = rt * TILE_ROWS + (l & 15);
    }
    const int wlg = lane >> 4;  // lane group of every weight piece of this thread
    // token pieces: pad rows read a valid row (their outputs are discarded, H pad rows written as 0)
    const uint16_t* tsrc[TPIECES];
#pragma unroll
    for (int i = 0; i < TPIECES; ++i) {
        const int id = tid + PF_THREADS * i;
        const int r = id >> 3, ch = id & 7;
        const int p = row0 + r;
        const int pair = g.sorted[p];
        const int src = g.a_direct ? p : (pair < T ? pair / g.topk : 0);
        tsrc[i] = g.a + (size_t)src * g.k_in + ch * 8;
    }

    // two register sets: data of even / odd K steps
    u32x4 wv[2][WPIECES];
    u32x2 wv4[2][WPIECES];
    uint32_t sc[2][WPIECES];
    u32x4 tv[2][TPIECES];

    auto gload = [&](int step, auto SET) {
        constexpr int set = decltype(SET)::value;
        if constexpr (WBITS == 8) {
#pragma unroll
            for (int i = 0; i < WPIECES; ++i) wv[set][i] = ldg128_stream(wsrc[i] + (size_t)step * CHUNK_BYTES);
        } else {
            const int c = step >> 1, half = step & 1;  // a 128-channel chunk spans two K steps
#pragma unroll
            for (int i = 0; i < WPIECES; ++i)
                wv4[set][i] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x2*>(wsrc[i] + (size_t)c * CHUNK_BYTES + 8 * half));
            const int grp = g.groups > 1 ? c : 0;
#pragma unroll
            for (int i = 0; i < WPIECES; ++i) sc[set][i] = se[(size_t)grp * g.n_out + ntile * BN + wrow[i]];
        }
#pragma unroll
        for (int i = 0; i < TPIECES; ++i) tv[set][i] = ldg128(tsrc[i] + step * PF_BK);
    };
    // store unit u of one K step: weight units (piece, half) first, then token pieces
    constexpr int WUNITS = 2 * WPIECES;
    constexpr int UNITS = WUNITS + TPIECES;
    auto store_unit = [&](auto SET, int u) {
        constexpr int set = decltype(SET)::value;  // register set, also the LDS buffer it goes to
        uint8_t* As = lds + set * (A_BYTES + B_BYTES);
        uint8_t* Bs = As + A_BYTES;
        if (u < WUNITS) {
            const int i = u >> 1, s = u & 1;
            u32x4 v;
            if constexpr (WBITS == 8) {
                v = dequant_w8x8<BF16>(wv[set][i][2 * s], wv[set][i][2 * s + 1]);
            } else {
                const uint32_t sv = sc[set][i];
                v = dequant_w4_f16_scaled(wv4[set][i][s], __builtin_bit_cast(f16x2, sv | (sv << 16)));
            }
            *reinterpret_cast<u32x4*>(As + lds_off(wrow[i], 4 * s + wlg)) = v;
        } else {
            const int i = u - WUNITS;
            const int id = tid + PF_THREADS * i;
            *reinterpret_cast<u32x4*>(Bs + lds_off(id >> 3, id & 7)) = tv[set][i];
        }
    };

    // ---------------------------------------------------------- multipliers
    const int wave = tid >> 6;
    const int wn = wave % WN, wm = wave / WN;  // this wave's weight-row and token slice
    f32x16 acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    int aoff[TI], boff[TJ];  // LDS row byte offsets and swizzles of this lane's operand rows
    int aswz[TI], bswz[TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i) {
        const int r = (BN / WN) * wn + 32 * i + (lane & 31);
        aoff[i] = r * PF_ROWB;
        aswz[i] = lds_swz(r);
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
        const int r = (BM / WM) * wm + 32 * j + (lane & 31);
        boff[j] = A_BYTES + r * PF_ROWB;
        bswz[j] = lds_swz(r);
    }
    const int khalf = lane >> 5;

    // one K step: MFMAs from buffer BUF; with NEXT, dequantize and store the
    // following step (register set BUF ^ 1) into the other buffer in between
    auto step_body = [&](auto BUF, auto NEXT) {
        constexpr int buf = decltype(BUF)::value;
        constexpr bool next = decltype(NEXT)::value;
        const uint8_t* base = lds + buf * (A_BYTES + B_BYTES);
        u32x4 a[2][TI], b[2][TJ];
        auto read_ops = [&](int kk, int x) {
            const int ch = 2 * kk + khalf;
#pragma unroll
            for (int i = 0; i < TI; ++i)
                a[x][i] = *reinterpret_cast<const u32x4*>(base + aoff[i] + ((ch ^ aswz[i]) << 4));
#pragma unroll
            for (int j = 0; j < TJ; ++j)
                b[x][j] = *reinterpret_cast<const u32x4*>(base + boff[j] + ((ch ^ bswz[j]) << 4));
        };
        read_ops(0, 0);
#pragma unroll
        for (int kk = 0; kk < PF_BK / 16; ++kk) {
            if (kk + 1 < PF_BK / 16) read_ops(kk + 1, (kk + 1) & 1);
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int j = 0; j < TJ; ++j)
                    acc[i][j] = mfma32x32x16<BF16>(a[kk & 1][i], b[kk & 1][j], acc[i][j]);
            if constexpr (next) {
#pragma unroll
                for (int u = kk * UNITS / (PF_BK / 16); u < (kk + 1) * UNITS / (PF_BK / 16); ++u)
                    store_unit(std::integral_constant<int, buf ^ 1>{}, u);
            }
        }
    };
    const std::integral_constant<int, 0> B0{};
    const std::integral_constant<int, 1> B1{};
    const std::true_type MORE{};
    const std::false_type LAST{};

    // K steps two at a time so every buffer and register-set index is static
    gload(0, B0);
    if (STEPS > 1) gload(1, B1);
#pragma unroll
    for (int u = 0; u < UNITS; ++u) store_unit(B0, u);
    if (STEPS > 2) gload(2, B0);
    __syncthreads();
    int step = 0;
    for (; step + 2 < STEPS; step += 2) {
        step_body(B0, MORE);
        gload(min(step + 3, STEPS - 1), B1);  // the last step is re-read near the end
        __syncthreads();
        step_body(B1, MORE);
        gload(min(step + 4, STEPS - 1), B0);
        __syncthreads();
    }
    if (step + 1 < STEPS) {
        step_body(B0, MORE);
        __syncthreads();
        step_body(B1, LAST);
    } else {
        step_body(B0, LAST);
    }

    // epilogue
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
        const int p = row0 + (BM / WM) * wm + 32 * j + (lane & 31);
        const int pair = g.sorted[p];
#pragma unroll
        for (int i = 0; i < TI; ++i) {
            const int wbase = ntile * BN + (BN / WN) * wn + 32 * i;  // first packed row of the 32-row tile
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
                        h[q] = (pair < T) ? silu_f32(gt) * up : 0.0f;
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

template <int WBITS, bool BF16, int STAGE, int BN, int BM, int WN>
static void launch_prefill_cfg(const GemmArgs& g, hipStream_t s) {
    const dim3 grid(g.n_out / BN, g.cap / BM);
    hipLaunchKernelGGL((gemm_prefill_kernel<WBITS, BF16, STAGE, BN, BM, WN>), grid, dim3(PF_THREADS), 0, s, g);
}

// 128-row token tiles (blocks of 128 or more): 128 x 128 tiles, 2 x 2 waves;
// 64-row token tiles (blocks of 64, less padding for thin experts): 256 weight
// rows over 4 waves when n_out allows, else 128 x 64 tiles
template <int WBITS, bool BF16, int STAGE>
static void launch_prefill_st(const GemmArgs& g, hipStream_t s) {
    if (g.block_size % 128 == 0) launch_prefill_cfg<WBITS, BF16, STAGE, 128, 128, 2>(g, s);
    else if (g.n_out % 256 == 0) launch_prefill_cfg<WBITS, BF16, STAGE, 256, 64, 4>(g, s);
    else launch_prefill_cfg<WBITS, BF16, STAGE, 128, 64, 2>(g, s);
}

template <int WBITS, bool BF16>
static void launch_prefill_s(int stage, const GemmArgs& g, hipStream_t s) {
    if (stage == STAGE_GATE_UP) launch_prefill_st<WBITS, BF16, STAGE_GATE_UP>(g, s);
    else if (stage == STAGE_DOWN) launch_prefill_st<WBITS, BF16, STAGE_DOWN>(g, s);
    else launch_prefill_st<WBITS, BF16, STAGE_RAW>(g, s);
}

bool prefill_supported(int n_out, int k_in, int block_size) {
    return (block_size == 64 || block_size % 128 == 0) && n_out % 128 == 0 && k_in % PF_BK == 0;
}

void launch_gemm_prefill(int wbits, bool bf16, int stage, const GemmArgs& g, hipStream_t s) {
    if (wbits == 4) launch_prefill_s<4, false>(stage, g, s);
    else if (bf16) launch_prefill_s<8, true>(stage, g, s);
    else launch_prefill_s<8, false>(stage, g, s);
}

}  // namespace wq

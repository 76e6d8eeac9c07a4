// gemm_prefill.hip -- large-batch grouped GEMM of the quantized MoE layer.
//
// Works on blocks of 64 or a multiple of 128 sorted token rows, so every
// BM-row slice (BM = 64 or 128) of the sorted order belongs to one expert.
// One workgroup computes BN weight rows x BM token rows of one expert:
//  - per K step of 64 input channels the packed weight tile (16 rows x 64
//    channels per 1 KiB of int8, per 512 B of int4) and the token rows
//    (gathered through sorted_token_ids, or read directly for H and the
//    act-order-permuted activations) are loaded with vector loads, the weights
//    dequantized once per workgroup (int4: q * group scale rounded once to
//    fp16; int8: exact) and both tiles stored to one LDS buffer;
//  - the next K step's global loads are issued right after the LDS stores, so
//    they are in flight while the MFMAs of the current step run; several
//    workgroups (or the 8 waves of a large one) per CU cover each other's
//    store phases;
//  - each wave owns a 64 x 64 (or 64 x 32) slice of the outputs as 32 x 32
//    v_mfma_f32_32x32x16 tiles with fp32 accumulators;
//  - 128-byte LDS rows are split in 16-byte chunks stored at
//    chunk ^ ((row ^ (row >> 3)) & 7), measured free of bank conflicts on
//    gfx950 for the operand reads and both tile writes.
// The MFMA A operand is the weight tile (rows = output channels), B the
// tokens, so with the gate/up interleave of the packer a 32-row A tile holds 16
// gate rows and the matching 16 up rows and SiLU(gate)*up is lane-local
// (accumulator registers r and r + 8).
//
// DOWN may split K over gridDim.z slices when its output grid is too small to
// fill the chip: slice z writes its partial sums to its own fp32 slab of Y and
// the combine kernel adds the slabs in ascending order (deterministic).
#include "common.hpp"
#include "launch.hpp"

#include <algorithm>

namespace wq {

constexpr int PF_BK = 64;  // input channels per K step
constexpr int PF_ROWB = PF_BK * 2;

// 16-byte chunk swizzle of a 128-byte LDS row: measured on gfx950 to be free of
// bank conflicts for the MFMA operand reads (lane -> row l%32), the weight
// writes (lane -> row l%16) and the token writes (8 lanes per row)
__device__ __forceinline__ int lds_swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int row, int ch) { return row * PF_ROWB + ((ch ^ lds_swz(row)) << 4); }

// BN weight rows x BM token rows per workgroup of NW waves; WN waves along the
// weight rows, NW / WN along the tokens; OCC workgroups per CU.  SKIP: a wave
// skips the MFMAs of its 32-row token tiles that hold pad rows only
template <int WBITS, bool BF16, int STAGE, int BN, int BM, int WN, int NW, int OCC, bool SKIP>
__global__ __launch_bounds__(NW * 64, OCC) void gemm_prefill_kernel(GemmArgs g) {
    constexpr int NT = NW * 64;
    constexpr int WM = NW / WN;
    constexpr int TI = BN / WN / 32;                      // 32-row weight tiles per wave
    constexpr int TJ = BM / WM / 32;                      // 32-row token tiles per wave
    constexpr int WPIECES = (BN / TILE_ROWS) * 64 / NT;  // weight pieces (16 rows x 64 ch over 64 lanes) per thread
    constexpr int TPIECES = BM * (PF_BK / 8) / NT;       // 16-byte token pieces per thread
    constexpr int A_BYTES = BN * PF_ROWB, B_BYTES = BM * PF_ROWB;
    static_assert(TI >= 1 && TJ >= 1 && WPIECES >= 1 && TPIECES >= 1, "tile shape");
    __shared__ __attribute__((aligned(16))) uint8_t lds[A_BYTES + B_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int ntile = blockIdx.x;
    const int mtile = blockIdx.y;
    const int T = g.M * g.topk;
    const int row0 = mtile * BM;
    if (row0 >= *g.ntpp) return;
    const int e = g.expert_ids[row0 / g.block_size];

    if (g.sorted[row0] >= T) {  // a slice of pad rows only (blocks larger than BM)
        if constexpr (STAGE == STAGE_GATE_UP) {
            const int N = g.n_out / 2;
            for (int k = tid; k < BM * (BN / 2); k += NT)
                static_cast<uint16_t*>(g.out)[(size_t)(row0 + k / (BN / 2)) * N + ntile * (BN / 2) + k % (BN / 2)] = 0;
        }
        return;
    }

    constexpr int KCHUNK = WFmt<WBITS>::KCHUNK;
    const int C = g.k_in / KCHUNK;  // packed chunks per 16-row tile
    // K slice of this workgroup (only DOWN is ever split)
    const int steps_per = g.k_in / PF_BK / (int)gridDim.z;
    const int step0 = (int)blockIdx.z * steps_per;
    const int step_end = step0 + steps_per;
    const size_t expert_bytes = (size_t)(g.n_out / TILE_ROWS) * C * CHUNK_BYTES;
    const uint16_t* se = g.s + (size_t)e * g.groups * g.n_out;

    // ----------------------------------------------------------- loaders
    const uint8_t* we = g.w + (size_t)e * expert_bytes;
    const uint8_t* wsrc[WPIECES];
    int wrow[WPIECES];
#pragma unroll
    for (int i = 0; i < WPIECES; ++i) {
        const int piece = tid + NT * i;
        const int rt = piece >> 6, l = piece & 63;
        wsrc[i] = we + (size_t)(ntile * (BN / TILE_ROWS) + rt) * C * CHUNK_BYTES + l * 16;
        wrow[i] = rt * TILE_ROWS + (l & 15);
    }
    const int wlg = lane >> 4;  // lane group of every weight piece of this thread
    // token pieces: pad rows read a valid row (their outputs are discarded, H pad rows written as 0)
    const uint16_t* tsrc[TPIECES];
#pragma unroll
    for (int i = 0; i < TPIECES; ++i) {
        const int id = tid + NT * i;
        const int p = row0 + (id >> 3);
        const int pair = g.sorted[p];
        const int src = g.a_direct ? p : (pair < T ? pair / g.topk : 0);
        tsrc[i] = g.a + (size_t)src * g.k_in + (id & 7) * 8;
    }

    u32x4 wv[WPIECES];
    u32x2 wv4[WPIECES];
    uint32_t sc[WPIECES];
    u32x4 tv[TPIECES];
    auto gload = [&](int step) {
        if constexpr (WBITS == 8) {
#pragma unroll
            for (int i = 0; i < WPIECES; ++i) wv[i] = ldg128_stream(wsrc[i] + (size_t)step * CHUNK_BYTES);
        } else {
            const int c = step >> 1, half = step & 1;  // a 128-channel chunk spans two K steps
#pragma unroll
            for (int i = 0; i < WPIECES; ++i)
                wv4[i] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x2*>(wsrc[i] + (size_t)c * CHUNK_BYTES + 8 * half));
            const int grp = g.groups > 1 ? c : 0;
#pragma unroll
            for (int i = 0; i < WPIECES; ++i) sc[i] = se[(size_t)grp * g.n_out + ntile * BN + wrow[i]];
        }
#pragma unroll
        for (int i = 0; i < TPIECES; ++i) tv[i] = ldg128(tsrc[i] + step * PF_BK);
    };
    auto lds_store = [&]() {
        uint8_t* As = lds;
        uint8_t* Bs = lds + A_BYTES;
#pragma unroll
        for (int i = 0; i < WPIECES; ++i)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                u32x4 v;
                if constexpr (WBITS == 8) {
                    v = dequant_w8x8<BF16>(wv[i][2 * s], wv[i][2 * s + 1]);
                } else {
                    const uint32_t sv = sc[i];
                    v = dequant_w4_f16_scaled(wv4[i][s], __builtin_bit_cast(f16x2, sv | (sv << 16)));
                }
                *reinterpret_cast<u32x4*>(As + lds_off(wrow[i], 4 * s + wlg)) = v;
            }
#pragma unroll
        for (int i = 0; i < TPIECES; ++i) {
            const int id = tid + NT * i;
            *reinterpret_cast<u32x4*>(Bs + lds_off(id >> 3, id & 7)) = tv[i];
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
    int aoff[TI], boff[TJ], aswz[TI], bswz[TJ];  // LDS row offsets and swizzles of this lane's operand rows
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
    // 32-row token tiles of this wave that hold a valid row; the valid rows of
    // a tile are a prefix (the alignment pads each expert's rows at the end)
    int jact = TJ;
    if constexpr (SKIP) {
        jact = 0;
#pragma unroll
        for (int j = 0; j < TJ; ++j)
            jact += __builtin_amdgcn_readfirstlane(g.sorted[row0 + (BM / WM) * wm + 32 * j]) < T ? 1 : 0;
    }
    auto compute = [&]() {
#pragma unroll
        for (int kk = 0; kk < PF_BK / 16; ++kk) {
            const int ch = 2 * kk + khalf;
            u32x4 a[TI], b[TJ];
#pragma unroll
            for (int i = 0; i < TI; ++i) a[i] = *reinterpret_cast<const u32x4*>(lds + aoff[i] + ((ch ^ aswz[i]) << 4));
#pragma unroll
            for (int j = 0; j < TJ; ++j)
                if (j < jact) b[j] = *reinterpret_cast<const u32x4*>(lds + boff[j] + ((ch ^ bswz[j]) << 4));
#pragma unroll
            for (int j = 0; j < TJ; ++j)
                if (j < jact) {
#pragma unroll
                    for (int i = 0; i < TI; ++i) acc[i][j] = mfma32x32x16<BF16>(a[i], b[j], acc[i][j]);
                }
        }
    };

    gload(step0);
    for (int step = step0; step < step_end; ++step) {
        lds_store();
        __syncthreads();
        gload(min(step + 1, step_end - 1));  // the last step is loaded twice, keeping the loop branch-free
        compute();
        __syncthreads();
    }

    // epilogue
    float* yslab = nullptr;
    if constexpr (STAGE != STAGE_GATE_UP)
        yslab = static_cast<float*>(g.out) + (size_t)blockIdx.z * ((size_t)T * g.n_out);
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
                        *reinterpret_cast<f32x4*>(yslab + (size_t)pair * g.n_out + wbase + rr) = o;
                    }
                }
            }
        }
    }
}

// ------------------------------------------------------------------ plans
// Tile shapes, chosen by timing on MI355X with random data:
//   WIDE8  256 x 128, 8 waves of 64 x 64, one workgroup per CU: the fastest
//          int8 GATE_UP shape for large grids with little padding;
//   WIDE4  256 x 128, 4 waves of 128 x 64 with pad-tile skipping, two
//          workgroups per CU: int4, and int8 with much padding;
//   SQ     128 x 128, 4 waves of 64 x 64 with pad-tile skipping, three
//          workgroups per CU: small grids (with K split for DOWN);
//   THIN   128 x 64, 4 waves of 64 x 32: blocks of 64 token rows.
enum PrefillShape { PF_WIDE8, PF_WIDE4, PF_SQ, PF_THIN };

// expected count of 128-row token tiles: T rows plus, per touched expert, a
// half-filled last tile (at most E experts are touched)
static long est_mtiles(int T, int E) { return ((long)T + (long)std::min(T, E) * 64 + 127) / 128; }

// rounds of SQ workgroups (3 per CU) needed for tiles, in units of one full-K workgroup
static double sq_rounds(long tiles, int ks) {
    const long slots = 3L * 256;
    return (double)((tiles * ks + slots - 1) / slots) / ks;
}

// K slices of DOWN.  A grid of 256-row tiles with fewer than 1024 workgroups
// (four rounds of one per CU) takes the smallest split, 2 or 4, that reaches
// 1024, run with a 256-row shape; otherwise the 128 x 128 shape splits when
// that cuts its rounds of three workgroups per CU by 15 %.  Measured on the
// Mixtral shapes: 409 -> 356 us (int8, M = 1024), 266 -> 216 us (M = 512).
int prefill_down_split(int T, int E, int n_out, int k_in) {
    if (n_out % 128 != 0 || k_in % PF_BK != 0) return 1;
    const int steps = k_in / PF_BK;
    if (n_out % 256 == 0) {
        const long tiles256 = (long)(n_out / 256) * est_mtiles(T, E);
        if (tiles256 >= 1024) return 1;
        for (int ks = 2; ks <= 4; ks *= 2)
            if (steps % ks == 0 && steps / ks >= 16 && tiles256 * ks >= 1024) return ks;
    }
    const long tiles = (long)(n_out / 128) * est_mtiles(T, E);
    int best = 1;
    double best_t = sq_rounds(tiles, 1);
    for (int ks = 2; ks <= 4; ks *= 2) {
        if (steps % ks != 0 || steps / ks < 16) break;
        const double t = sq_rounds(tiles, ks);
        if (t < 0.85 * best_t) best = ks, best_t = t;
    }
    return best;
}

static PrefillShape prefill_shape(int wbits, int stage, const GemmArgs& g, int ksplit) {
    if (g.block_size == 64) return PF_THIN;
    if (g.n_out % 256 != 0) return PF_SQ;
    const int T = g.M * g.topk;
    const long tiles256 = (long)(g.n_out / 256) * est_mtiles(T, g.E);
    if (ksplit > 1) {  // a split DOWN: 256-row shape when the split grid fills 4 rounds
        if (tiles256 * ksplit >= 1024) return wbits == 8 ? PF_WIDE8 : PF_WIDE4;
        return PF_SQ;
    }
    const double pad = (double)std::min(T, g.E) * 64 / (T + (double)std::min(T, g.E) * 64);  // expected pad share
    if (wbits == 8 && stage != STAGE_DOWN && tiles256 >= 1024 && pad <= 0.25) return PF_WIDE8;
    return tiles256 >= 512 ? PF_WIDE4 : PF_SQ;
}

template <int WBITS, bool BF16, int STAGE, int BN, int BM, int WN, int NW, int OCC, bool SKIP>
static void launch_prefill_cfg(const GemmArgs& g, int ksplit, hipStream_t s) {
    const dim3 grid(g.n_out / BN, g.cap / BM, ksplit);
    hipLaunchKernelGGL((gemm_prefill_kernel<WBITS, BF16, STAGE, BN, BM, WN, NW, OCC, SKIP>), grid, dim3(NW * 64), 0, s,
                       g);
}

template <int WBITS, bool BF16, int STAGE>
static void launch_prefill_st(const GemmArgs& g, int ksplit, hipStream_t s) {
    switch (prefill_shape(WBITS, STAGE, g, ksplit)) {
        case PF_WIDE8: launch_prefill_cfg<WBITS, BF16, STAGE, 256, 128, 4, 8, 1, false>(g, ksplit, s); break;
        case PF_WIDE4: launch_prefill_cfg<WBITS, BF16, STAGE, 256, 128, 2, 4, 2, true>(g, ksplit, s); break;
        case PF_SQ: launch_prefill_cfg<WBITS, BF16, STAGE, 128, 128, 2, 4, 3, true>(g, ksplit, s); break;
        default: launch_prefill_cfg<WBITS, BF16, STAGE, 128, 64, 2, 4, 3, true>(g, ksplit, s); break;
    }
}

template <int WBITS, bool BF16>
static void launch_prefill_s(int stage, const GemmArgs& g, int ksplit, hipStream_t s) {
    if (stage == STAGE_GATE_UP) launch_prefill_st<WBITS, BF16, STAGE_GATE_UP>(g, 1, s);
    else if (stage == STAGE_DOWN) launch_prefill_st<WBITS, BF16, STAGE_DOWN>(g, ksplit, s);
    else launch_prefill_st<WBITS, BF16, STAGE_RAW>(g, 1, s);
}

bool prefill_supported(int n_out, int k_in, int block_size) {
    return (block_size == 64 || block_size % 128 == 0) && n_out % 128 == 0 && k_in % PF_BK == 0;
}

int launch_gemm_prefill(int wbits, bool bf16, int stage, const GemmArgs& g, hipStream_t s) {
    const int ksplit =
        (stage == STAGE_DOWN && g.block_size % 128 == 0) ? prefill_down_split(g.M * g.topk, g.E, g.n_out, g.k_in) : 1;
    if (wbits == 4) launch_prefill_s<4, false>(stage, g, ksplit, s);
    else if (bf16) launch_prefill_s<8, true>(stage, g, ksplit, s);
    else launch_prefill_s<8, false>(stage, g, ksplit, s);
    return ksplit;
}

}  // namespace wq

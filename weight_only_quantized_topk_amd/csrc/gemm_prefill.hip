// gemm_prefill.hip -- large-batch grouped GEMM of the quantized MoE layer.
//
// Works on blocks of 64 or a multiple of 128 sorted token rows, so every
// BM-row slice (BM = 64 or 128) of the sorted order belongs to one expert.
// One workgroup of NW waves computes BN = NW * RT * 16 weight rows x BM token
// rows of one expert; wave w owns the RT 16-row weight tiles
// [w * RT, (w + 1) * RT) of the workgroup and all BM token rows.
//  - Weights never pass through LDS.  The packed 16-row x 64-channel (int8) or
//    16-row x 128-channel (int4) chunk gives lane l the 8 channels
//    [8 (l/16), +8) and [32 + 8 (l/16), +8) of row l % 16 for every 64-channel
//    K step, which is exactly the A operand layout of two
//    v_mfma_f32_16x16x32 instructions; each wave loads its own tiles with
//    coalesced 128-bit (int8) or 64-bit (int4) loads and dequantizes them in
//    registers (int8 exact; int4: q * group scale rounded once to fp16).  The
//    weights go through the caches: an expert's weight tile is re-read by
//    every token tile of the expert (about 2 at M = 1024, 8 at M = 4096).
//  - Software pipeline of a K step: the MFMAs of step s run with step s + 1's
//    weights converted between them, each tile's raw registers are refilled
//    with step s + 2 as soon as they are converted, and the B operands of
//    token tile j + 1 are read from LDS before tile j is multiplied.
//  - The BM token rows of a K step (gathered through sorted_token_ids, or read
//    directly for H and the act-order-permuted activations) are staged in one
//    of two LDS buffers: step s + 1 is stored while step s is multiplied, so a
//    K step costs one barrier.  Rows are 128 bytes split in 16-byte pieces;
//    see lds_swz for the bank-conflict-free placement.
//  - Accumulators are fp32 (v_mfma_f32_16x16x32_{bf16,f16}).  Lane l holds
//    output rows 4 (l/16) + r of a weight tile for token row l % 16.  With the
//    gate/up interleave of the packer, weight tile 2q holds 16 gate rows and
//    tile 2q + 1 the matching up rows, so SiLU(gate) * up is lane-local.
//  - The valid rows of a BM slice are a prefix (the alignment pads each
//    expert at the end): the MFMAs of 16-row token tiles past them are skipped
//    (one uniform branch per tile), and when they fit in the slice's first
//    half the LDS reads of the second half too.
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

// buffer resource over 4 GiB from base (raw addressing: offsets are bytes)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
}

// 16-byte piece ch of token row `row` sits at piece ch ^ ((row >> 1) & 7) of
// the row: the 16 lanes of one 128-bit LDS access (16 consecutive rows, one
// piece, for the B operand reads; 2 rows, 8 pieces, for the stores) then hit
// 16 distinct 16-byte bank groups, and the swizzle of row 16 j + r does not
// depend on j, so a wave's reads of its 16-row token tiles differ by
// immediate offsets only.
__device__ __forceinline__ int lds_swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int lds_off(int row, int ch) { return row * PF_ROWB + ((ch ^ lds_swz(row)) << 4); }

template <int WBITS, bool BF16, int STAGE, int NW, int RT, int BM, int OCC>
__global__ __launch_bounds__(NW * 64, OCC) void gemm_prefill_kernel(GemmArgs g) {
    constexpr int NT = NW * 64;
    constexpr int BN = NW * RT * 16;
    constexpr int TJ = BM / 16;               // 16-row token tiles
    constexpr int TPIECES = BM * 8 / NT;      // 16-byte token pieces per thread and K step
    constexpr int BUF = BM * PF_ROWB;
    static_assert(TPIECES >= 1 && TJ >= 4 && (STAGE != STAGE_GATE_UP || RT % 2 == 0), "tile shape");
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * BUF];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ntile = blockIdx.x, mtile = blockIdx.y;
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
    const int nsteps = g.k_in / PF_BK;
    const int step0 = (int)((long)blockIdx.z * nsteps / gridDim.z);
    const int step_end = (int)((long)(blockIdx.z + 1) * nsteps / gridDim.z);
    const size_t expert_bytes = (size_t)(g.n_out / TILE_ROWS) * C * CHUNK_BYTES;
    const uint16_t* se = g.s + (size_t)e * g.groups * g.n_out;

    // ----------------------------------------------------------- loaders
    // Buffer loads: the wave-uniform part of a weight address (expert, weight
    // tile, K step) is the resource base or the scalar offset, and a token
    // piece's address a 32-bit offset from the activations' base, which frees
    // the vector registers 64-bit addresses would hold (int4 large-batch
    // Mixtral gate/up 1.83 -> 1.77 ms at M = 4096).
    const int rt0 = ntile * (BN / TILE_ROWS) + __builtin_amdgcn_readfirstlane(wave) * RT;  // first tile of the wave
    const int tile_stride = C * CHUNK_BYTES;
    const __amdgpu_buffer_rsrc_t wres = make_rsrc(g.w + (size_t)e * expert_bytes + (size_t)rt0 * tile_stride);
    const int wlane = lane * 16;
    const uint16_t* ssrc = se + rt0 * TILE_ROWS + (lane & 15);  // int4: scale of this lane's row
    // raw weights of one K step (loaded one step before they are dequantized)
    u32x4 w8[RT];
    u32x2 w4[RT];
    uint32_t sc[RT];
    // raw weights (and int4 group scale) of weight tile t for one K step
    auto wload_t = [&](int step, int t) {
        if constexpr (WBITS == 8) {
            w8[t] = __builtin_amdgcn_raw_buffer_load_b128(wres, wlane, t * tile_stride + step * CHUNK_BYTES, 0);
        } else {
            const int c = step >> 1, half = step & 1;  // a 128-channel chunk spans two K steps
            // cached: the token tiles of an expert re-read its weight tiles
            w4[t] = __builtin_amdgcn_raw_buffer_load_b64(wres, wlane, t * tile_stride + c * CHUNK_BYTES + 8 * half, 0);
            const int grp = g.groups > 1 ? c : 0;
            sc[t] = ssrc[(size_t)grp * g.n_out + t * TILE_ROWS];
        }
    };
    auto wload = [&](int step) {
#pragma unroll
        for (int t = 0; t < RT; ++t) wload_t(step, t);
    };
    // token pieces: pad rows read a valid row (their outputs are discarded, H pad rows written as 0)
    // (byte offsets fit 32 bits: the host checks rows x k_in x 2 < 2^32)
    const __amdgpu_buffer_rsrc_t ares = make_rsrc(g.a);
    uint32_t toff[TPIECES];
#pragma unroll
    for (int i = 0; i < TPIECES; ++i) {
        const int id = tid + NT * i;
        const int p = row0 + (id >> 3);
        const int pair = g.sorted[p];
        const int src = g.a_direct ? p : (pair < T ? pair / g.topk : 0);
        toff[i] = (uint32_t)src * (uint32_t)(g.k_in * 2) + (id & 7) * 16;
    }
    u32x4 tv[TPIECES];
    auto tload = [&](int step) {
#pragma unroll
        for (int i = 0; i < TPIECES; ++i) tv[i] = __builtin_amdgcn_raw_buffer_load_b128(ares, toff[i], step * PF_BK * 2, 0);
    };
    auto tstore = [&](uint8_t* buf) {
#pragma unroll
        for (int i = 0; i < TPIECES; ++i) {
            const int id = tid + NT * i;
            *reinterpret_cast<u32x4*>(buf + lds_off(id >> 3, id & 7)) = tv[i];
        }
    };

    // ---------------------------------------------------------- multipliers
    f32x4 acc[RT][TJ];
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int brow = lane & 15, g4 = lane >> 4;
    int jact = 0;  // token tiles holding a valid row (a prefix: the alignment pads each expert at the end)
#pragma unroll
    for (int j = 0; j < TJ; ++j) jact += __builtin_amdgcn_readfirstlane(g.sorted[row0 + 16 * j]) < T ? 1 : 0;
    // the MFMAs of token tiles j >= jact (padding only) are skipped, one
    // uniform branch per tile; the second half's LDS reads too when jact <= TJ/2
    // (DeepSeek-V2 shape, 4096 tokens: 75 of its 293 token tiles hold at most 16 rows)
    const bool full = jact > TJ / 2;
    // One K step multiplies this step's weights (dequantized during the
    // previous step, in registers) by the token tile in `cur`, and spreads the
    // dequantization of the next step's weights over the MFMAs of the first
    // half of the token tiles, so the VALU work of one step overlaps the matrix
    // work of the other instead of running ahead of it (the barrier that ends
    // each step keeps the waves of a SIMD in phase, which made the two phases
    // serial).  Each tile's raw weight registers are refilled with step + 2 as
    // soon as they are converted, one step ahead of their dequantization.  The token loads go out before the
    // weight loads, so waiting for them one step later does not wait for the
    // weights.
    constexpr int PIECES = RT * 2;  // dequantized A operands per step
    constexpr int HALF = TJ / 2;
    auto deq = [&](u32x4 (&an)[RT][2], auto P) {
        constexpr int t = decltype(P)::value / 2, kk = decltype(P)::value % 2;
        if constexpr (WBITS == 8) {
            an[t][kk] = dequant_w8x8<BF16>(w8[t][2 * kk], w8[t][2 * kk + 1]);
        } else {
            const uint32_t sv = sc[t];
            an[t][kk] = dequant_w4_f16_scaled(w4[t][kk], __builtin_bit_cast(f16x2, sv | (sv << 16)));
        }
        // pin the result here: without it the compiler sinks the conversion to
        // the first use, one step later, ahead of that step's MFMAs
        asm volatile("" : "+v"(an[t][kk]));
    };
    // B operands of one 16-row token tile (the two 32-channel halves of the step)
    auto bread = [&](int j, const uint8_t* cur, u32x4 (&b)[2]) {
        const int r = 16 * j + brow;
        b[0] = *reinterpret_cast<const u32x4*>(cur + lds_off(r, g4));
        b[1] = *reinterpret_cast<const u32x4*>(cur + lds_off(r, 4 + g4));
    };
    auto mma = [&](auto J, const u32x4 (&b)[2], const u32x4 (&ac)[RT][2]) {
        constexpr int j = decltype(J)::value;
#pragma unroll
        for (int t = 0; t < RT; ++t) acc[t][j] = mfma16x16x32<BF16>(ac[t][0], b[0], acc[t][j]);
#pragma unroll
        for (int t = 0; t < RT; ++t) acc[t][j] = mfma16x16x32<BF16>(ac[t][1], b[1], acc[t][j]);
    };
    // the B operands of token tile j + 1 are read from LDS before the MFMAs
    // of tile j are issued (two register sets), so the LDS latency is hidden
    // behind those MFMAs rather than waited for before each tile
    auto body = [&](int step, const uint8_t* cur, uint8_t* nxt, const u32x4 (&ac)[RT][2], u32x4 (&an)[RT][2]) {
        tstore(nxt);
        tload(min(step + 2, step_end - 1));  // the last steps reload step_end - 1: no branch
        u32x4 bx[2], by[2];
        bread(0, cur, bx);
        static_for<0, HALF>([&](auto J) {
            constexpr int j = decltype(J)::value;
            if constexpr (j % 2 == 0) {
                bread(j + 1, cur, by);
                if (j == 0 || j < jact) mma(J, bx, ac);
            } else {
                bread(j + 1, cur, bx);
                if (j < jact) mma(J, by, ac);
            }
            static_for<j * PIECES / HALF, (j + 1) * PIECES / HALF>([&](auto P) {
                deq(an, P);
                // tile t's raw registers are free once both its halves are
                // converted: refill them with step + 2 right away (one full
                // step of latency for every tile)
                if constexpr (decltype(P)::value % 2 == 1) wload_t(min(step + 2, step_end - 1), decltype(P)::value / 2);
            });
        });
        if (full) {
            static_for<HALF, TJ>([&](auto J) {
                constexpr int j = decltype(J)::value;
                if constexpr ((j - HALF) % 2 == 0) {
                    if constexpr (j + 1 < TJ) bread(j + 1, cur, by);
                    if (j < jact) mma(J, HALF % 2 == 0 ? bx : by, ac);
                } else {
                    if constexpr (j + 1 < TJ) bread(j + 1, cur, bx);
                    if (j < jact) mma(J, HALF % 2 == 0 ? by : bx, ac);
                }
            });
        }
        __syncthreads();
    };
    uint8_t* b0 = lds;
    uint8_t* b1 = lds + BUF;
    u32x4 aA[RT][2], aB[RT][2];
    tload(step0);
    wload(step0);
    tstore(b0);
    static_for<0, PIECES>([&](auto P) { deq(aA, P); });
    tload(min(step0 + 1, step_end - 1));
    wload(min(step0 + 1, step_end - 1));
    __syncthreads();
    for (int step = step0; step < step_end; step += 2) {
        body(step, b0, b1, aA, aB);
        if (step + 1 < step_end) body(step + 1, b1, b0, aB, aA);
    }

    // epilogue
    float* yslab = nullptr;
    if constexpr (STAGE != STAGE_GATE_UP)
        yslab = static_cast<float*>(g.out) + (size_t)blockIdx.z * ((size_t)T * g.n_out);
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
        const int p = row0 + 16 * j + brow;
        const int pair = g.sorted[p];
        if constexpr (STAGE == STAGE_GATE_UP) {
            const int N = g.n_out / 2;
#pragma unroll
            for (int q = 0; q < RT / 2; ++q) {
                const int gtile = rt0 + 2 * q;  // gate rows; gtile + 1 holds the matching up rows
                const int hcol = (gtile / 2) * TILE_ROWS + 4 * g4;
                float h[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float gt = acc[2 * q][j][r], up = acc[2 * q + 1][j][r];
                    if constexpr (WBITS == 8) {
                        gt *= act_to_f32<BF16>(se[gtile * TILE_ROWS + 4 * g4 + r]);
                        up *= act_to_f32<BF16>(se[(gtile + 1) * TILE_ROWS + 4 * g4 + r]);
                    }
                    h[r] = (pair < T) ? silu_f32(gt) * up : 0.0f;
                }
                u32x2 st;
                st[0] = (uint32_t)f32_to_act<BF16>(h[0]) | ((uint32_t)f32_to_act<BF16>(h[1]) << 16);
                st[1] = (uint32_t)f32_to_act<BF16>(h[2]) | ((uint32_t)f32_to_act<BF16>(h[3]) << 16);
                *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(g.out) + (size_t)p * N + hcol) = st;
            }
        } else {
            if (pair < T) {
                const float rw = (STAGE == STAGE_DOWN) ? g.topk_w[pair] : 1.0f;
#pragma unroll
                for (int t = 0; t < RT; ++t) {
                    const int n0 = (rt0 + t) * TILE_ROWS + 4 * g4;
                    f32x4 o;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float v = acc[t][j][r];
                        if constexpr (WBITS == 8) v *= act_to_f32<BF16>(se[n0 + r]);
                        o[r] = v * rw;
                    }
                    if (STAGE == STAGE_DOWN && g.y_act) {  // one K slice: the row rounded once to act
                        u32x2 st;
                        st[0] = (uint32_t)f32_to_act<BF16>(o[0]) | ((uint32_t)f32_to_act<BF16>(o[1]) << 16);
                        st[1] = (uint32_t)f32_to_act<BF16>(o[2]) | ((uint32_t)f32_to_act<BF16>(o[3]) << 16);
                        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(g.out) + (size_t)pair * g.n_out + n0) = st;
                    } else {
                        *reinterpret_cast<f32x4*>(yslab + (size_t)pair * g.n_out + n0) = o;
                    }
                }
            }
        }
    }
}

template <int WBITS, bool BF16, int STAGE, int NW, int RT, int BM, int OCC>
static void launch_prefill_cfg(const GemmArgs& g, int ksplit, hipStream_t s) {
    const dim3 grid(g.n_out / (NW * RT * 16), g.cap / BM, ksplit);
    hipLaunchKernelGGL((gemm_prefill_kernel<WBITS, BF16, STAGE, NW, RT, BM, OCC>), grid, dim3(NW * 64), 0, s, g);
}

// The 256 x 128 shape for int8 weights, built in a translation unit of its own
// (gemm_prefill_n256.hip, which includes this file with
// WQ_PREFILL_KERNEL_ONLY defined) that stays under the default instruction
// scheduler when this file is built under LLVM's iterative ILP one (a build
// option), which spills that shape's registers.
template <int WBITS, bool BF16, int STAGE>
void launch_prefill_n256(const GemmArgs& g, int ksplit, hipStream_t s);

#ifndef WQ_PREFILL_KERNEL_ONLY
// ------------------------------------------------------------------ plans
// Workgroup shapes (weight rows x token rows, waves, workgroups per CU):
//   N512  512 x 128, 8 waves, 1 per CU
//   N256  256 x 128, 4 waves, 2 per CU
//   N128  128 x 128, 4 waves (32 weight rows each), 3 per CU
//   T256  256 x 64,  4 waves, 2 per CU  (blocks of 64 token rows)
//   T128  128 x 64,  4 waves (32 weight rows each), 3 per CU
// Measured on MI355X with random data (Mixtral and DeepSeek-V2 shapes, int8
// and int4): N512 is the fastest where n_out allows it, at equal or fewer
// rounds of resident workgroups; int4 N256 spills registers; T128 is the
// faster GATE_UP shape for blocks of 64.
enum PrefillShape { PF_N512, PF_N256, PF_N128, PF_T256, PF_T128 };

struct ShapeInfo {
    int bn, bm, slots;  // weight rows, token rows, resident workgroups on 256 CUs
};
static ShapeInfo shape_info(PrefillShape sh) {
    switch (sh) {
        case PF_N512: return {512, 128, 256};
        case PF_N256: return {256, 128, 512};
        case PF_N128: return {128, 128, 768};
        case PF_T256: return {256, 64, 512};
        default: return {128, 64, 768};
    }
}

static PrefillShape prefill_shape(int wbits, int stage, int n_out, int k_in, int block_size) {
    if (block_size == 64) return (stage == STAGE_DOWN && n_out % 256 == 0) ? PF_T256 : PF_T128;
    // int8 DOWN with a reduction too short to split (under 32 K steps) takes
    // two 256-row workgroups per CU (DeepSeek-V2 shape, k_in 1536, M = 4096:
    // DOWN 715 -> 681 us; Mixtral M = 1024, 3 K slices, stays at 512 rows:
    // 278 against 284 us)
    if (n_out % 512 == 0 && !(stage == STAGE_DOWN && wbits == 8 && k_in < 32 * PF_BK)) return PF_N512;
    if (n_out % 256 == 0 && wbits == 8) return PF_N256;
    return PF_N128;
}

// expected count of bm-row token tiles: T rows plus, per touched expert, a
// half-filled last tile (at most E experts are touched)
static long est_mtiles(int T, int E, int bm) { return ((long)T + (long)std::min(T, E) * (bm / 2) + bm - 1) / bm; }

// K slices of DOWN for blocks of block_size rows: the smallest split in
// {1, 2, 3, 4} whose grid, counted in rounds of resident workgroups of 1/ks of
// the full K, takes at least 15 % fewer rounds than the smallest split before
// it, with at least 16 K steps per slice (slices of unequal length where ks
// does not divide the steps).  Measured (Mixtral int8 DOWN): M = 1024
// 337 -> 296 us (4 slices), M = 512 327 -> 184 us (2 slices).
int prefill_down_split(int T, int E, int n_out, int k_in, int block_size) {
    if (!prefill_supported(n_out, k_in, block_size) || T <= 0) return 1;
    const int steps = k_in / PF_BK;
    const ShapeInfo si = shape_info(prefill_shape(8, STAGE_DOWN, n_out, k_in, block_size));
    const long wgs = (long)(n_out / si.bn) * est_mtiles(T, E, si.bm);
    auto rounds = [&](int ks) { return (double)((wgs * ks + si.slots - 1) / si.slots) / ks; };
    int best = 1;
    double best_t = rounds(1);
    for (int ks = 2; ks <= 4; ++ks) {
        if (steps / ks < 16) break;
        const double t = rounds(ks);
        if (t < 0.85 * best_t) best = ks, best_t = t;
    }
    return best;
}

int prefill_down_split_max(int T, int E, int n_out, int k_in) {
    return std::max(prefill_down_split(T, E, n_out, k_in, 64), prefill_down_split(T, E, n_out, k_in, 128));
}

template <int WBITS, bool BF16, int STAGE>
static void launch_prefill_shape(PrefillShape sh, const GemmArgs& g, int ksplit, hipStream_t s) {
    switch (sh) {
        case PF_N512: launch_prefill_cfg<WBITS, BF16, STAGE, 8, 4, 128, 1>(g, ksplit, s); break;
        case PF_N256:  // int8 only
            if constexpr (WBITS == 8) launch_prefill_n256<WBITS, BF16, STAGE>(g, ksplit, s);
            else launch_prefill_cfg<WBITS, BF16, STAGE, 4, 2, 128, 3>(g, ksplit, s);
            break;
        case PF_N128: launch_prefill_cfg<WBITS, BF16, STAGE, 4, 2, 128, 3>(g, ksplit, s); break;
        case PF_T256: launch_prefill_cfg<WBITS, BF16, STAGE, 4, 4, 64, 2>(g, ksplit, s); break;
        default: launch_prefill_cfg<WBITS, BF16, STAGE, 4, 2, 64, 3>(g, ksplit, s); break;
    }
}

template <int WBITS, bool BF16>
static void launch_prefill_s(int stage, const GemmArgs& g, int ksplit, hipStream_t s) {
    const PrefillShape sh = prefill_shape(WBITS, stage, g.n_out, g.k_in, g.block_size);
    if (stage == STAGE_GATE_UP) launch_prefill_shape<WBITS, BF16, STAGE_GATE_UP>(sh, g, 1, s);
    else if (stage == STAGE_DOWN) launch_prefill_shape<WBITS, BF16, STAGE_DOWN>(sh, g, ksplit, s);
    else launch_prefill_shape<WBITS, BF16, STAGE_RAW>(sh, g, 1, s);
}

bool prefill_supported(int n_out, int k_in, int block_size) {
    return (block_size == 64 || block_size % 128 == 0) && n_out % 128 == 0 && k_in % PF_BK == 0;
}

bool prefill_fits(size_t rows, int k_in) { return rows * (size_t)k_in * 2 <= (size_t)0xffffffffu; }

int launch_gemm_prefill(int wbits, bool bf16, int stage, const GemmArgs& g, hipStream_t s) {
    const int ksplit =
        (stage == STAGE_DOWN) ? prefill_down_split(g.M * g.topk, g.E, g.n_out, g.k_in, g.block_size) : 1;
    if (wbits == 4) launch_prefill_s<4, false>(stage, g, ksplit, s);
    else if (bf16) launch_prefill_s<8, true>(stage, g, ksplit, s);
    else launch_prefill_s<8, false>(stage, g, ksplit, s);
    return ksplit;
}
#endif  // WQ_PREFILL_KERNEL_ONLY

}  // namespace wq

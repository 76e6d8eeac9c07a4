// gemm_decode.hip -- small-batch grouped GEMM of the quantized MoE layer.
//
// Work unit: one workgroup per (up to RMAX 16-row token sub-blocks of one
// expert, 16 weight rows) -- 32 rows for the fused gate/up stage, a gate tile
// and the matching up tile.  The grid runs over the sub-blocks of
// sorted_token_ids, so an expert holding many token blocks (skewed routing)
// is spread over several workgroups that run side by side, and experts no
// token chose launch nothing.  The weights are
// the MFMA A operand (16 rows x 32 input channels per v_mfma_f32_16x16x32),
// streamed once from HBM with 128-bit loads: a packed 1 KiB chunk gives every
// lane 16 bytes, i.e. 4 MFMA k-steps of int4 or 2 of int8.  The token rows of
// the expert (16 per MFMA, B operand) come from L2.  The four waves split the
// input channels and meet in LDS; one pass covers up to RMAX 16-row token
// blocks, so the weights are read once for all of them.  Dequantisation is
// in registers: int4 -> fp16 by exponent bits, group scale folded in fp32 per
// 128-channel chunk; int8 -> bf16/fp16 exactly, per-column scale in the fp32
// epilogue.  Epilogues: SiLU(gate)*up to H (sorted rows), or the routed weight
// times the down projection to the per-pair buffer Y.
//
// Sources: int4 GPTQ group-128 experts ("Marlin moe integration", nm-vllm PR
// 266, opening description); per-column int8 experts cast to the activation
// type inside the kernel ("[Kernel] W8A16 Int8 inside FusedMoE", vLLM PR 7415,
// opening description); small-batch kernels chosen by batch size ("[WIP] AWQ
// Faster Kernels", vLLM issue 3289, the GEMV/GEMM mix and the batch-dimension
// heuristics).
#include "common.hpp"
#include "launch.hpp"
#include "route_common.hpp"

#include <algorithm>
#include <type_traits>

namespace wq {

// Kernel shape: NP weight-row tiles per workgroup (pairs of gate+up tiles for
// the fused stage), NW waves splitting the input channels, DEPTH 1 KiB chunks
// per tile in flight per wave, up to RMAX 16-row token blocks per pass.
// FR: the workgroup first routes and sorts the batch itself (every workgroup
// the same, in LDS; the first one also writes the routing arrays for the
// later stages), so route, sort and gate/up are one launch.  For batches of at
// most FR_MAX_PAIRS pairs over at most 64 experts and a capacity of at most
// FR_MAX_CAP rows.
// AO (with FR, one token of an act-order layer): the workgroup gathers the
// token's row in its expert's channel order, x[perm[e][k]], into LDS (the
// values the act-order gather launch writes) and reads every B operand there.
template <int WBITS, bool BF16, int STAGE, int RMAX, int NP, int NW, int DEPTH, bool FR = false, bool AO = false>
__global__ __launch_bounds__(64 * NW) void gemm_decode_kernel(GemmArgs g, RouteArgs ra) {
    constexpr int NT = (STAGE == STAGE_GATE_UP) ? 2 * NP : NP;  // 16-row tiles per workgroup
    constexpr int KCHUNK = WFmt<WBITS>::KCHUNK;
    constexpr int KSTEPS = KCHUNK / 32;
    static_assert(NW * NT * RMAX * 1024 <= 64 * 1024, "LDS reduction buffer");
    static_assert(RMAX == 1 || RMAX == 2 || RMAX == 4, "passes of RMAX, then 2 and/or 1 blocks");

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int unit = blockIdx.x;
    const int T = g.M * g.topk;
    const int BS = g.block_size;
    const int spb = BS / 16;
    __shared__ f32x4 red[NW][NT][RMAX][64];
    extern __shared__ __attribute__((aligned(16))) uint16_t ao_x[];  // AO: the gathered row, k_in values
    static_assert(!AO || (FR && WBITS == 4 && STAGE == STAGE_GATE_UP), "act-order rows in LDS: one-token int4 GATE_UP");

    // the routing arrays: the caller's, or (FR) computed here into LDS
    const int32_t* sorted_ids = g.sorted;
    const int32_t* block_expert = g.expert_ids;
    int ntpp;
    if constexpr (FR) {
        __shared__ int fr_sorted[FR_MAX_CAP];
        __shared__ int fr_blocks[FR_MAX_CAP / 16];
        __shared__ int fr_ids[FR_MAX_PAIRS];
        __shared__ float fr_w[FR_MAX_PAIRS];
        __shared__ int fr_ntpp;
        for (int m = wave; m < g.M; m += NW)  // E <= 64: the rank-counting top-k
            route_token_rank(ra.logits + (size_t)m * g.E, g.E, g.topk, ra.renormalize, lane, fr_w + m * g.topk,
                             fr_ids + m * g.topk, nullptr);
        __syncthreads();
        if (wave == 0) align_wave(fr_ids, T, g.E, BS, g.cap, lane, fr_sorted, fr_blocks, &fr_ntpp);
        __syncthreads();
        if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0) {
            for (int i = threadIdx.x; i < T; i += 64 * NW) {
                ra.w_out[i] = fr_w[i];
                ra.ids_out[i] = fr_ids[i];
            }
            for (int i = threadIdx.x; i < g.cap; i += 64 * NW) ra.sorted_out[i] = fr_sorted[i];
            for (int i = threadIdx.x; i < g.cap / BS; i += 64 * NW) ra.expert_ids_out[i] = fr_blocks[i];
            if (threadIdx.x == 0) *ra.ntpp_out = fr_ntpp;
        }
        sorted_ids = fr_sorted;
        block_expert = fr_blocks;
        ntpp = fr_ntpp;
    } else {
        ntpp = *g.ntpp;
    }

    // 16-row sub-block sbi of sorted_token_ids (grid y, then z past 65535), in block b.  The lanes read the
    // expert ids of blocks b - 31 .. b + 32 at once; the used blocks of one
    // expert are contiguous, so the lanes holding b's expert form one run
    // around lane 31 (searched for beyond the window only when it reaches an end)
    const int sbi = blockIdx.y + 65535 * blockIdx.z;
    const int b = sbi / spb;
    const int bi = b - 31 + lane;
    const int ecand = (bi >= 0 && bi < g.cap / BS) ? block_expert[bi] : -1;
    if (sbi * 16 >= ntpp) return;
    const int nbu = ntpp / BS;
    const int e = __shfl(ecand, 31);
    const uint64_t run = __ballot(bi >= 0 && bi < nbu && ecand == e);
    const int b0 = (run & 1ull) ? lower_bound_i32(block_expert, 0, b - 31, e) : b - 31 + __builtin_ctzll(run);
    const int b1 = (run >> 63) ? lower_bound_i32(block_expert, b + 33, nbu, e + 1) : b - 31 + 64 - __builtin_clzll(run);
    const int sb_first = b0 * spb;
    const int j = sbi - sb_first;  // sub-block index within the expert
    if (j % RMAX != 0) return;     // one workgroup per RMAX sub-blocks
    // live 16-row sub-blocks of the expert's last block (those whose first row
    // is a real pair: a prefix of the block)
    const int q = __popcll(__ballot(lane < spb && sorted_ids[(b1 - 1) * BS + 16 * min(lane, spb - 1)] < T));
    const int S = (b1 - 1 - b0) * spb + q;

    const int C = g.k_in / KCHUNK;
    const size_t expert_bytes = (size_t)(g.n_out / TILE_ROWS) * C * CHUNK_BYTES;
    const uint8_t* wt[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
        wt[t] = g.w + (size_t)e * expert_bytes + (size_t)(NT * unit + t) * C * CHUNK_BYTES + lane * 16;
    const uint16_t* se = g.s + (size_t)e * g.groups * g.n_out;
    const int rowq = 4 * (lane >> 4);  // first of this lane's 4 output rows in a tile
    const bool grouped = (WBITS == 4) && g.groups > 1;

    // one pass multiplies R token blocks (a compile-time count: full passes take
    // RMAX, the remainder one pass of 2 and/or 1), so no load depends on R
    auto pass = [&](const int s0, auto RC) {
        constexpr int R = decltype(RC)::value;
        constexpr int ITEMS_R = NP * R;  // epilogue items (tile or tile pair, token block)
        const uint16_t* arow[R];
        bool avalid[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            // pad rows read the block's first row, a real one (same address as
            // lane 0: one fetch; their H rows are written as 0, their other
            // outputs dropped), so every load below is unconditional
            const int p_first = (sb_first + s0 + r) * 16;
            const int p = p_first + (lane & 15);
            const int pair = sorted_ids[p];
            avalid[r] = pair < T;
            const int pl = avalid[r] ? p : p_first;
            const int row = g.a_direct ? pl : sorted_ids[pl] / g.topk;
            arow[r] = g.a + (size_t)row * g.k_in + 8 * (lane >> 4);
        }

        f32x4 acc[NT][R];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < R; ++r) acc[t][r] = f32x4{0.f, 0.f, 0.f, 0.f};

        // DEPTH rotating buffers of one chunk each
        u32x4 wv[DEPTH][NT];
        u32x4 xv[DEPTH][R][KSTEPS];
        u32x2 sv[DEPTH][NT];

        // no load sits under a branch: a branch would make the compiler wait for
        // every load in flight before the next multiply
        auto load = [&](int c, int d) {
#pragma unroll
            for (int t = 0; t < NT; ++t) wv[d][t] = ldg128_stream(wt[t] + (size_t)c * CHUNK_BYTES);
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int s = 0; s < KSTEPS; ++s) {
                    if constexpr (AO) xv[d][r][s] = *reinterpret_cast<const u32x4*>(ao_x + c * KCHUNK + 32 * s + 8 * (lane >> 4));
                    else xv[d][r][s] = ldg128(arow[r] + c * KCHUNK + 32 * s);
                }
            if constexpr (WBITS == 4) {
                const size_t gc = grouped ? (size_t)c : 0;  // per-column scales: a harmless reread of group 0
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    sv[d][t] = *reinterpret_cast<const u32x2*>(se + gc * g.n_out + (NT * unit + t) * TILE_ROWS + rowq);
            }
        };

        auto compute = [&](int d) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                if constexpr (WBITS == 4) {
                    f32x4 part[R];
#pragma unroll
                    for (int r = 0; r < R; ++r) part[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < KSTEPS; ++s) {
                        const u32x4 a = dequant_w4_f16(wv[d][t][s]);
#pragma unroll
                        for (int r = 0; r < R; ++r) part[r] = mfma16x16x32<false>(a, xv[d][r][s], part[r]);
                    }
                    if (grouped) {
                        const uint32_t lo = sv[d][t][0], hi = sv[d][t][1];
                        const float s0f = f16_to_f32((uint16_t)(lo & 0xffffu));
                        const float s1f = f16_to_f32((uint16_t)(lo >> 16));
                        const float s2f = f16_to_f32((uint16_t)(hi & 0xffffu));
                        const float s3f = f16_to_f32((uint16_t)(hi >> 16));
#pragma unroll
                        for (int r = 0; r < R; ++r) {
                            acc[t][r][0] += part[r][0] * s0f;
                            acc[t][r][1] += part[r][1] * s1f;
                            acc[t][r][2] += part[r][2] * s2f;
                            acc[t][r][3] += part[r][3] * s3f;
                        }
                    } else {
#pragma unroll
                        for (int r = 0; r < R; ++r) acc[t][r] += part[r];
                    }
                } else {
#pragma unroll
                    for (int s = 0; s < KSTEPS; ++s) {
                        const u32x4 a = dequant_w8x8<BF16>(wv[d][t][2 * s], wv[d][t][2 * s + 1]);
#pragma unroll
                        for (int r = 0; r < R; ++r) acc[t][r] = mfma16x16x32<BF16>(a, xv[d][r][s], acc[t][r]);
                    }
                }
            }
        };

        // split-K over the waves; DEPTH - 1 chunks in flight while one is
        // multiplied.  Chunk indices past the end are clamped to this wave's
        // last chunk (a cache hit), keeping every load unconditional.
        // (a wave without chunks, C <= wave, loads chunk C - 1 and multiplies nothing)
        const int clast = wave < C ? wave + ((C - 1 - wave) / NW) * NW : C - 1;
#pragma unroll
        for (int i = 0; i < DEPTH - 1; ++i) load(min(wave + i * NW, clast), i);
        for (int base = wave; base < C; base += DEPTH * NW) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                const int c = base + d * NW;
                load(min(c + (DEPTH - 1) * NW, clast), (d + DEPTH - 1) % DEPTH);
                if (c < C) compute(d);
            }
        }

#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < R; ++r) red[wave][t][r][lane] = acc[t][r];
        __syncthreads();

        for (int item = wave; item < ITEMS_R; item += NW) {
            const int pp = item / R;  // tile (or gate/up tile pair) within the workgroup
            const int r = item % R;
            const int p = (sb_first + s0 + r) * 16 + (lane & 15);
            const int pair = sorted_ids[p];
            if constexpr (STAGE == STAGE_GATE_UP) {
                const int tg = 2 * pp, tu = 2 * pp + 1;  // gate and up tile within the workgroup
                f32x4 gv = red[0][tg][r][lane], uv = red[0][tu][r][lane];
#pragma unroll
                for (int w = 1; w < NW; ++w) {
                    gv += red[w][tg][r][lane];
                    uv += red[w][tu][r][lane];
                }
                const int N = g.n_out / 2;
                const int hcol = (NP * unit + pp) * TILE_ROWS + rowq;
                float h[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float gt = gv[i], up = uv[i];
                    if (!grouped) {
                        gt *= act_to_f32<BF16>(se[(NT * unit + tg) * TILE_ROWS + rowq + i]);
                        up *= act_to_f32<BF16>(se[(NT * unit + tu) * TILE_ROWS + rowq + i]);
                    }
                    h[i] = pair < T ? silu_f32(gt) * up : 0.0f;
                }
                u32x2 st;
                st[0] = (uint32_t)f32_to_act<BF16>(h[0]) | ((uint32_t)f32_to_act<BF16>(h[1]) << 16);
                st[1] = (uint32_t)f32_to_act<BF16>(h[2]) | ((uint32_t)f32_to_act<BF16>(h[3]) << 16);
                *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(g.out) + (size_t)p * N + hcol) = st;
            } else {
                if (pair < T) {
                    f32x4 o = red[0][pp][r][lane];
#pragma unroll
                    for (int w = 1; w < NW; ++w) o += red[w][pp][r][lane];
                    const int row = (NT * unit + pp) * TILE_ROWS + rowq;
                    if (!grouped) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) o[i] *= act_to_f32<BF16>(se[row + i]);
                    }
                    if constexpr (STAGE == STAGE_DOWN) o *= g.topk_w[pair];
                    *reinterpret_cast<f32x4*>(static_cast<float*>(g.out) + (size_t)pair * g.n_out + row) = o;
                }
            }
        }
        __syncthreads();
    };
    if constexpr (STAGE == STAGE_GATE_UP) {
        // H rows of all-pad sub-blocks (only with blocks larger than 16) are
        // zero; the expert's first workgroup writes them
        if (j == 0) {
            const int N = g.n_out / 2;
            const int p_lo = (sb_first + S) * 16;
            const int p_hi = b1 * BS;
            constexpr int COLS = NP * TILE_ROWS;
            for (int k = threadIdx.x; k < (p_hi - p_lo) * COLS; k += 64 * NW) {
                const int p = p_lo + k / COLS;
                static_cast<uint16_t*>(g.out)[(size_t)p * N + NP * unit * TILE_ROWS + (k % COLS)] = 0;
            }
        }
    }
    if (j >= S) return;
    if constexpr (AO) {
        // one token (M == 1): every real row of the expert is row 0 of x
        const int32_t* pe = ra.perm + (size_t)e * g.k_in;
        for (int k = threadIdx.x * 8; k < g.k_in; k += 64 * NW * 8) {
            const u32x4 i0 = ldg128(pe + k);
            const u32x4 i1 = ldg128(pe + k + 4);
            u32x4 v;
            v[0] = (uint32_t)g.a[i0[0]] | ((uint32_t)g.a[i0[1]] << 16);
            v[1] = (uint32_t)g.a[i0[2]] | ((uint32_t)g.a[i0[3]] << 16);
            v[2] = (uint32_t)g.a[i1[0]] | ((uint32_t)g.a[i1[1]] << 16);
            v[3] = (uint32_t)g.a[i1[2]] | ((uint32_t)g.a[i1[3]] << 16);
            *reinterpret_cast<u32x4*>(ao_x + k) = v;
        }
        __syncthreads();
    }
    // sub-blocks j .. j + RMAX - 1 of the expert: one pass of RMAX, or of 2
    // and/or 1 for the expert's last R < RMAX
    const int R = min(RMAX, S - j);
    if (R == RMAX) {
        pass(j, std::integral_constant<int, RMAX>{});
    } else {
        int s0 = j;
        if constexpr (RMAX >= 4) {
            if (R >= 2) {
                pass(s0, std::integral_constant<int, 2>{});
                s0 += 2;
            }
        }
        if constexpr (RMAX >= 2) {
            if (s0 < j + R) pass(s0, std::integral_constant<int, 1>{});
        }
    }
}

template <int WBITS, bool BF16, int STAGE, int RMAX, int NP, int NW, int DEPTH, bool FR = false, bool AO = false>
static void launch_decode_cfg(const GemmArgs& g, hipStream_t s, const RouteArgs& ra = RouteArgs{}) {
    constexpr int NT = (STAGE == STAGE_GATE_UP) ? 2 * NP : NP;
    const int nsb = g.cap / 16;  // 16-row sub-blocks, over grid y (at most 65535) and z
    const dim3 grid(g.n_out / (TILE_ROWS * NT), std::min(nsb, 65535), (nsb + 65534) / 65535);
    hipLaunchKernelGGL((gemm_decode_kernel<WBITS, BF16, STAGE, RMAX, NP, NW, DEPTH, FR, AO>), grid, dim3(64 * NW),
                       AO ? (size_t)g.k_in * 2 : 0, s, g, ra);
}

// Shapes by batch, measured on MI355X with the last-level cache flushed before
// every launch (Mixtral-shaped int8 and int4 layers, and the 160-expert int8
// layer with skewed routing).  One token block per
// pass when experts are thin, two up to ~24 rows per expert, four beyond
// (larger batches normally take the large-batch kernel).  The waves of a
// workgroup split the input channels, so their count follows the number of
// 1 KiB chunks per weight row tile C: a short reduction (C <= 32) keeps 2
// waves with 2 or 4 row tiles, a long one 8 waves; int4 (half the bytes per
// weight, so half the work per wave) takes two gate/up tile pairs per
// workgroup, and four row tiles in DOWN once that grid still fills the GPU.
// The int4 gate/up of one or two tokens (at most 4 pairs) splits K over 2
// waves instead of 4 (Mixtral act-order layer M = 1: 66.6 -> 65.3 us; 4 and
// 16 tokens measured slower that way).
// A single expert (the dense linear layer: the grid is one expert's tiles)
// takes 4 row tiles on 4 waves for int4 and 2 on 2 waves for int8 (7168 ->
// 20480, 16 tokens: int4 47.9 -> 32.5 us, int8 42.7 -> 39.3 us).
// Both stages of a many-expert layer (E >= 64, skewed routing) take two token
// blocks per pass whatever the mean rows per expert: its head experts hold
// several blocks (DeepSeek-V2 shape M = 64: gate/up 157 -> 132 us in the
// layer).
// DOWN of a long reduction (Mixtral, 224 int8 or 112 int4 chunks per row
// tile) takes four row tiles on 8 waves: every token row a wave loads then
// feeds four tiles instead of two (the token rows, read again by every
// workgroup of the expert, are most of what a wave loads at 16 rows per
// expert) -- Mixtral M = 64: int8 DOWN 106 -> 96 us, int4 100 -> 72 us;
// int8 M = 32: 90 -> 83 us, M = 8: 75 -> 73 us (int4 keeps its 4-wave shape
// there); one tile per workgroup (twice the token reads) ran 164-173 us at
// M = 64, eight (32 workgroups per expert) 167 us.
template <int WBITS, bool BF16, int STAGE>
static void launch_decode_r(const GemmArgs& g, hipStream_t s) {
    constexpr bool GU = STAGE == STAGE_GATE_UP;
    constexpr int NT1 = GU ? 2 : 1;
    const int T = g.M * g.topk;
    const int touched = T < g.E ? T : g.E;
    const int rows = (T + touched - 1) / touched;  // expected rows per touched expert
    const bool np2_ok = (g.n_out % (TILE_ROWS * NT1 * 2)) == 0;
    const bool np4_ok = (g.n_out % (TILE_ROWS * NT1 * 4)) == 0;
    const bool short_k = g.k_in / WFmt<WBITS>::KCHUNK <= 32;
    // workgroups of a 4-tile DOWN grid over the touched experts
    const long wg4 = (long)touched * (g.n_out / (TILE_ROWS * 4));
    if (GU && g.E >= 64 && T > 16 && np2_ok) {
        // many experts with skewed routing: the head experts hold several token
        // blocks, which one block per pass would stream their weights for each
        launch_decode_cfg<WBITS, BF16, STAGE, 2, 2, 4, 2>(g, s);
    } else if (!GU && g.E >= 64 && T > 16 && short_k && np4_ok) {
        // the same for DOWN, whose short rows (few chunks) take 4 row tiles
        // on 2 waves (DeepSeek-V2 shape M = 64: 93.7 -> 85.1 us)
        launch_decode_cfg<WBITS, BF16, STAGE, 2, 4, 2, 2>(g, s);
    } else if (T <= 16 || rows <= 8) {
        if (GU && WBITS == 4 && np2_ok && T <= 4) launch_decode_cfg<WBITS, BF16, STAGE, 1, 2, 2, 2>(g, s);
        else if (GU && WBITS == 4 && np2_ok) launch_decode_cfg<WBITS, BF16, STAGE, 1, 2, 4, 2>(g, s);
        else if (GU) launch_decode_cfg<WBITS, BF16, STAGE, 1, 1, 4, 2>(g, s);
        else if (!np2_ok) launch_decode_cfg<WBITS, BF16, STAGE, 1, 1, 8, 4>(g, s);
        else if (g.E == 1 && WBITS == 4 && np4_ok) launch_decode_cfg<WBITS, BF16, STAGE, 1, 4, 4, 2>(g, s);
        else if (g.E == 1) launch_decode_cfg<WBITS, BF16, STAGE, 1, 2, 2, 4>(g, s);
        else if (short_k) launch_decode_cfg<WBITS, BF16, STAGE, 1, 2, 2, 3>(g, s);
        else if (WBITS == 4 && np4_ok && wg4 >= 512) launch_decode_cfg<WBITS, BF16, STAGE, 1, 4, 4, 2>(g, s);
        else if (WBITS == 8 && np4_ok) launch_decode_cfg<WBITS, BF16, STAGE, 1, GU ? 1 : 4, 8, 2>(g, s);
        else launch_decode_cfg<WBITS, BF16, STAGE, 1, 2, 8, 3>(g, s);
    } else if (rows <= 24) {
        if (!GU && short_k && np4_ok) launch_decode_cfg<WBITS, BF16, STAGE, 2, 4, 2, 2>(g, s);
        else if (!GU && np4_ok) launch_decode_cfg<WBITS, BF16, STAGE, 2, GU ? 1 : 4, 8, 2>(g, s);
        else if (np2_ok) launch_decode_cfg<WBITS, BF16, STAGE, 2, 2, 4, 2>(g, s);
        else launch_decode_cfg<WBITS, BF16, STAGE, 2, 1, 4, 2>(g, s);
    } else {
        if (!GU && np2_ok) launch_decode_cfg<WBITS, BF16, STAGE, 4, 2, 4, 2>(g, s);
        else launch_decode_cfg<WBITS, BF16, STAGE, 4, 1, 4, 2>(g, s);
    }
}

// the GATE_UP shapes launch_decode_r picks for up to 16 pairs, with the routing done in the kernel
bool decode_route_supported(int stage, int M, int topk, int E, int cap, int block_size) {
    const long T = (long)M * topk;
    return stage == STAGE_GATE_UP && M >= 1 && T <= 16 && T <= FR_MAX_PAIRS && E >= 1 && E <= 64 &&
           cap <= FR_MAX_CAP && (block_size == 16 || block_size == 32);
}

bool decode_route_ao_supported(int M, int topk, int n_out, int k_in) {
    return M == 1 && topk <= 16 && n_out % (TILE_ROWS * 2 * 2) == 0 && k_in <= DECODE_AO_MAX_K && k_in % 8 == 0;
}

template <int WBITS, bool BF16>
static void launch_decode_route_w(const GemmArgs& g, const RouteArgs& ra, hipStream_t s) {
    const int T = g.M * g.topk;
    const bool np2_ok = (g.n_out % (TILE_ROWS * 2 * 2)) == 0;
    if constexpr (WBITS == 4) {
        if (ra.perm) {  // decode_route_ao_supported: the shapes launch_decode_r picks for one int4 token
            if (T <= 4) launch_decode_cfg<WBITS, BF16, STAGE_GATE_UP, 1, 2, 2, 2, true, true>(g, s, ra);
            else launch_decode_cfg<WBITS, BF16, STAGE_GATE_UP, 1, 2, 4, 2, true, true>(g, s, ra);
            return;
        }
    }
    if (WBITS == 4 && np2_ok && T <= 4) launch_decode_cfg<WBITS, BF16, STAGE_GATE_UP, 1, 2, 2, 2, true>(g, s, ra);
    else if (WBITS == 4 && np2_ok) launch_decode_cfg<WBITS, BF16, STAGE_GATE_UP, 1, 2, 4, 2, true>(g, s, ra);
    else launch_decode_cfg<WBITS, BF16, STAGE_GATE_UP, 1, 1, 4, 2, true>(g, s, ra);
}

void launch_gemm_decode_route(int wbits, bool bf16, const GemmArgs& g, const RouteArgs& ra, hipStream_t s) {
    if (wbits == 4) launch_decode_route_w<4, false>(g, ra, s);
    else if (bf16) launch_decode_route_w<8, true>(g, ra, s);
    else launch_decode_route_w<8, false>(g, ra, s);
}

template <int WBITS, bool BF16>
static void launch_decode_s(int stage, const GemmArgs& g, hipStream_t s) {
    if (stage == STAGE_GATE_UP) launch_decode_r<WBITS, BF16, STAGE_GATE_UP>(g, s);
    else if (stage == STAGE_DOWN) launch_decode_r<WBITS, BF16, STAGE_DOWN>(g, s);
    else launch_decode_r<WBITS, BF16, STAGE_RAW>(g, s);
}

void launch_gemm_decode(int wbits, bool bf16, int stage, const GemmArgs& g, hipStream_t s) {
    if (wbits == 4) launch_decode_s<4, false>(stage, g, s);  // int4: fp16 activations
    else if (bf16) launch_decode_s<8, true>(stage, g, s);
    else launch_decode_s<8, false>(stage, g, s);
}

// ---------------------------------------------------------------------------
// act-order gather: A1[p, k'] = x[token(p), perm[e(p), k']], zero rows for pads
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gather_perm_kernel(const uint16_t* __restrict__ x,
                                                          const int32_t* __restrict__ perm,
                                                          const int32_t* __restrict__ sorted,
                                                          const int32_t* __restrict__ expert_ids,
                                                          const int32_t* __restrict__ ntpp, int topk, int T, int k_in,
                                                          int BS, uint16_t* __restrict__ a1) {
    const int p = blockIdx.x;
    if (p >= *ntpp) return;
    const int pair = sorted[p];
    uint16_t* dst = a1 + (size_t)p * k_in;
    if (pair >= T) {
        for (int k = threadIdx.x * 8; k < k_in; k += 256 * 8)
            *reinterpret_cast<u32x4*>(dst + k) = u32x4{0u, 0u, 0u, 0u};
        return;
    }
    const int e = expert_ids[p / BS];
    const uint16_t* src = x + (size_t)(pair / topk) * k_in;
    const int32_t* pe = perm + (size_t)e * k_in;
    for (int k = threadIdx.x * 8; k < k_in; k += 256 * 8) {
        const u32x4 i0 = ldg128(pe + k);
        const u32x4 i1 = ldg128(pe + k + 4);
        u32x4 v;
        v[0] = (uint32_t)src[i0[0]] | ((uint32_t)src[i0[1]] << 16);
        v[1] = (uint32_t)src[i0[2]] | ((uint32_t)src[i0[3]] << 16);
        v[2] = (uint32_t)src[i1[0]] | ((uint32_t)src[i1[1]] << 16);
        v[3] = (uint32_t)src[i1[2]] | ((uint32_t)src[i1[3]] << 16);
        *reinterpret_cast<u32x4*>(dst + k) = v;
    }
}

void launch_gather_perm(const uint16_t* x, const int32_t* perm, const int32_t* sorted, const int32_t* expert_ids,
                        const int32_t* ntpp, int M, int topk, int k_in, int block_size, int cap, uint16_t* a1,
                        hipStream_t s) {
    hipLaunchKernelGGL(gather_perm_kernel, dim3(cap), dim3(256), 0, s, x, perm, sorted, expert_ids, ntpp, topk,
                       M * topk, k_in, block_size, a1);
}

// ---------------------------------------------------------------------------
// top-k weighted combine: out[m, c] = sum_{j<topk} sum_{z<ksplit} Y[z][m*topk+j, c]
// (Y already carries the routed weight; z runs over the K slices of a split
// DOWN stage), ascending j then z in fp32, one rounding to act
// ---------------------------------------------------------------------------
constexpr int COMBINE_MAXT = 16;  // terms loaded together (topk * K slices)

template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, int M, int topk, int n, int ksplit,
                                                      uint16_t* __restrict__ out) {
    const size_t q = (size_t)blockIdx.x * 256 + threadIdx.x;  // 4 outputs each
    const size_t total = (size_t)M * n / 4;
    if (q >= total) return;
    const size_t m = q * 4 / n;
    const int c = (int)(q * 4 % n);
    const size_t slab = (size_t)M * topk * n;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int cnt = topk * ksplit;  // terms, in summation order i = j * ksplit + z
    if (cnt <= COMBINE_MAXT) {
        // every load issued before the first add: all terms in flight at once
        f32x4 v[COMBINE_MAXT];
        int j = 0, z = 0;
#pragma unroll
        for (int i = 0; i < COMBINE_MAXT; ++i) {
            if (i < cnt) v[i] = *reinterpret_cast<const f32x4*>(y + z * slab + (m * topk + j) * n + c);
            if (++z == ksplit) z = 0, ++j;
        }
#pragma unroll
        for (int i = 0; i < COMBINE_MAXT; ++i)
            if (i < cnt) acc += v[i];
    } else {
        for (int j = 0; j < topk; ++j)
            for (int z = 0; z < ksplit; ++z) acc += *reinterpret_cast<const f32x4*>(y + z * slab + (m * topk + j) * n + c);
    }
    u32x2 st;
    st[0] = (uint32_t)f32_to_act<BF16>(acc[0]) | ((uint32_t)f32_to_act<BF16>(acc[1]) << 16);
    st[1] = (uint32_t)f32_to_act<BF16>(acc[2]) | ((uint32_t)f32_to_act<BF16>(acc[3]) << 16);
    *reinterpret_cast<u32x2*>(out + m * n + c) = st;
}

// the same sum over Y rows already rounded to the activation type (a large-
// batch DOWN without a K split writes them so): each term widened exactly to
// fp32, ascending j, one rounding
template <bool BF16>
__global__ __launch_bounds__(256) void combine_act_kernel(const uint16_t* __restrict__ y, int M, int topk, int n,
                                                          uint16_t* __restrict__ out) {
    const size_t q = (size_t)blockIdx.x * 256 + threadIdx.x;  // 4 outputs each
    const size_t total = (size_t)M * n / 4;
    if (q >= total) return;
    const size_t m = q * 4 / n;
    const int c = (int)(q * 4 % n);
    const uint16_t* row = y + m * topk * n + c;  // pair m * topk + j at row + j * n
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    auto add = [&](u32x2 v) {
        const uint32_t lo = v[0], hi = v[1];
        acc[0] += act_to_f32<BF16>((uint16_t)(lo & 0xffffu));
        acc[1] += act_to_f32<BF16>((uint16_t)(lo >> 16));
        acc[2] += act_to_f32<BF16>((uint16_t)(hi & 0xffffu));
        acc[3] += act_to_f32<BF16>((uint16_t)(hi >> 16));
    };
    int j = 0;
    for (; j + 4 <= topk; j += 4) {  // four rows in flight at once
        const u32x2 v0 = *reinterpret_cast<const u32x2*>(row + (size_t)j * n);
        const u32x2 v1 = *reinterpret_cast<const u32x2*>(row + (size_t)(j + 1) * n);
        const u32x2 v2 = *reinterpret_cast<const u32x2*>(row + (size_t)(j + 2) * n);
        const u32x2 v3 = *reinterpret_cast<const u32x2*>(row + (size_t)(j + 3) * n);
        add(v0);
        add(v1);
        add(v2);
        add(v3);
    }
    for (; j < topk; ++j) add(*reinterpret_cast<const u32x2*>(row + (size_t)j * n));
    u32x2 st;
    st[0] = (uint32_t)f32_to_act<BF16>(acc[0]) | ((uint32_t)f32_to_act<BF16>(acc[1]) << 16);
    st[1] = (uint32_t)f32_to_act<BF16>(acc[2]) | ((uint32_t)f32_to_act<BF16>(acc[3]) << 16);
    *reinterpret_cast<u32x2*>(out + m * n + c) = st;
}

void launch_combine_act(const uint16_t* y, int M, int topk, int n, bool bf16, uint16_t* out, hipStream_t s) {
    const size_t total = (size_t)M * n / 4;
    const dim3 grid((unsigned)((total + 255) / 256));
    if (bf16) hipLaunchKernelGGL(combine_act_kernel<true>, grid, dim3(256), 0, s, y, M, topk, n, out);
    else hipLaunchKernelGGL(combine_act_kernel<false>, grid, dim3(256), 0, s, y, M, topk, n, out);
}

void launch_combine(const float* y, int M, int topk, int n, int ksplit, bool bf16, uint16_t* out, hipStream_t s) {
    const size_t total = (size_t)M * n / 4;
    const dim3 grid((unsigned)((total + 255) / 256));
    if (bf16) hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(256), 0, s, y, M, topk, n, ksplit, out);
    else hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(256), 0, s, y, M, topk, n, ksplit, out);
}

}  // namespace wq

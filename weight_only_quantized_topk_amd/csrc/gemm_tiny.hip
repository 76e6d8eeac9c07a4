// gemm_tiny.hip -- grouped GEMM of the quantized MoE layer for batches of a
// few tokens.
//
// With M tokens each expert receives at most M rows (top-k picks distinct
// experts per token), and its real rows are a prefix of its block(s) of
// sorted_token_ids.  One workgroup per (used block of sorted_token_ids, NT
// 16-row weight tiles of the block's expert) -- no workgroups for the experts
// no token chose, whose launches alone cost microseconds when E is large: the
// block's token rows are staged in LDS once, before the chunk loop --
// gathered through the expert's act-order permutation when one is given, so
// no gathered copy of x is written -- together with the tiles' int4 group
// scales, so the loop's only global loads are the weight stream: NW waves
// split the 1 KiB chunks of the tiles (wave w takes chunks w, w + NW, ...),
// DEPTH chunks per tile in flight.  The MFMA B operand's 16 columns read token
// rows min(column, nv - 1); columns at or beyond nv are dropped, and H rows of
// the expert's pad entries are written as 0, as the other small-batch kernel
// does.  The LDS holds M rows; an expert with more (a token's top-k naming it
// twice) is multiplied in passes of M rows, each streaming the weights again.
// Numerics are those of the other small-batch kernel: int4 codes exact in
// fp16 with the group scale on the fp32 partial sum of each 128-channel chunk,
// int8 exact with the per-column scale in the fp32 epilogue; the NW partial
// sums are added in LDS in wave order.
//
// Sources: int4 GPTQ group-128 experts with act-order ("Marlin moe
// integration", nm-vllm PR 266, opening description); per-column int8 experts
// ("[Kernel] W8A16 Int8 inside FusedMoE", vLLM PR 7415, opening description);
// a GEMV-like kernel for the smallest batches ("[WIP] AWQ Faster Kernels",
// vLLM issue 3289, the GEMV/GEMM mix).
#include "common.hpp"
#include "launch.hpp"
#include "one_token.hpp"

namespace wq {

// token rows staged in LDS: M <= TINY_MAX_ROWS rows of one K slice's 16-bit
// values, each padded by 16 bytes so the 16 B-operand columns hit distinct banks
constexpr int TINY_MAX_ROWS = 4;

template <int WBITS, bool BF16, int STAGE, int NT, int NW, int DEPTH>
__global__ __launch_bounds__(NW * 64) void gemm_tiny_kernel(GemmArgs g, const int32_t* __restrict__ perm) {
    constexpr int KCHUNK = WFmt<WBITS>::KCHUNK;
    constexpr int KSTEPS = KCHUNK / 32;
    static_assert(STAGE != STAGE_GATE_UP || NT % 2 == 0, "gate/up tiles come in pairs");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    __shared__ f32x4 red[NW][NT][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int unit = blockIdx.x;
    const int T = g.M * g.topk;
    const int BS = g.block_size;
    const int K = g.k_in;
    // K slice z of gridDim.z (DOWN only): chunks [cb, cb + C) of the C_all
    // chunks of a weight row tile; slice z writes fp32 slab z of the output
    const int C_all = K / KCHUNK;
    const int z = blockIdx.z;
    const int cb = (int)((long)z * C_all / gridDim.z);
    const int C = (int)((long)(z + 1) * C_all / gridDim.z) - cb;
    const int KL = C * KCHUNK;  // staged channels per row

    // block b of sorted_token_ids (grid.y covers the capacity's blocks; those
    // past the used ones exit).  Its real rows are a prefix of it: nv <= M
    // normally; a token's top-k naming an expert twice gives more, multiplied
    // in passes of RL rows
    const int b = blockIdx.y;
    if (b >= *g.ntpp / BS) return;
    const int e = g.expert_ids[b];
    const int p0 = b * BS;
    const int plim = p0 + BS;
    int nv_all = 0;
    while (nv_all < BS && g.sorted[p0 + nv_all] < T) ++nv_all;
    const int RL = min(g.M, 16);  // rows the LDS holds

    const size_t expert_bytes = (size_t)(g.n_out / TILE_ROWS) * C_all * CHUNK_BYTES;
    const uint8_t* wt[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
        wt[t] = g.w + (size_t)e * expert_bytes + ((size_t)(NT * unit + t) * C_all + cb) * CHUNK_BYTES + lane * 16;
    const uint16_t* se = g.s + (size_t)e * g.groups * g.n_out;  // group c of the slice: se + (cb + c) * n_out
    const bool grouped = (WBITS == 4) && g.groups > 1;
    const int rowq = 4 * (lane >> 4);  // first of this lane's 4 output rows in a tile
    const int xrow_b = 2 * KL + 16;
    uint8_t* scl = lds + (size_t)RL * xrow_b;  // group c's scales at scl + c * NT * 16 values

    // chunks wave + NW * i, i < nw; indices clamp to the wave's last chunk
    // (chunk C - 1 for a wave without chunks, whose loads are then never used)
    const int nw = wave < C ? (C - 1 - wave) / NW + 1 : 0;
    const int clast = wave < C ? wave + (nw - 1) * NW : C - 1;

    auto rows_pass = [&](const int r0, const int nv) {
        u32x4 wv[DEPTH][NT];
        auto wload = [&](int i, int slot) {
            const size_t off = (size_t)min(wave + NW * i, clast) * CHUNK_BYTES;
#pragma unroll
            for (int t = 0; t < NT; ++t) wv[slot][t] = ldg128_stream(wt[t] + off);
        };
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) wload(d, d);

        // stage channels [cb * KCHUNK, + KL) of rows p0 + r0 .. p0 + r0 + nv - 1
        // (and, once, the slice's scale slab)
        const int kp = KL / 8;  // 16-byte pieces per row
        for (int q = tid; q < nv * kp; q += NW * 64) {
            const int r = q / kp;
            const int pc = q - r * kp + cb * (KCHUNK / 8);  // piece of the full row
            const int p = p0 + r0 + r;
            u32x4 v;
            if (g.a_direct) {
                v = ldg128(g.a + (size_t)p * K + 8 * pc);
            } else {
                const uint16_t* xr = g.a + (size_t)(g.sorted[p] / g.topk) * K;
                if (perm) {
                    const int32_t* pe = perm + (size_t)e * K + 8 * pc;
                    const u32x4 i0 = ldg128(pe), i1 = ldg128(pe + 4);
                    v[0] = (uint32_t)xr[i0[0]] | ((uint32_t)xr[i0[1]] << 16);
                    v[1] = (uint32_t)xr[i0[2]] | ((uint32_t)xr[i0[3]] << 16);
                    v[2] = (uint32_t)xr[i1[0]] | ((uint32_t)xr[i1[1]] << 16);
                    v[3] = (uint32_t)xr[i1[2]] | ((uint32_t)xr[i1[3]] << 16);
                } else {
                    v = ldg128(xr + 8 * pc);
                }
            }
            *reinterpret_cast<u32x4*>(lds + (size_t)r * xrow_b + 16 * (pc - cb * (KCHUNK / 8))) = v;
        }
        if (grouped && r0 == 0) {
            constexpr int SP = NT * TILE_ROWS / 8;  // 16-byte pieces of one group's scales
            for (int q = tid; q < C * SP; q += NW * 64) {
                const int c = q / SP, pc = q - c * SP;
                *reinterpret_cast<u32x4*>(scl + 16 * q) =
                    ldg128(se + (size_t)(cb + c) * g.n_out + NT * unit * TILE_ROWS + 8 * pc);
            }
        }
        __syncthreads();

        const uint8_t* xl = lds + (size_t)min(lane & 15, nv - 1) * xrow_b + 16 * (lane >> 4);
        f32x4 acc[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        auto body = [&](int i, auto U) {
            constexpr int u = decltype(U)::value;
            const int c = min(wave + NW * i, clast);
            const uint8_t* xc = xl + (size_t)c * (2 * KCHUNK);
            u32x4 b[KSTEPS];
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) b[ks] = *reinterpret_cast<const u32x4*>(xc + 64 * ks);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                if constexpr (WBITS == 4) {
                    f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KSTEPS; ++ks)
                        part = mfma16x16x32<false>(dequant_w4_f16(wv[u][t][ks]), b[ks], part);
                    if (grouped) {
                        const u32x2 sv = *reinterpret_cast<const u32x2*>(
                            scl + 2 * ((size_t)c * NT * TILE_ROWS + t * TILE_ROWS + rowq));
                        acc[t][0] += part[0] * f16_to_f32((uint16_t)(sv[0] & 0xffffu));
                        acc[t][1] += part[1] * f16_to_f32((uint16_t)(sv[0] >> 16));
                        acc[t][2] += part[2] * f16_to_f32((uint16_t)(sv[1] & 0xffffu));
                        acc[t][3] += part[3] * f16_to_f32((uint16_t)(sv[1] >> 16));
                    } else {
                        acc[t] += part;
                    }
                } else {
#pragma unroll
                    for (int ks = 0; ks < KSTEPS; ++ks)
                        acc[t] = mfma16x16x32<BF16>(dequant_w8x8<BF16>(wv[u][t][2 * ks], wv[u][t][2 * ks + 1]),
                                                    b[ks], acc[t]);
                }
            }
            wload(i + DEPTH, u);
        };
        int i0 = 0;
        for (; i0 + DEPTH <= nw; i0 += DEPTH) static_for<0, DEPTH>([&](auto U) { body(i0 + decltype(U)::value, U); });
        static_for<0, DEPTH - 1>([&](auto U) {
            if (i0 + decltype(U)::value < nw) body(i0 + decltype(U)::value, U);
        });

#pragma unroll
        for (int t = 0; t < NT; ++t) red[wave][t][lane] = acc[t];
        __syncthreads();

        const int m = lane & 15;  // token row of this lane's outputs
        if (m < nv) {
            const int p = p0 + r0 + m;
            constexpr int ITEMS = STAGE == STAGE_GATE_UP ? NT / 2 : NT;
            for (int item = wave; item < ITEMS; item += NW) {
                if constexpr (STAGE == STAGE_GATE_UP) {
                    const int tg = 2 * item, tu = 2 * item + 1;
                    f32x4 gv = red[0][tg][lane], uv = red[0][tu][lane];
#pragma unroll
                    for (int w = 1; w < NW; ++w) {
                        gv += red[w][tg][lane];
                        uv += red[w][tu][lane];
                    }
                    const int N = g.n_out / 2;
                    const int hcol = ((NT / 2) * unit + item) * TILE_ROWS + rowq;
                    float h[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float gt = gv[i], up = uv[i];
                        if (!grouped) {
                            gt *= act_to_f32<BF16>(se[(NT * unit + tg) * TILE_ROWS + rowq + i]);
                            up *= act_to_f32<BF16>(se[(NT * unit + tu) * TILE_ROWS + rowq + i]);
                        }
                        h[i] = silu_f32(gt) * up;
                    }
                    u32x2 st;
                    st[0] = (uint32_t)f32_to_act<BF16>(h[0]) | ((uint32_t)f32_to_act<BF16>(h[1]) << 16);
                    st[1] = (uint32_t)f32_to_act<BF16>(h[2]) | ((uint32_t)f32_to_act<BF16>(h[3]) << 16);
                    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(g.out) + (size_t)p * N + hcol) = st;
                } else {
                    f32x4 o = red[0][item][lane];
#pragma unroll
                    for (int w = 1; w < NW; ++w) o += red[w][item][lane];
                    const int row = (NT * unit + item) * TILE_ROWS + rowq;
                    if (!grouped) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) o[i] *= act_to_f32<BF16>(se[row + i]);
                    }
                    const int pair = g.sorted[p];
                    if constexpr (STAGE == STAGE_DOWN) o *= g.topk_w[pair];
                    float* y = static_cast<float*>(g.out) + (size_t)z * T * g.n_out;
                    *reinterpret_cast<f32x4*>(y + (size_t)pair * g.n_out + row) = o;
                }
            }
        }
    };
    for (int r0 = 0; r0 < nv_all; r0 += RL) {
        if (r0 > 0) __syncthreads();  // the previous pass's epilogue has read the reduction buffer
        rows_pass(r0, min(RL, nv_all - r0));
    }

    if constexpr (STAGE == STAGE_GATE_UP) {
        // H rows of the block's pad entries are zero
        const int N = g.n_out / 2;
        constexpr int COLS = (NT / 2) * TILE_ROWS;
        const int pz = p0 + nv_all;
        for (int k = tid; k < (plim - pz) * COLS; k += NW * 64) {
            const int p = pz + k / COLS;
            static_cast<uint16_t*>(g.out)[(size_t)p * N + (NT / 2) * unit * TILE_ROWS + (k % COLS)] = 0;
        }
    }
}

// LDS of one workgroup: the staged rows of one K slice, its scale slab, the
// reduction buffer
static size_t tiny_lds(int wbits, int M, int k_in, int groups, int nt, int nw, int ks) {
    const size_t kl = (size_t)k_in / ks;
    size_t b = (size_t)M * (2 * kl + 16);
    if (wbits == 4 && groups > 1) b += kl / 128 * nt * TILE_ROWS * 2;
    return b + (size_t)nw * nt * 64 * 16;
}

template <int WBITS, bool BF16, int STAGE, int NT, int NW, int DEPTH>
static int launch_tiny_cfg(const GemmArgs& g, const int32_t* perm, int ks, hipStream_t s) {
    auto kern = gemm_tiny_kernel<WBITS, BF16, STAGE, NT, NW, DEPTH>;
    const size_t red = (size_t)NW * NT * 64 * 16;
    const size_t dyn = tiny_lds(WBITS, g.M, g.k_in, g.groups, NT, NW, ks) - red;
    if (dyn + red > 65536)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)dyn);
    hipLaunchKernelGGL(kern, dim3(g.n_out / (TILE_ROWS * NT), g.cap / g.block_size, ks), dim3(NW * 64), dyn, s, g,
                       perm);
    return ks;
}

// K slices of a DOWN launch (its output is the fp32 slabs the combine adds):
// the most of 1, 2, 4 that divides the chunks, keeps >= 16 chunks per slice
// and fits the caller's slabs
static int tiny_down_split(int wbits, int k_in, int max_ks) {
    const int c = k_in / (wbits == 4 ? WFmt<4>::KCHUNK : WFmt<8>::KCHUNK);
    int ks = 1;
    while (ks < 4 && ks * 2 <= max_ks && c % (ks * 2) == 0 && c / (ks * 2) >= 16) ks *= 2;
    return ks;
}

int tiny_down_slabs(int M, int k_in) {
    return (M >= 1 && M <= TINY_MAX_ROWS) ? tiny_down_split(8, k_in, 4) : 1;  // 8-bit chunks: the most slices
}

// One shape, measured on MI355X with the last-level cache flushed before every
// launch: 2 weight tiles (one gate/up pair), 4 waves, 3 chunks in flight; the
// DOWN stage (Mixtral shape, K = 14336) in 4 K slices, which quadruples the
// workgroups of a grid of only 2 x 128 (M = 1: int8 34.4 -> 24.5 us, int4
// 24.2 -> 19.1 us; M = 4: int8 71.7 -> 67.1 us).
template <int WBITS, bool BF16, int STAGE>
static int launch_tiny_s(const GemmArgs& g, const int32_t* perm, int max_ks, hipStream_t s) {
    const int ks = STAGE == STAGE_DOWN ? tiny_down_split(WBITS, g.k_in, max_ks) : 1;
    if constexpr (STAGE != STAGE_GATE_UP) {
        if (g.n_out % (TILE_ROWS * 2) != 0) return launch_tiny_cfg<WBITS, BF16, STAGE, 1, 4, 3>(g, perm, ks, s);
    }
    return launch_tiny_cfg<WBITS, BF16, STAGE, 2, 4, 3>(g, perm, ks, s);
}

// Where it is used: DOWN with a long reduction (>= 64 chunks per tile) up to
// 4 tokens, where it beats the small-batch kernel; the RAW stage of int4
// weights for one token (staging through the act-order permutation in place
// of the gather kernel).  GATE_UP of one token now runs faster on the
// small-batch kernel after the gather (Mixtral act-order int4 layer 68.2 ->
// 67.0 us, equal without act-order).  Many-expert layers with short rows
// (K = 1536) and int8 GATE_UP gain nothing.
bool tiny_supported(int wbits, int stage, int M, int k_in, int groups, int max_ks) {
    if (M < 1 || M > TINY_MAX_ROWS) return false;
    const int c = k_in / (wbits == 4 ? WFmt<4>::KCHUNK : WFmt<8>::KCHUNK);
    int ks = 1;
    if (stage == STAGE_DOWN) {
        if (c < 64) return false;
        ks = tiny_down_split(wbits, k_in, max_ks);
    } else if (stage != STAGE_RAW || wbits != 4 || M != 1) {
        return false;
    }
    return tiny_lds(wbits, M, k_in, groups, 2, 4, ks) <= 96 * 1024;
}

int launch_gemm_tiny(int wbits, bool bf16, int stage, const GemmArgs& g, const int32_t* perm, int max_ks,
                     hipStream_t s) {
    auto by_stage = [&](auto W, auto B) {
        constexpr int WB = decltype(W)::value;
        constexpr bool BF = decltype(B)::value;
        if (stage == STAGE_GATE_UP) return launch_tiny_s<WB, BF, STAGE_GATE_UP>(g, perm, max_ks, s);
        if (stage == STAGE_DOWN) return launch_tiny_s<WB, BF, STAGE_DOWN>(g, perm, max_ks, s);
        return launch_tiny_s<WB, BF, STAGE_RAW>(g, perm, max_ks, s);
    };
    if (wbits == 4) return by_stage(std::integral_constant<int, 4>{}, std::false_type{});
    if (bf16) return by_stage(std::integral_constant<int, 8>{}, std::true_type{});
    return by_stage(std::integral_constant<int, 8>{}, std::false_type{});
}


// ---------------------------------------------------------------------------
// DOWN of one token with the top-k weighted sum folded in.  Slot b is block b
// of the sorted order (at most top-k blocks are used): the weights of its
// expert start streaming at once, while one wave reads which pairs sit in
// which block (one_token.hpp); the real H rows are then staged in LDS, and one
// workgroup per 16 output columns streams the 16-row weight tile of every
// used slot, NW waves splitting the 1 KiB chunks (wave w takes chunks w, w +
// NW, ...), DEPTH chunks per slot in flight.  B column c of slot b carries the
// block's c-th real row (its last one for the other columns), so a pair's
// product is one column of its slot's result.  The waves' partial sums of the
// pairs' columns meet in LDS and are added in wave order, scaled per column
// (int8, or int4 with one scale per column), multiplied by the pair's routed
// weight and summed over the pairs in slot order -- the output row in the
// activation type, with no per-pair fp32 rows and no combine launch.  A pair
// missing from the sorted order, or one whose block names no valid expert,
// adds nothing.
// ---------------------------------------------------------------------------
template <int WBITS, bool BF16, int TK, int NW, int DEPTH>
__global__ __launch_bounds__(NW * 64) void tiny_down_combine_kernel(GemmArgs g, uint16_t* __restrict__ out) {
    constexpr int KCHUNK = WFmt<WBITS>::KCHUNK;
    constexpr int KSTEPS = KCHUNK / 32;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    __shared__ OneTokenPlan<TK> pl;
    __shared__ f32x4 red[NW][TK][TK][4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int tile = blockIdx.x;
    const int K = g.k_in;
    const int C = K / KCHUNK;

    int eb[TK];
    one_token_experts<TK>(g.expert_ids, g.cap, g.block_size, g.E, eb);
    const size_t expert_bytes = (size_t)(g.n_out / TILE_ROWS) * C * CHUNK_BYTES;
    const uint8_t* wt[TK];
    const uint16_t* se[TK];
#pragma unroll
    for (int b = 0; b < TK; ++b) {
        wt[b] = g.w + (size_t)eb[b] * expert_bytes + (size_t)tile * C * CHUNK_BYTES + lane * 16;
        se[b] = g.s + (size_t)eb[b] * g.groups * g.n_out;
    }
    const bool grouped = (WBITS == 4) && g.groups > 1;
    const int rowq = 4 * (lane >> 4);

    // chunks wave + NW * i, i < nw; indices clamp to the wave's last chunk
    const int nw = wave < C ? (C - 1 - wave) / NW + 1 : 0;
    const int clast = wave < C ? wave + (nw - 1) * NW : C - 1;
    u32x4 wv[DEPTH][TK];
    u32x2 sv[DEPTH][TK];  // int4 group-128: the chunk's scales of this lane's 4 rows, loaded with it
    auto wload = [&](int i, int slot) {
        const int c = min(wave + NW * i, clast);
#pragma unroll
        for (int b = 0; b < TK; ++b) wv[slot][b] = ldg128_stream(wt[b] + (size_t)c * CHUNK_BYTES);
        if constexpr (WBITS == 4) {
            const size_t gc = grouped ? (size_t)c : 0;  // per-column scales: a harmless reread of group 0
#pragma unroll
            for (int b = 0; b < TK; ++b)
                sv[slot][b] = *reinterpret_cast<const u32x2*>(se[b] + gc * g.n_out + tile * TILE_ROWS + rowq);
        }
    };
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) wload(d, d);

    if (wave == 0) one_token_plan<TK>(pl, g.sorted, g.expert_ids, g.ntpp, g.cap, g.block_size, g.E, lane);
    __syncthreads();
    // every slot's weights stream (an unused one, left when a top-k names an
    // expert twice, reads a clamped expert's and is not multiplied)
    bool used[TK];
#pragma unroll
    for (int b = 0; b < TK; ++b) used[b] = __builtin_amdgcn_readfirstlane(pl.cnt[b]) > 0;

    // stage the real H rows (rows past them read as zeros)
    const int xrow_b = 2 * K + 16;
    const int kp = K / 8;  // 16-byte pieces per row
    for (int q = tid; q < TK * kp; q += NW * 64) {
        const int r = q / kp, pc = q - r * kp;
        const int p = pl.pos[r];
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (p >= 0) v = ldg128(g.a + (size_t)p * K + 8 * pc);
        *reinterpret_cast<u32x4*>(lds + (size_t)r * xrow_b + 16 * pc) = v;
    }
    const uint8_t* xr[TK];  // this lane's B row of each slot
#pragma unroll
    for (int b = 0; b < TK; ++b)
        xr[b] = lds + (size_t)(pl.row0[b] + min(lane & 15, max(pl.cnt[b], 1) - 1)) * xrow_b + 16 * (lane >> 4);
    __syncthreads();

    f32x4 acc[TK];
#pragma unroll
    for (int b = 0; b < TK; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto body = [&](int i, auto U) {
        constexpr int u = decltype(U)::value;
        const int c = min(wave + NW * i, clast);
#pragma unroll
        for (int b = 0; b < TK; ++b) {
            if (!used[b]) continue;
            const uint8_t* xc = xr[b] + (size_t)c * (2 * KCHUNK);
            u32x4 bv[KSTEPS];
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) bv[ks] = *reinterpret_cast<const u32x4*>(xc + 64 * ks);
            if constexpr (WBITS == 4) {
                f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks)
                    part = mfma16x16x32<false>(dequant_w4_f16(wv[u][b][ks]), bv[ks], part);
                if (grouped) {
                    acc[b][0] += part[0] * f16_to_f32((uint16_t)(sv[u][b][0] & 0xffffu));
                    acc[b][1] += part[1] * f16_to_f32((uint16_t)(sv[u][b][0] >> 16));
                    acc[b][2] += part[2] * f16_to_f32((uint16_t)(sv[u][b][1] & 0xffffu));
                    acc[b][3] += part[3] * f16_to_f32((uint16_t)(sv[u][b][1] >> 16));
                } else {
                    acc[b] += part;
                }
            } else {
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks)
                    acc[b] = mfma16x16x32<BF16>(dequant_w8x8<BF16>(wv[u][b][2 * ks], wv[u][b][2 * ks + 1]), bv[ks],
                                                acc[b]);
            }
        }
        wload(i + DEPTH, u);
    };
    int i0 = 0;
    for (; i0 + DEPTH <= nw; i0 += DEPTH) static_for<0, DEPTH>([&](auto U) { body(i0 + decltype(U)::value, U); });
    static_for<0, DEPTH - 1>([&](auto U) {
        if (i0 + decltype(U)::value < nw) body(i0 + decltype(U)::value, U);
    });

    if ((lane & 15) < TK) {
#pragma unroll
        for (int b = 0; b < TK; ++b) red[wave][b][lane & 15][lane >> 4] = acc[b];
    }
    __syncthreads();
    if (tid < 4) {
        const int row = tile * TILE_ROWS + 4 * tid;
        f32x4 res = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < TK; ++j) {
            const int b = pl.slot[j];
            if (b < 0) continue;
            const int c = pl.col[j];
            f32x4 o = red[0][b][c][tid];
#pragma unroll
            for (int w = 1; w < NW; ++w) o += red[w][b][c][tid];
            if (!grouped) {
                const uint16_t* sb = g.s + (size_t)min(max(g.expert_ids[b], 0), g.E - 1) * g.groups * g.n_out;
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] *= act_to_f32<BF16>(sb[row + i]);
            }
            res += o * g.topk_w[j];
        }
        u32x2 st;
        st[0] = (uint32_t)f32_to_act<BF16>(res[0]) | ((uint32_t)f32_to_act<BF16>(res[1]) << 16);
        st[1] = (uint32_t)f32_to_act<BF16>(res[2]) | ((uint32_t)f32_to_act<BF16>(res[3]) << 16);
        *reinterpret_cast<u32x2*>(out + row) = st;
    }
}

static size_t down_combine_lds(int topk, int k_in) { return (size_t)topk * (2 * (size_t)k_in + 16); }

// one token, top-k up to 4, a long reduction (>= 64 chunks per tile), whole
// H rows in LDS
bool tiny_down_combine_supported(int wbits, int M, int topk, int n_out, int k_in) {
    const int c = k_in / (wbits == 4 ? WFmt<4>::KCHUNK : WFmt<8>::KCHUNK);
    return M == 1 && topk >= 1 && topk <= 4 && c >= 64 && n_out % TILE_ROWS == 0 &&
           down_combine_lds(topk, k_in) <= 128 * 1024;
}

template <int WBITS, bool BF16, int TK>
static void launch_down_combine_tk(const GemmArgs& g, uint16_t* out, hipStream_t s) {
    constexpr int NW = 16, DEPTH = (WBITS == 4 && TK == 4) ? 2 : 3;  // int4 top-4: 3 deep exceeds 128 VGPRs
    auto kern = tiny_down_combine_kernel<WBITS, BF16, TK, NW, DEPTH>;
    const size_t dyn = down_combine_lds(TK, g.k_in);
    if (dyn > 64 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)dyn);
    hipLaunchKernelGGL(kern, dim3(g.n_out / TILE_ROWS), dim3(NW * 64), dyn, s, g, out);
}

template <int WBITS, bool BF16>
static void launch_down_combine_w(const GemmArgs& g, uint16_t* out, hipStream_t s) {
    switch (g.topk) {
        case 1: launch_down_combine_tk<WBITS, BF16, 1>(g, out, s); break;
        case 2: launch_down_combine_tk<WBITS, BF16, 2>(g, out, s); break;
        case 3: launch_down_combine_tk<WBITS, BF16, 3>(g, out, s); break;
        default: launch_down_combine_tk<WBITS, BF16, 4>(g, out, s); break;
    }
}

void launch_tiny_down_combine(int wbits, bool bf16, const GemmArgs& g, uint16_t* out, hipStream_t s) {
    if (wbits == 4) launch_down_combine_w<4, false>(g, out, s);
    else if (bf16) launch_down_combine_w<8, true>(g, out, s);
    else launch_down_combine_w<8, false>(g, out, s);
}

}  // namespace wq

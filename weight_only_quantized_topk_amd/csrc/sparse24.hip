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
// through ABID 0/1.
//
// Kernels:
//  - small and medium batches (M <= 128): one workgroup per 128 (16 tokens)
//    or 256 output rows (32 or 64 tokens), one 16-row tile per wave; all
//    waves walk the same 256-channel chunks, whose token tile is staged once
//    in LDS and shared; each wave keeps the weights of 4 chunks in flight in
//    registers;
//  - large batches: one workgroup per 256 output rows and 64 tokens; the token
//    tile of each chunk is staged once in LDS and shared by the 4 waves, each
//    of which multiplies its own 64 weight rows, read straight from the packed
//    layout into registers one chunk ahead -- for 4-bit codes the pipelined
//    form (sparse24_pipe_kernel: half-chunk LDS double buffer, one barrier per
//    half chunk, conversions and operand reads overlapped with the MFMAs),
//    for 8-bit codes the plain one (sparse24_tile_kernel).
// Token rows are 512-byte LDS rows of 16-byte pieces stored at
// piece ^ (row & 15), so the B-operand reads of 16 rows hit distinct banks.
// Weights are scaled in fp16 (q * s rounded once) before the multiply.
#include "common.hpp"
#include "launch.hpp"

namespace wq {

constexpr int SP_WAVES = 4;
constexpr int SP_THREADS = 64 * SP_WAVES;
constexpr int SP_KCHUNK = 256;  // dense input channels per packed piece
constexpr int SPT_ROWB_S = SP_KCHUNK * 2;  // LDS bytes of one token row of a chunk

// The kept values of one lane for one 256-channel chunk: 8 per 64-channel
// step s, as 4-bit offset codes (one dword per step, 16 bytes) or 8-bit two's
// complement codes in natural order (two dwords per step, 32 bytes).  A chunk
// of a 16-row tile holds 64 lanes' values, 1 or 2 KiB.
template <int VBITS>
struct SpVals {
    u32x4 v[VBITS / 4];
};
template <int VBITS>
constexpr int sp_lane_bytes() { return 4 * VBITS; }
template <int VBITS>
constexpr int sp_chunk_bytes() { return 64 * sp_lane_bytes<VBITS>(); }

template <int VBITS>
__device__ __forceinline__ SpVals<VBITS> sp_load(const uint8_t* p) {
    SpVals<VBITS> r;
#pragma unroll
    for (int h = 0; h < VBITS / 4; ++h) r.v[h] = ldg128_stream(p + 16 * h);
    return r;
}

// the 8 fp16 A-operand values of step s, each q * scale rounded once to fp16
template <int VBITS, int S>
__device__ __forceinline__ u32x4 sp_dequant(const SpVals<VBITS>& w, uint32_t sv) {
    const f16x2 s2 = __builtin_bit_cast(f16x2, sv | (sv << 16));
    if constexpr (VBITS == 4) {
        return dequant_w4_f16_scaled(w.v[0][S], s2);
    } else {
        const u32x4 d = dequant_w8x8<false>(w.v[S >> 1][2 * (S & 1)], w.v[S >> 1][2 * (S & 1) + 1]);
        const uint32_t d0 = d[0], d1 = d[1], d2 = d[2], d3 = d[3];
        return u32x4{f16x2_mul(d0, s2), f16x2_mul(d1, s2), f16x2_mul(d2, s2), f16x2_mul(d3, s2)};
    }
}

// ------------------------------------------------- streaming (small batches)
// One workgroup: NWV waves, wave w multiplies 16-row tile NWV*blockIdx.x + w by
// the 16*R tokens of blockIdx.y; all waves walk the same 256-channel chunks.
// The token tile of a chunk is staged in LDS (two slots), its global loads
// issued XP chunks ahead; each wave keeps the weights of PF chunks of its tile
// in flight in registers.  Chunk slots are static: the chunk loop is unrolled
// by PF.
template <int VBITS, int R, int PF, int NWV>
__global__ __launch_bounds__(NWV * 64) void sparse24_stream_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                                     int N, const uint8_t* __restrict__ vals,
                                                                     const uint8_t* __restrict__ meta,
                                                                     const uint16_t* __restrict__ scales,
                                                                     int sstride, uint16_t* __restrict__ y) {
    constexpr int XP = R == 1 ? 4 : 2;              // token chunks in flight
    constexpr int ROWS = 16 * R;                    // tokens per workgroup
    constexpr int NT = NWV * 64;
    constexpr int XPIECES = ROWS * 32 / NT;         // 16-byte token pieces per thread per chunk
    constexpr int SPS_PF = PF;
    __shared__ __attribute__((aligned(16))) uint8_t xs[2][ROWS * SPT_ROWB_S];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ntiles = N / 16;
    const int t_raw = NWV * blockIdx.x + wave;
    const bool tvalid = t_raw < ntiles;
    const int t = tvalid ? t_raw : ntiles - 1;
    const int m0 = blockIdx.y * ROWS;
    const int C = K / SP_KCHUNK;
    const int nrow = lane & 15;

    const uint8_t* vt = vals + (size_t)t * C * sp_chunk_bytes<VBITS>() + lane * sp_lane_bytes<VBITS>();
    const uint8_t* mt = meta + (size_t)t * C * 512 + lane * 8;
    const uint16_t* sn = scales + 16 * t + nrow;
    // the two scale halves stay apart until used, so no wait follows their loads
    SpVals<VBITS> wv[SPS_PF];
    u32x2 wm[SPS_PF];
    uint32_t ws0[SPS_PF], ws1[SPS_PF];
    auto wload = [&](int c, int slot) {
        wv[slot] = sp_load<VBITS>(vt + (size_t)c * sp_chunk_bytes<VBITS>());
        wm[slot] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(mt + (size_t)c * 512));
        ws0[slot] = sn[(size_t)(2 * c) * sstride];
        ws1[slot] = sn[(size_t)(2 * c + 1) * sstride];
    };
    const uint16_t* xcol = x + (tid & 31) * 8;
    const int xrow0 = m0 + (tid >> 5);
    u32x4 xv[XP][XPIECES];
    auto xload = [&](int c, int slot) {
#pragma unroll
        for (int i = 0; i < XPIECES; ++i)
            xv[slot][i] = ldg128(xcol + (size_t)min(xrow0 + (NT / 32) * i, M - 1) * K + c * SP_KCHUNK);
    };
    auto xstore = [&](int slot, int buf) {
#pragma unroll
        for (int i = 0; i < XPIECES; ++i) {
            const int id = tid + NT * i;
            const int row = id >> 5, piece = id & 31;
            *reinterpret_cast<u32x4*>(&xs[buf][row * SPT_ROWB_S + ((piece ^ (row & 15)) << 4)]) = xv[slot][i];
        }
    };
    f32x4 acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int slot, int buf) {
        const uint8_t* xb = xs[buf];
        static_for<0, 4>([&](auto S_) {
            constexpr int s = decltype(S_)::value;
            const uint32_t sv = (s < 2) ? ws0[slot] : ws1[slot];
            const u32x4 a = sp_dequant<VBITS, s>(wv[slot], sv);
            const int idx = (int)wm[slot][s >> 1];
            const int plo = 8 * s + (lane >> 4), phi = plo + 4;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int row = 16 * r + nrow;
                const u32x4 lo = *reinterpret_cast<const u32x4*>(xb + row * SPT_ROWB_S + ((plo ^ nrow) << 4));
                const u32x4 hi = *reinterpret_cast<const u32x4*>(xb + row * SPT_ROWB_S + ((phi ^ nrow) << 4));
                const u32x8 b = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                acc[r] = smfmac16x16x64<s & 1>(a, b, idx, acc[r]);
            }
        });
    };

    // every load is unconditional (chunk indices clamped to the last chunk, which
    // the tail then reads again from cache): loads under a branch would make the
    // compiler wait for all of them before the LDS stores
    auto body = [&](int c, auto U) {
        constexpr int u = decltype(U)::value;
        xstore(u % XP, u & 1);
        xload(min(c + XP, C - 1), u % XP);
        __syncthreads();
        compute(u, u & 1);
        wload(min(c + SPS_PF, C - 1), u);
    };
#pragma unroll
    for (int p = 0; p < SPS_PF; ++p) wload(min(p, C - 1), p);
#pragma unroll
    for (int q = 0; q < XP; ++q) xload(min(q, C - 1), q);
    int c0 = 0;
    for (; c0 + SPS_PF <= C; c0 += SPS_PF)
        static_for<0, SPS_PF>([&](auto U) { body(c0 + decltype(U)::value, U); });
    // tail of fewer than PF chunks (the guard is uniform over the workgroup)
    static_for<0, SPS_PF - 1>([&](auto U) {
        if (c0 + decltype(U)::value < C) body(c0 + decltype(U)::value, U);
    });

    if (tvalid) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int m = m0 + 16 * r + nrow;
            if (m < M) {
                u32x2 stv;
                stv[0] = (uint32_t)f32_to_f16(acc[r][0]) | ((uint32_t)f32_to_f16(acc[r][1]) << 16);
                stv[1] = (uint32_t)f32_to_f16(acc[r][2]) | ((uint32_t)f32_to_f16(acc[r][3]) << 16);
                *reinterpret_cast<u32x2*>(y + (size_t)m * N + 16 * t + 4 * (lane >> 4)) = stv;
            }
        }
    }
}

// ------------------------------------------------- decode (few tokens)
// One workgroup per TPW 16-row weight tiles, NW waves per tile splitting its
// 256-channel chunks (wave w takes chunks w, w + NW, ...), each keeping DEPTH
// chunks of its weights in flight in registers.  The token rows (M * K fp16, at most
// 64 KiB) are staged in LDS once, before the chunk loop, rows padded by 16
// bytes so the 16 column lanes of the B operand hit distinct banks; columns
// at or beyond M read row M - 1.  So the loop's only global loads are the
// weight stream: a token load among them would make every wait for it also
// wait for the weight loads issued before it (the wait counter is in order),
// shortening the prefetch.  The NW partial sums are added in LDS in wave
// order.  Loads sit outside branches except in the guarded tail of fewer than
// DEPTH chunks.
template <int VBITS, int NW, int DEPTH, int TPW>
__global__ __launch_bounds__(NW * TPW * 64) void sparse24_decode_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                                    int N, const uint8_t* __restrict__ vals,
                                                                    const uint8_t* __restrict__ meta,
                                                                    const uint16_t* __restrict__ scales,
                                                                    int sstride, uint16_t* __restrict__ y) {
    extern __shared__ __attribute__((aligned(16))) uint8_t xs_dyn[];
    __shared__ f32x4 red[TPW][NW][64];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = (tid >> 6) % NW;  // K slice of this wave
    const int tw = (tid >> 6) / NW;    // tile of this wave within the workgroup
    const int t = min(TPW * (int)blockIdx.x + tw, N / 16 - 1);
    const bool tvalid = TPW * (int)blockIdx.x + tw < N / 16;
    const int C = K / SP_KCHUNK;
    const int nrow = lane & 15;
    const int xrow_b = 2 * K + 16;  // LDS bytes per token row

    // weights first, so their loads are in flight during the token staging
    const int nw = wave < C ? (C - 1 - wave) / NW + 1 : 0;
    const int clast = wave < C ? wave + (nw - 1) * NW : C - 1;  // chunk C - 1 for a wave without chunks
    const uint8_t* vt = vals + (size_t)t * C * sp_chunk_bytes<VBITS>() + lane * sp_lane_bytes<VBITS>();
    const uint8_t* mt = meta + (size_t)t * C * 512 + lane * 8;
    const uint16_t* sn = scales + 16 * t + nrow;
    SpVals<VBITS> wv[DEPTH];
    u32x2 wm[DEPTH];
    uint32_t ws0[DEPTH], ws1[DEPTH];
    auto wload = [&](int i, int slot) {
        const int c = min(wave + NW * i, clast);
        wv[slot] = sp_load<VBITS>(vt + (size_t)c * sp_chunk_bytes<VBITS>());
        wm[slot] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(mt + (size_t)c * 512));
        ws0[slot] = sn[(size_t)(2 * c) * sstride];
        ws1[slot] = sn[(size_t)(2 * c + 1) * sstride];
    };
#pragma unroll
    for (int p = 0; p < DEPTH; ++p) wload(p, p);

    const int pieces = M * (K / 8);  // 16-byte token pieces
    for (int q = tid; q < pieces; q += NW * TPW * 64) {
        const int row = q / (K / 8), pc = q - row * (K / 8);
        *reinterpret_cast<u32x4*>(xs_dyn + row * xrow_b + 16 * pc) = ldg128(x + (size_t)row * K + 8 * pc);
    }
    __syncthreads();

    const uint8_t* xl = xs_dyn + min(nrow, M - 1) * xrow_b + 16 * (lane >> 4);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    auto body = [&](int i, auto U) {
        constexpr int u = decltype(U)::value;
        const uint8_t* xc = xl + (size_t)min(wave + NW * i, clast) * (2 * SP_KCHUNK);
        static_for<0, 4>([&](auto S_) {
            constexpr int s = decltype(S_)::value;
            const uint32_t sv = (s < 2) ? ws0[u] : ws1[u];
            const u32x4 a = sp_dequant<VBITS, s>(wv[u], sv);
            const int idx = (int)wm[u][s >> 1];
            const u32x4 lo = *reinterpret_cast<const u32x4*>(xc + 128 * s);
            const u32x4 hi = *reinterpret_cast<const u32x4*>(xc + 128 * s + 64);
            const u32x8 b = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            acc = smfmac16x16x64<s & 1>(a, b, idx, acc);
        });
        wload(i + DEPTH, u);
    };
    int i0 = 0;
    for (; i0 + DEPTH <= nw; i0 += DEPTH) static_for<0, DEPTH>([&](auto U) { body(i0 + decltype(U)::value, U); });
    static_for<0, DEPTH - 1>([&](auto U) {
        if (i0 + decltype(U)::value < nw) body(i0 + decltype(U)::value, U);
    });

    red[tw][wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int w = 1; w < NW; ++w) acc += red[tw][w][lane];
        if (tvalid && nrow < M) {
            u32x2 stv;
            stv[0] = (uint32_t)f32_to_f16(acc[0]) | ((uint32_t)f32_to_f16(acc[1]) << 16);
            stv[1] = (uint32_t)f32_to_f16(acc[2]) | ((uint32_t)f32_to_f16(acc[3]) << 16);
            *reinterpret_cast<u32x2*>(y + (size_t)nrow * N + 16 * t + 4 * (lane >> 4)) = stv;
        }
    }
}

// LDS bytes of the decode kernel's token rows, and the most it takes
static size_t sparse24_decode_lds(int M, int K) { return (size_t)M * (2 * (size_t)K + 16); }
constexpr size_t SP_DECODE_LDS_MAX = 96 * 1024;

// ------------------------------------------------------------ large batches
constexpr int SPT_BN = 256;  // weight rows per workgroup (4 waves x 4 tiles of 16)
constexpr int SPT_BM = 64;   // tokens per workgroup (4 B tiles of 16)
constexpr int SPT_ROWB = SP_KCHUNK * 2;
constexpr int SPT_XPIECES = SPT_BM * (SPT_ROWB / 16) / SP_THREADS;  // 16-byte token pieces per thread per chunk

__device__ __forceinline__ int spt_off(int row, int piece) { return row * SPT_ROWB + ((piece ^ (row & 15)) << 4); }

template <int VBITS, int OCC>
__global__ __launch_bounds__(SP_THREADS, OCC) void sparse24_tile_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                                      int N, const uint8_t* __restrict__ vals,
                                                                      const uint8_t* __restrict__ meta,
                                                                      const uint16_t* __restrict__ scales,
                                                                      int sstride, uint16_t* __restrict__ y) {
    __shared__ __attribute__((aligned(16))) uint8_t xs[SPT_BM * SPT_ROWB];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int m0 = blockIdx.y * SPT_BM;
    const int C = K / SP_KCHUNK;
    const int t0 = blockIdx.x * (SPT_BN / 16) + 4 * wave;  // first 16-row tile of this wave
    const int nrow = lane & 15;

    // token pieces: row id/32 = tid/32 + 8i, piece id%32 = tid%32 (rows past M read row M-1; their
    // outputs are not stored)
    const uint16_t* xcol = x + (tid & 31) * 8;
    const int xrow0 = m0 + (tid >> 5);
    u32x4 xv[SPT_XPIECES];
    SpVals<VBITS> v[4], vn[4];
    u32x2 md[4], mdn[4];
    uint32_t sc0[4], sc1[4], scn0[4], scn1[4];  // scales of groups 2c and 2c+1 of this lane's row
    auto gload = [&](int c) {
#pragma unroll
        for (int i = 0; i < SPT_XPIECES; ++i)
            xv[i] = ldg128(xcol + (size_t)min(xrow0 + 8 * i, M - 1) * K + c * SP_KCHUNK);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const size_t pc = ((size_t)(t0 + i) * C + c) * 64 + lane;
            vn[i] = sp_load<VBITS>(vals + pc * sp_lane_bytes<VBITS>());
            mdn[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(meta + pc * 8));
            const int n = 16 * (t0 + i) + nrow;
            scn0[i] = scales[(size_t)(2 * c) * sstride + n];
            scn1[i] = scales[(size_t)(2 * c + 1) * sstride + n];
        }
    };
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    int boff[4];  // LDS row offsets of this lane's B columns (token tiles j)
#pragma unroll
    for (int j = 0; j < 4; ++j) boff[j] = (16 * j + nrow) * SPT_ROWB;
    const int bsw = nrow;  // row & 15 of every B row this lane reads

    auto step = [&](auto ST) {
        constexpr int s = decltype(ST)::value;  // 64-channel step within the chunk
        u32x4 a[4];
        int idx[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t sv = (s < 2) ? sc0[i] : sc1[i];
            a[i] = sp_dequant<VBITS, s>(v[i], sv);
            idx[i] = (int)md[i][s >> 1];
        }
        const int plo = 8 * s + (lane >> 4), phi = plo + 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u32x4 lo = *reinterpret_cast<const u32x4*>(xs + boff[j] + ((plo ^ bsw) << 4));
            const u32x4 hi = *reinterpret_cast<const u32x4*>(xs + boff[j] + ((phi ^ bsw) << 4));
            const u32x8 b = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i][j] = smfmac16x16x64<s & 1>(a[i], b, idx[i], acc[i][j]);
        }
    };

    gload(0);
    for (int c = 0; c < C; ++c) {
#pragma unroll
        for (int i = 0; i < SPT_XPIECES; ++i) {
            const int id = tid + SP_THREADS * i;
            *reinterpret_cast<u32x4*>(xs + spt_off(id >> 5, id & 31)) = xv[i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = vn[i];
            md[i] = mdn[i];
            sc0[i] = scn0[i];
            sc1[i] = scn1[i];
        }
        __syncthreads();
        gload(min(c + 1, C - 1));  // the last chunk is loaded twice, keeping the loop branch-free
        step(std::integral_constant<int, 0>{});
        step(std::integral_constant<int, 1>{});
        step(std::integral_constant<int, 2>{});
        step(std::integral_constant<int, 3>{});
        __syncthreads();
    }

    // D[row 4*(lane/16) + r][col lane%16]: rows are weight rows, columns tokens
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int m = m0 + 16 * j + nrow;
        if (m < M) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                u32x2 stv;
                stv[0] = (uint32_t)f32_to_f16(acc[i][j][0]) | ((uint32_t)f32_to_f16(acc[i][j][1]) << 16);
                stv[1] = (uint32_t)f32_to_f16(acc[i][j][2]) | ((uint32_t)f32_to_f16(acc[i][j][3]) << 16);
                *reinterpret_cast<u32x2*>(y + (size_t)m * N + 16 * (t0 + i) + 4 * (lane >> 4)) = stv;
            }
        }
    }
}

// ------------------------------------------------ large batches, pipelined
// One workgroup of NW waves: NW * RT 16-row weight tiles x 16 * TJ tokens;
// wave w owns RT weight tiles and all the token tiles.  The K loop runs in
// half chunks of 128 dense channels (two smfmac steps):
//  - the token rows of a half chunk go to one of two LDS buffers (256-byte
//    rows of 16-byte pieces at piece ^ (row & 15)) while the other is
//    multiplied: one barrier per half chunk;
//  - a wave's weights (kept codes, index metadata, the two group scales of
//    the chunk) come straight from the packed layout into registers, one
//    chunk ahead (two register slots), and the A operands of the next step
//    are dequantised between the MFMAs of the current one;
//  - the B operands of token tile j + 1 are read from LDS before the MFMAs of
//    tile j are issued.
// Token tiles wholly past M skip their MFMAs (one uniform branch per tile);
// rows past M inside a tile read row M - 1 and are not stored.
constexpr int SPP_HROWB = 256;  // LDS bytes of one token row per half chunk
#ifndef SPP_BA
#define SPP_BA 2  // token tiles of B operands read ahead
#endif

template <int VBITS, int NW, int RT, int TJ, int OCC>
__global__ __launch_bounds__(NW * 64, OCC) void sparse24_pipe_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                                     int N, const uint8_t* __restrict__ vals,
                                                                     const uint8_t* __restrict__ meta,
                                                                     const uint16_t* __restrict__ scales,
                                                                     int sstride, uint16_t* __restrict__ y) {
    constexpr int NT = NW * 64;
    constexpr int BM = 16 * TJ;
    constexpr int BUF = BM * SPP_HROWB;
    constexpr int TPIECES = BM * 16 / NT;  // 16-byte token pieces per thread and half chunk
    static_assert(TPIECES >= 1 && (BM * 16) % NT == 0, "token staging");
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * BUF];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nrow = lane & 15, g4 = lane >> 4;
    const int m0 = blockIdx.y * BM;
    const int t0 = ((int)blockIdx.x * NW + __builtin_amdgcn_readfirstlane(wave)) * RT;
    const int C = K / SP_KCHUNK;
    const int HC = 2 * C;
    const int jact = min(TJ, (M - m0 + 15) / 16);  // token tiles holding a row below M

    // ------------------------------------------------------------- loaders
    const size_t tstride = (size_t)C * sp_chunk_bytes<VBITS>();
    const uint8_t* vt = vals + (size_t)t0 * tstride + lane * sp_lane_bytes<VBITS>();
    const uint8_t* mt = meta + (size_t)t0 * C * 512 + lane * 8;
    const uint16_t* sn = scales + 16 * t0 + nrow;
    SpVals<VBITS> wv[2][RT];
    u32x2 wm[2][RT];
    uint32_t ws[2][RT];  // scales of groups 2c (low half) and 2c + 1 (high half) of this lane's row
    auto wload = [&](int c, auto SL) {
        constexpr int sl = decltype(SL)::value;
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            wv[sl][t] = sp_load<VBITS>(vt + t * tstride + (size_t)c * sp_chunk_bytes<VBITS>());
            wm[sl][t] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(mt + ((size_t)t * C + c) * 512));
            ws[sl][t] = (uint32_t)sn[16 * t + (size_t)(2 * c) * sstride] |
                        ((uint32_t)sn[16 * t + (size_t)(2 * c + 1) * sstride] << 16);
        }
    };
    const uint16_t* xp[TPIECES];
#pragma unroll
    for (int i = 0; i < TPIECES; ++i) {
        const int id = tid + NT * i;
        xp[i] = x + (size_t)min(m0 + (id >> 4), M - 1) * K + (id & 15) * 8;
    }
    u32x4 tv[TPIECES];
    auto tload = [&](int hc) {
#pragma unroll
        for (int i = 0; i < TPIECES; ++i) tv[i] = ldg128(xp[i] + (size_t)hc * 128);
    };
    auto tstore = [&](uint8_t* buf) {
#pragma unroll
        for (int i = 0; i < TPIECES; ++i) {
            const int id = tid + NT * i;
            const int row = id >> 4, pc = id & 15;
            *reinterpret_cast<u32x4*>(buf + row * SPP_HROWB + ((pc ^ (row & 15)) << 4)) = tv[i];
        }
    };

    // --------------------------------------------------------- multipliers
    f32x4 acc[RT][TJ];
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // A operands of step S (0..3 within the chunk) of tile t from slot SL
    auto deq = [&](u32x4 (&an)[RT], auto SL, auto ST, auto TT) {
        constexpr int sl = decltype(SL)::value, st = decltype(ST)::value, t = decltype(TT)::value;
        const uint32_t sv = st < 2 ? (ws[sl][t] & 0xffffu) : (ws[sl][t] >> 16);
        an[t] = sp_dequant<VBITS, st>(wv[sl][t], sv);
        asm volatile("" : "+v"(an[t]));  // keep the conversion here, between this step's MFMAs
    };
    // B operands of token tile j for step S (its 64 channels are pieces 8 (S & 1) .. + 8 of the half row)
    auto bread = [&](int j, const uint8_t* cur, auto ST, u32x8& b) {
        constexpr int sh = decltype(ST)::value & 1;
        const int r = 16 * j + nrow;
        const int plo = 8 * sh + g4, phi = plo + 4;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(cur + r * SPP_HROWB + ((plo ^ nrow) << 4));
        const u32x4 hi = *reinterpret_cast<const u32x4*>(cur + r * SPP_HROWB + ((phi ^ nrow) << 4));
        b = u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    // index metadata of step ST from slot SL
    auto midx = [&](int (&idx)[RT], auto SL, auto ST) {
        constexpr int sl = decltype(SL)::value, st = decltype(ST)::value;
#pragma unroll
        for (int t = 0; t < RT; ++t) idx[t] = (int)wm[sl][t][st >> 1];
    };
    // one smfmac step: MFMAs of step ST with `a` and `idx`; the RT conversions
    // of `next` spread over the token tiles
    auto step = [&](const uint8_t* cur, auto ST, const u32x4 (&a)[RT], const int (&idx)[RT], auto&& next) {
        constexpr int st = decltype(ST)::value;
        // B operands of token tile j + BA are read before tile j's MFMAs (a
        // tile's RT MFMAs alone are too short to cover one LDS read)
        constexpr int BA = SPP_BA < TJ ? SPP_BA : TJ;
        u32x8 bq[BA + 1];
        static_for<0, BA>([&](auto J) { bread(decltype(J)::value, cur, ST, bq[decltype(J)::value]); });
        static_for<0, TJ>([&](auto J) {
            constexpr int j = decltype(J)::value;
            if constexpr (j + BA < TJ) bread(j + BA, cur, ST, bq[(j + BA) % (BA + 1)]);
            if (j == 0 || j < jact) {
#pragma unroll
                for (int t = 0; t < RT; ++t)
                    acc[t][j] = smfmac16x16x64<st & 1>(a[t], bq[j % (BA + 1)], idx[t], acc[t][j]);
            }
            static_for<j * RT / TJ, (j + 1) * RT / TJ>([&](auto TT) { next(TT); });
        });
    };
    uint8_t* b0 = lds;
    uint8_t* b1 = lds + BUF;
    u32x4 aA[RT], aB[RT];
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    // chunk c from slot SL: halves 0 (buffer b0) and 1 (buffer b1); the last
    // step converts step 0 of chunk c + 1 (slot 1 - SL, loaded one chunk ago)
    // and, once slot SL is dead, loads chunk c + 2 into it
    auto chunk = [&](int c, auto SL) {
        constexpr int sl = decltype(SL)::value;
        using SN = std::integral_constant<int, 1 - sl>;
        int ia[RT], ib[RT];
        tstore(b1);
        tload(min(2 * c + 2, HC - 1));
        midx(ia, SL, I0{});
        step(b0, I0{}, aA, ia, [&](auto TT) { deq(aB, SL, I1{}, TT); });
        step(b0, I1{}, aB, ia, [&](auto TT) { deq(aA, SL, I2{}, TT); });
        __syncthreads();
        tstore(b0);
        tload(min(2 * c + 3, HC - 1));
        midx(ib, SL, I2{});
        step(b1, I2{}, aA, ib, [&](auto TT) { deq(aB, SL, I3{}, TT); });
        // slot SL is dead once step 3's operands are converted and its
        // metadata is in `ib`: chunk c + 2 goes into it
        wload(min(c + 2, C - 1), SL);
        step(b1, I3{}, aB, ib, [&](auto TT) { deq(aA, SN{}, I0{}, TT); });
        __syncthreads();
    };
    wload(0, I0{});
    tload(0);
    tstore(b0);
    tload(1);
    wload(min(1, C - 1), I1{});
    static_for<0, RT>([&](auto TT) { deq(aA, I0{}, I0{}, TT); });
    __syncthreads();
    for (int c = 0; c < C; c += 2) {
        chunk(c, I0{});
        if (c + 1 < C) chunk(c + 1, I1{});
    }

    // D[row 4 g4 + r][col nrow]: rows are weight rows, columns tokens
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
        const int m = m0 + 16 * j + nrow;
        if (m < M) {
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                u32x2 stv;
                stv[0] = (uint32_t)f32_to_f16(acc[t][j][0]) | ((uint32_t)f32_to_f16(acc[t][j][1]) << 16);
                stv[1] = (uint32_t)f32_to_f16(acc[t][j][2]) | ((uint32_t)f32_to_f16(acc[t][j][3]) << 16);
                *reinterpret_cast<u32x2*>(y + (size_t)m * N + 16 * (t0 + t) + 4 * g4) = stv;
            }
        }
    }
}

// Workgroup shape: every workgroup stages its token rows once per chunk, so
// the token traffic from L2 falls as a workgroup covers more weight rows;
// measured at K = 7168, N = 20480 (4-bit / 8-bit codes): 16 tokens on 8
// waves (128 weight rows, 4 chunks in flight) 25.0 -> 20.8 / 35.5 -> 33.4 us,
// 32 and 64 tokens on 16 waves (256 rows) M = 64 45.7 -> 36.1 / 61.4 -> 52.6 us,
// M = 128 76.7 -> 51.2 / 106.8 -> 73.4 us, against 4 waves, 8 in flight
template <int VBITS, int R>
static void launch_stream(const uint16_t* x, int M, int K, int N, const uint8_t* vals, const uint8_t* meta,
                          const uint16_t* scales, int sstride, uint16_t* y, hipStream_t s) {
    constexpr int NWV = R == 1 ? 8 : 16;
    const dim3 grid((N / 16 + NWV - 1) / NWV, (M + 16 * R - 1) / (16 * R));
    hipLaunchKernelGGL((sparse24_stream_kernel<VBITS, R, 4, NWV>), grid, dim3(64 * NWV), 0, s, x, M, K, N, vals, meta,
                       scales, sstride, y);
}

template <int VBITS, int NW, int TPW>
static void launch_decode(const uint16_t* x, int M, int K, int N, const uint8_t* vals, const uint8_t* meta,
                          const uint16_t* scales, int sstride, uint16_t* y, hipStream_t s) {
    const size_t lds = sparse24_decode_lds(M, K);
    auto kern = sparse24_decode_kernel<VBITS, NW, 4, TPW>;
    if (lds + sizeof(f32x4) * 64 * NW * TPW > 65536)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)lds);
    hipLaunchKernelGGL(kern, dim3((N / 16 + TPW - 1) / TPW), dim3(NW * TPW * 64), lds, s, x, M, K, N, vals, meta,
                       scales, sstride, y);
}

// the pipelined kernel's shape, measured at M = 1024, K = 7168, N = 20480 with
// 4-bit codes: 4 waves x 4 weight tiles x 4 token tiles, 2 per CU, 232-235 us
// (the 256 x 64 tile kernel: 243 us); 512 x 64 (8 waves) 256 us, 256 x 128
// (2 weight tiles per wave) 252 us, 128 x 128 (4 waves) 262 us, 128 x 64 at 3
// per CU 277 us; B operands read 1-4 token tiles ahead: equal.  8-bit codes
// take the tile kernel: two chunks of their 32-byte pieces exceed the 256
// registers of two waves per SIMD (445 against 354 us)
#ifndef SPP_NW
#define SPP_NW 4
#define SPP_RT 4
#define SPP_TJ 4
#define SPP_OCC 2
#endif
constexpr int SPP_BN = 16 * SPP_NW * SPP_RT;

template <int VBITS, int NW, int RT, int TJ, int OCC>
static void launch_pipe(const uint16_t* x, int M, int K, int N, const uint8_t* vals, const uint8_t* meta,
                        const uint16_t* scales, int sstride, uint16_t* y, hipStream_t s) {
    const dim3 grid(N / (16 * NW * RT), (M + 16 * TJ - 1) / (16 * TJ));
    hipLaunchKernelGGL((sparse24_pipe_kernel<VBITS, NW, RT, TJ, OCC>), grid, dim3(NW * 64), 0, s, x, M, K, N, vals,
                       meta, scales, sstride, y);
}

constexpr long SP_STREAM_SLOTS = 256;  // resident 16-wave streaming workgroups: one per CU

// batch-size dispatch, chosen by timing on MI355X at K = 7168, N = 20480:
// M = 1, 2: 18 -> 13 us; M = 4: 18.6 -> 17.0 us with the decode kernel
template <int VBITS>
static void launch_sparse24_b(const uint16_t* x, int M, int K, int N, const uint8_t* vals, const uint8_t* meta,
                              const uint16_t* scales, int ss, uint16_t* y, hipStream_t s) {
    if (M <= 4 && sparse24_decode_lds(M, K) <= SP_DECODE_LDS_MAX) {
        if (M <= 2) launch_decode<VBITS, 2, 2>(x, M, K, N, vals, meta, scales, ss, y, s);
        else launch_decode<VBITS, 4, 2>(x, M, K, N, vals, meta, scales, ss, y, s);
    } else if (M > 128 && VBITS == 4 && N % SPP_BN == 0) {
        launch_pipe<VBITS, SPP_NW, SPP_RT, SPP_TJ, SPP_OCC>(x, M, K, N, vals, meta, scales, ss, y, s);
    } else if (M > 128 && N % SPT_BN == 0) {
        const dim3 grid(N / SPT_BN, (M + SPT_BM - 1) / SPT_BM);
        hipLaunchKernelGGL((sparse24_tile_kernel<VBITS, 2>), grid, dim3(SP_THREADS), 0, s, x, M, K, N, vals, meta,
                           scales, ss, y);
    } else if (M <= 16) {
        launch_stream<VBITS, 1>(x, M, K, N, vals, meta, scales, ss, y, s);
    } else if (M <= 64 || (M <= 128 && (long)((N / 16 + 15) / 16) * ((M + 31) / 32) <= SP_STREAM_SLOTS)) {
        // 32-token groups while they all fit one round of resident 16-wave
        // workgroups (M = 96: 49.2 -> 37.5 us; M = 128 would take two rounds: 66 us
        // against 49.5 us for two 64-token groups)
        launch_stream<VBITS, 2>(x, M, K, N, vals, meta, scales, ss, y, s);
    } else {
        launch_stream<VBITS, 4>(x, M, K, N, vals, meta, scales, ss, y, s);
    }
}

void launch_sparse24(int bits, const uint16_t* x, int M, int K, int N, const uint8_t* vals, const uint8_t* meta,
                     const uint16_t* scales, int group_size, uint16_t* y, hipStream_t s) {
    const int ss = group_size == -1 ? 0 : N;  // scale row stride: per-column scales reread row 0
    if (bits == 8) launch_sparse24_b<8>(x, M, K, N, vals, meta, scales, ss, y, s);
    else launch_sparse24_b<4>(x, M, K, N, vals, meta, scales, ss, y, s);
}

}  // namespace wq

// gemm_fp8.hip -- FP8 (OCP E4M3) W8A8 grouped GEMM of the MoE layer, the
// comparison method of the ExpertsInt8 latency table ("[Kernel] W8A16 Int8
// inside FusedMoE", vLLM PR 7415: rows "FP8 (MoE quant-only)", and the review
// thread naming it use_fp8_w8a8).  Weights and activations are E4M3 codes, so
// nothing is dequantised in the loop: the codes go straight into gfx950's
// v_mfma_scale_f32_16x16x128_f8f6f4 (128 input channels per instruction, unit
// block scales); the per-column weight scale and the static activation scale
// multiply the fp32 accumulator in the epilogue.
//
//  - fp8_quant_kernel: x (16-bit) -> E4M3 codes of x / a1 (float32 division,
//    clamped to +-448, the hardware's nearest-even conversion).
//  - fp8_decode_kernel (block 16 / 32): the small-batch shape of the int8
//    path -- a workgroup per (up to RMAX 16-row token blocks of one expert,
//    16 or 32 weight rows), its waves splitting the input channels, the
//    weights streamed once from HBM (a 2 KiB chunk is one MFMA A operand per
//    lane, loaded by two contiguous 1 KiB wave loads), the token codes (B
//    operand) read from L2.
//  - fp8_prefill_kernel (blocks of 64 / 128+): BN weight rows x BM token rows
//    per workgroup; the weights are loaded straight into the A registers one
//    K step ahead, the token rows of a step staged in one of two LDS buffers.
// Epilogues: GATE_UP computes SiLU(gate) * up in fp32 and writes H as E4M3
// codes of h / a2 (the layer's intermediate, 1 byte per value); DOWN writes
// the routed-weight-scaled fp32 rows of Y for the combine; RAW the fp32
// projections (testing).
#include "common.hpp"
#include "launch.hpp"
#include "one_token.hpp"

#include <algorithm>
#include <type_traits>

namespace wq {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// D += A B over 128 input channels: A = 16 weight rows x 128 codes (lane l:
// row l % 16, 32 codes), B = 128 x 16 tokens (lane l: token l % 16, the same
// 32 channels), both E4M3 (format 0), block scales 2^0 (E8M0 127).  The
// channel order inside a lane's 32 bytes is the same for A and B, so the sum
// runs over all 128 channels whatever order the instruction pairs them in.
__device__ __forceinline__ f32x4 mfma_e4m3(const u32x8& a, const u32x8& b, f32x4 c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(__builtin_bit_cast(i32x8, a), __builtin_bit_cast(i32x8, b),
                                                            c, 0, 0, 0, 127, 0, 127);
}

// four floats -> four E4M3 codes (byte i = value i): clamped to +-448 (the
// saturating reading), then v_cvt_pk_fp8_f32, round to nearest even
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    const float lim = 448.0f;
    a = fminf(fmaxf(a, -lim), lim);
    b = fminf(fmaxf(b, -lim), lim);
    c = fminf(fmaxf(c, -lim), lim);
    d = fminf(fmaxf(d, -lim), lim);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

__device__ __forceinline__ u32x8 cat8(const u32x4& lo, const u32x4& hi) {
    return u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// ---------------------------------------------------------------------------
// activation quantisation
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(256) void fp8_quant_kernel(const uint16_t* __restrict__ x, int64_t n8, float scale,
                                                        uint8_t* __restrict__ q) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    const u32x4 v = ldg128(x + i * 8);
    float f[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = __fdiv_rn(act_to_f32<BF16>((uint16_t)(v[j >> 1] >> (16 * (j & 1)))), scale);
    u32x2 o;
    o[0] = e4m3x4(f[0], f[1], f[2], f[3]);
    o[1] = e4m3x4(f[4], f[5], f[6], f[7]);
    *reinterpret_cast<u32x2*>(q + i * 8) = o;
}

void launch_fp8_quant(const uint16_t* x, int64_t rows, int k, bool bf16, float scale, uint8_t* q, hipStream_t s) {
    const int64_t n8 = rows * (int64_t)k / 8;
    if (n8 == 0) return;
    const dim3 grid((unsigned)((n8 + 255) / 256));
    if (bf16) hipLaunchKernelGGL(fp8_quant_kernel<true>, grid, dim3(256), 0, s, x, n8, scale, q);
    else hipLaunchKernelGGL(fp8_quant_kernel<false>, grid, dim3(256), 0, s, x, n8, scale, q);
}

// ---------------------------------------------------------------------------
// small-batch kernel
// ---------------------------------------------------------------------------
// QX (GATE_UP of one token): the workgroup quantises the token's row into LDS
// itself (the quantisation kernel's arithmetic, so the same codes) and takes
// every B operand from there; all rows of the sorted order are that token's.
template <int STAGE, int RMAX, int NP, int NW, int DEPTH, bool QX = false>
__global__ __launch_bounds__(64 * NW) void fp8_decode_kernel(Fp8GemmArgs g) {
    constexpr int NT = (STAGE == STAGE_GATE_UP) ? 2 * NP : NP;  // 16-row weight tiles per workgroup
    static_assert(NW * NT * RMAX * 1024 <= 64 * 1024, "LDS reduction buffer");
    static_assert(RMAX == 1 || RMAX == 2 || RMAX == 4, "passes of RMAX, then 2 and/or 1 blocks");

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int unit = blockIdx.x;
    const int T = g.M * g.topk;
    const int BS = g.block_size;
    const int spb = BS / 16;
    __shared__ f32x4 red[NW][NT][RMAX][64];
    extern __shared__ __attribute__((aligned(16))) uint8_t xq_lds[];  // QX: the token's k_in codes

    // the expert's run of blocks around block b (as in the int8 small-batch kernel)
    const int sbi = blockIdx.y + 65535 * blockIdx.z;
    const int b = sbi / spb;
    const int bi = b - 31 + lane;
    const int ecand = (bi >= 0 && bi < g.cap / BS) ? g.expert_ids[bi] : -1;
    const int ntpp = *g.ntpp;
    if (sbi * 16 >= ntpp) return;
    const int nbu = ntpp / BS;
    const int e = __shfl(ecand, 31);
    const uint64_t run = __ballot(bi >= 0 && bi < nbu && ecand == e);
    const int b0 = (run & 1ull) ? lower_bound_i32(g.expert_ids, 0, b - 31, e) : b - 31 + __builtin_ctzll(run);
    const int b1 = (run >> 63) ? lower_bound_i32(g.expert_ids, b + 33, nbu, e + 1) : b - 31 + 64 - __builtin_clzll(run);
    const int sb_first = b0 * spb;
    const int j = sbi - sb_first;
    if (j % RMAX != 0) return;
    const int q = __popcll(__ballot(lane < spb && g.sorted[(b1 - 1) * BS + 16 * min(lane, spb - 1)] < T));
    const int S = (b1 - 1 - b0) * spb + q;  // live 16-row sub-blocks of the expert

    const int C = g.k_in / FP8_KCHUNK;
    const size_t expert_bytes = (size_t)g.n_out * g.k_in;
    const uint8_t* wt[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
        wt[t] = g.w + (size_t)e * expert_bytes + (size_t)(NT * unit + t) * C * FP8_CHUNK_BYTES + lane * 16;
    const float* se = g.s + (size_t)e * g.n_out;
    const int rowq = 4 * (lane >> 4);

    auto pass = [&](const int s0, auto RC) {
        constexpr int R = decltype(RC)::value;
        constexpr int ITEMS_R = NP * R;
        const uint8_t* arow[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            // pad rows read the block's first row (a real one): every load is unconditional
            const int p_first = (sb_first + s0 + r) * 16;
            const int p = p_first + (lane & 15);
            const int pl = g.sorted[p] < T ? p : p_first;
            const int row = g.a_direct ? pl : g.sorted[pl] / g.topk;
            arow[r] = g.a + (size_t)row * g.k_in + 32 * (lane >> 4);
        }
        f32x4 acc[NT][R];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < R; ++r) acc[t][r] = f32x4{0.f, 0.f, 0.f, 0.f};

        u32x8 wv[DEPTH][NT];
        u32x8 xv[DEPTH][R];
        auto load = [&](int c, int d) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
                wv[d][t] = cat8(ldg128_stream(wt[t] + (size_t)c * FP8_CHUNK_BYTES),
                                ldg128_stream(wt[t] + (size_t)c * FP8_CHUNK_BYTES + 1024));
#pragma unroll
            for (int r = 0; r < R; ++r) {
                if constexpr (QX) {
                    const uint8_t* xl = xq_lds + c * FP8_KCHUNK + 32 * (lane >> 4);
                    xv[d][r] = cat8(*reinterpret_cast<const u32x4*>(xl), *reinterpret_cast<const u32x4*>(xl + 16));
                } else {
                    xv[d][r] = cat8(ldg128(arow[r] + c * FP8_KCHUNK), ldg128(arow[r] + c * FP8_KCHUNK + 16));
                }
            }
        };
        auto compute = [&](int d) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int r = 0; r < R; ++r) acc[t][r] = mfma_e4m3(wv[d][t], xv[d][r], acc[t][r]);
        };
        // split-K over the waves, DEPTH - 1 chunks in flight; indices past the
        // end are clamped to the wave's last chunk (a cache hit)
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
            const int pp = item / R;
            const int r = item % R;
            const int p = (sb_first + s0 + r) * 16 + (lane & 15);
            const int pair = g.sorted[p];
            if constexpr (STAGE == STAGE_GATE_UP) {
                const int tg = 2 * pp, tu = 2 * pp + 1;
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
                    const float gt = gv[i] * g.in_scale * se[(NT * unit + tg) * TILE_ROWS + rowq + i];
                    const float up = uv[i] * g.in_scale * se[(NT * unit + tu) * TILE_ROWS + rowq + i];
                    h[i] = pair < T ? __fdiv_rn(silu_f32(gt) * up, g.out_scale) : 0.0f;
                }
                *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(g.out) + (size_t)p * N + hcol) =
                    e4m3x4(h[0], h[1], h[2], h[3]);
            } else {
                if (pair < T) {
                    f32x4 o = red[0][pp][r][lane];
#pragma unroll
                    for (int w = 1; w < NW; ++w) o += red[w][pp][r][lane];
                    const int row = (NT * unit + pp) * TILE_ROWS + rowq;
                    const float rw = (STAGE == STAGE_DOWN) ? g.topk_w[pair] : 1.0f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) o[i] = o[i] * g.in_scale * se[row + i] * rw;
                    *reinterpret_cast<f32x4*>(static_cast<float*>(g.out) + (size_t)pair * g.n_out + row) = o;
                }
            }
        }
        __syncthreads();
    };
    if constexpr (STAGE == STAGE_GATE_UP) {
        // H rows of all-pad sub-blocks (blocks larger than 16 only): code 0,
        // written by the expert's first workgroup
        if (j == 0) {
            const int N = g.n_out / 2;
            const int p_lo = (sb_first + S) * 16;
            const int p_hi = b1 * BS;
            constexpr int COLS = NP * TILE_ROWS;
            for (int k = threadIdx.x; k < (p_hi - p_lo) * COLS; k += 64 * NW) {
                const int p = p_lo + k / COLS;
                static_cast<uint8_t*>(g.out)[(size_t)p * N + NP * unit * TILE_ROWS + (k % COLS)] = 0;
            }
        }
    }
    if (j >= S) return;
    if constexpr (QX) {
        for (int i = threadIdx.x; i < g.k_in / 8; i += 64 * NW) {
            const u32x4 v = ldg128(g.x16 + 8 * i);
            float f[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint16_t h = (uint16_t)(v[k >> 1] >> (16 * (k & 1)));
                f[k] = __fdiv_rn(g.x_bf16 ? act_to_f32<true>(h) : act_to_f32<false>(h), g.in_scale);
            }
            u32x2 o;
            o[0] = e4m3x4(f[0], f[1], f[2], f[3]);
            o[1] = e4m3x4(f[4], f[5], f[6], f[7]);
            *reinterpret_cast<u32x2*>(xq_lds + 8 * i) = o;
        }
        __syncthreads();
    }
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

template <int STAGE, int RMAX, int NP, int NW, int DEPTH, bool QX = false>
static void launch_fp8_decode_cfg(const Fp8GemmArgs& g, hipStream_t s) {
    constexpr int NT = (STAGE == STAGE_GATE_UP) ? 2 * NP : NP;
    const int nsb = g.cap / 16;
    const dim3 grid(g.n_out / (TILE_ROWS * NT), std::min(nsb, 65535), (nsb + 65534) / 65535);
    hipLaunchKernelGGL((fp8_decode_kernel<STAGE, RMAX, NP, NW, DEPTH, QX>), grid, dim3(64 * NW), QX ? g.k_in : 0, s,
                       g);
}

bool fp8_fold_quant_supported(int stage, int M, int n_out, int k_in, int block_size) {
    return stage == STAGE_GATE_UP && M == 1 && k_in <= FP8_FOLD_MAX_K && !fp8_prefill_supported(n_out, k_in, block_size);
}

// Shapes by the mean rows per touched expert, as for the int8 small-batch
// kernel (the same bytes per weight); a 2 KiB chunk covers 128 channels, so
// half as many chunks per row as int8.  DOWN of a long reduction at 9-24 rows
// per expert takes four row tiles on 8 waves, as int8 does (Mixtral M = 64:
// layer 0.276 -> 0.266 ms); at 8 tokens that shape measured slower (0.184 ->
// 0.191 ms), so one block per pass keeps two tiles.
template <int STAGE>
static void launch_fp8_decode_r(const Fp8GemmArgs& g, hipStream_t s) {
    constexpr bool GU = STAGE == STAGE_GATE_UP;
    constexpr int NT1 = GU ? 2 : 1;
    const int T = g.M * g.topk;
    const int touched = T < g.E ? T : g.E;
    const int rows = (T + touched - 1) / touched;
    const bool np2_ok = (g.n_out % (TILE_ROWS * NT1 * 2)) == 0;
    const bool np4_ok = (g.n_out % (TILE_ROWS * NT1 * 4)) == 0;
    const bool short_k = g.k_in / FP8_KCHUNK <= 16;
    if constexpr (GU) {
        if (g.x16) {  // one token, quantised in the kernel
            launch_fp8_decode_cfg<STAGE, 1, 1, 4, 2, true>(g, s);
            return;
        }
    }
    if (g.E >= 64 && T > 16) {
        if (GU && np2_ok) launch_fp8_decode_cfg<STAGE, 2, 2, 4, 2>(g, s);
        else if (!GU && np2_ok) launch_fp8_decode_cfg<STAGE, 2, 2, 2, 2>(g, s);
        else launch_fp8_decode_cfg<STAGE, 2, 1, 4, 2>(g, s);
    } else if (T <= 16 || rows <= 8) {
        if (GU) launch_fp8_decode_cfg<STAGE, 1, 1, 4, 2>(g, s);
        else if (!np2_ok) launch_fp8_decode_cfg<STAGE, 1, 1, 8, 2>(g, s);
        else if (short_k) launch_fp8_decode_cfg<STAGE, 1, 2, 2, 3>(g, s);
        else launch_fp8_decode_cfg<STAGE, 1, 2, 8, 2>(g, s);
    } else if (rows <= 24) {
        if (!GU && !short_k && np4_ok) launch_fp8_decode_cfg<STAGE, 2, GU ? 1 : 4, 8, 2>(g, s);
        else if (np2_ok) launch_fp8_decode_cfg<STAGE, 2, 2, 4, 2>(g, s);
        else launch_fp8_decode_cfg<STAGE, 2, 1, 4, 2>(g, s);
    } else {
        if (!GU && np2_ok) launch_fp8_decode_cfg<STAGE, 4, 2, 4, 2>(g, s);
        else launch_fp8_decode_cfg<STAGE, 4, 1, 4, 2>(g, s);
    }
}

// ---------------------------------------------------------------------------
// large-batch kernel
// ---------------------------------------------------------------------------
constexpr int FP8_ROWB = FP8_KCHUNK;  // bytes of one token row per K step

// buffer resource over 4 GiB from base (raw addressing: offsets are bytes)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t fp8_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
}

// A token row of one K step is 8 pieces of 16 bytes (channels 16 p .. 16 p +
// 15).  Lane group g of an MFMA reads channels [32 g, 32 g + 32), pieces 2 g
// and 2 g + 1, so piece p is kept in slot (p >> 1) + 4 (p & 1): the first
// read of lane group g is slot g, the second slot 4 + g.  Slot ch of row `row`
// sits at ch ^ ((row >> 1) & 7) of the row.  A B read (16 rows x one slot
// per lane group) and a store (rows x all 8 slots) then fall on distinct
// 16-byte bank groups for each 32 lanes (with the two reads of a lane in
// slots g and 2 g + 1 instead, 2 LDS conflict cycles per LDS instruction
// were counted)
__device__ __forceinline__ int fp8_lds_off(int row, int ch) { return row * FP8_ROWB + ((ch ^ ((row >> 1) & 7)) << 4); }
__device__ __forceinline__ int fp8_slot(int piece) { return (piece >> 1) + 4 * (piece & 1); }

template <int STAGE, int NW, int RT, int BM, int OCC>
__global__ __launch_bounds__(NW * 64, OCC) void fp8_prefill_kernel(Fp8GemmArgs g) {
    constexpr int NT = NW * 64;
    constexpr int BN = NW * RT * 16;
    constexpr int TJ = BM / 16;
    constexpr int TPIECES = BM * 8 / NT;
    constexpr int BUF = BM * FP8_ROWB;
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
            for (int k = tid; k < BM * (BN / 8); k += NT)  // 4 codes per store
                *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(g.out) + (size_t)(row0 + k / (BN / 8)) * N +
                                             ntile * (BN / 2) + 4 * (k % (BN / 8))) = 0u;
        }
        return;
    }

    const int C = g.k_in / FP8_KCHUNK;
    const int step0 = (int)((long)blockIdx.z * C / gridDim.z);  // K slices of unequal length where gridDim.z does not divide C
    const int step_end = (int)((long)(blockIdx.z + 1) * C / gridDim.z);
    const size_t expert_bytes = (size_t)g.n_out * g.k_in;
    const float* se = g.s + (size_t)e * g.n_out;

    const int rt0 = ntile * (BN / TILE_ROWS) + __builtin_amdgcn_readfirstlane(wave) * RT;
    const int tile_stride = C * FP8_CHUNK_BYTES;
    const __amdgpu_buffer_rsrc_t wres = fp8_rsrc(g.w + (size_t)e * expert_bytes + (size_t)rt0 * tile_stride);
    const int wlane = lane * 16;
    u32x8 wA[RT], wB[RT];  // the A operands of two K steps
    auto wload = [&](int step, u32x8 (&w)[RT]) {
#pragma unroll
        for (int t = 0; t < RT; ++t)
            w[t] = cat8(__builtin_amdgcn_raw_buffer_load_b128(wres, wlane, t * tile_stride + step * FP8_CHUNK_BYTES, 0),
                        __builtin_amdgcn_raw_buffer_load_b128(wres, wlane + 1024,
                                                              t * tile_stride + step * FP8_CHUNK_BYTES, 0));
    };
    // token pieces: pad rows read a valid row (their outputs are dropped, H pad rows written as 0)
    const __amdgpu_buffer_rsrc_t ares = fp8_rsrc(g.a);
    uint32_t toff[TPIECES];
#pragma unroll
    for (int i = 0; i < TPIECES; ++i) {
        const int id = tid + NT * i;
        const int p = row0 + (id >> 3);
        const int pair = g.sorted[p];
        const int src = g.a_direct ? p : (pair < T ? pair / g.topk : 0);
        toff[i] = (uint32_t)src * (uint32_t)g.k_in + (id & 7) * 16;
    }
    u32x4 tv[TPIECES];
    auto tload = [&](int step) {
#pragma unroll
        for (int i = 0; i < TPIECES; ++i) tv[i] = __builtin_amdgcn_raw_buffer_load_b128(ares, toff[i], step * FP8_KCHUNK, 0);
    };
    auto tstore = [&](uint8_t* buf) {
#pragma unroll
        for (int i = 0; i < TPIECES; ++i) {
            const int id = tid + NT * i;
            *reinterpret_cast<u32x4*>(buf + fp8_lds_off(id >> 3, fp8_slot(id & 7))) = tv[i];
        }
    };

    f32x4 acc[RT][TJ];
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int brow = lane & 15, g4 = lane >> 4;
    int jact = 0;
#pragma unroll
    for (int j = 0; j < TJ; ++j) jact += __builtin_amdgcn_readfirstlane(g.sorted[row0 + 16 * j]) < T ? 1 : 0;
    const bool full = jact > TJ / 2;  // else the second half of the token tiles is padding only
    constexpr int HALF = TJ / 2;

    // B operand of token tile j: the lane's 32 bytes of its row, pieces 2 g4 and 2 g4 + 1 (slots g4, 4 + g4)
    auto bread = [&](int j, const uint8_t* cur) {
        const int r = 16 * j + brow;
        return cat8(*reinterpret_cast<const u32x4*>(cur + fp8_lds_off(r, g4)),
                    *reinterpret_cast<const u32x4*>(cur + fp8_lds_off(r, 4 + g4)));
    };
    auto body = [&](int step, const uint8_t* cur, uint8_t* nxt, u32x8 (&a)[RT]) {
        tstore(nxt);
        tload(min(step + 2, step_end - 1));
        u32x8 bx = bread(0, cur), by;
        // MFMAs of token tiles j >= jact (padding only) are skipped
        static_for<0, HALF>([&](auto J) {
            constexpr int j = decltype(J)::value;
            if constexpr (j % 2 == 0) {
                by = bread(j + 1, cur);
                if (j == 0 || j < jact) {
#pragma unroll
                    for (int t = 0; t < RT; ++t) acc[t][j] = mfma_e4m3(a[t], bx, acc[t][j]);
                }
            } else {
                if constexpr (j + 1 < TJ) bx = bread(j + 1, cur);
                if (j < jact) {
#pragma unroll
                    for (int t = 0; t < RT; ++t) acc[t][j] = mfma_e4m3(a[t], by, acc[t][j]);
                }
            }
        });
        if (full) {
            static_for<HALF, TJ>([&](auto J) {
                constexpr int j = decltype(J)::value;
                if constexpr (j % 2 == 0) {
                    if constexpr (j + 1 < TJ) by = bread(j + 1, cur);
                    if (j < jact) {
#pragma unroll
                        for (int t = 0; t < RT; ++t) acc[t][j] = mfma_e4m3(a[t], bx, acc[t][j]);
                    }
                } else {
                    if constexpr (j + 1 < TJ) bx = bread(j + 1, cur);
                    if (j < jact) {
#pragma unroll
                        for (int t = 0; t < RT; ++t) acc[t][j] = mfma_e4m3(a[t], by, acc[t][j]);
                    }
                }
            });
        }
        // this step's weight registers are free once its MFMAs are issued:
        // refill them with step + 2 (one full step of latency)
        wload(min(step + 2, step_end - 1), a);
        __syncthreads();
    };
    uint8_t* b0 = lds;
    uint8_t* b1 = lds + BUF;
    tload(step0);
    wload(step0, wA);
    tstore(b0);
    tload(min(step0 + 1, step_end - 1));
    wload(min(step0 + 1, step_end - 1), wB);
    __syncthreads();
    for (int step = step0; step < step_end; step += 2) {
        body(step, b0, b1, wA);
        if (step + 1 < step_end) body(step + 1, b1, b0, wB);
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
            for (int qq = 0; qq < RT / 2; ++qq) {
                const int gtile = rt0 + 2 * qq;  // gate rows; gtile + 1 holds the matching up rows
                const int hcol = (gtile / 2) * TILE_ROWS + 4 * g4;
                float h[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float gt = acc[2 * qq][j][r] * g.in_scale * se[gtile * TILE_ROWS + 4 * g4 + r];
                    const float up = acc[2 * qq + 1][j][r] * g.in_scale * se[(gtile + 1) * TILE_ROWS + 4 * g4 + r];
                    h[r] = (pair < T) ? __fdiv_rn(silu_f32(gt) * up, g.out_scale) : 0.0f;
                }
                *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(g.out) + (size_t)p * N + hcol) =
                    e4m3x4(h[0], h[1], h[2], h[3]);
            }
        } else {
            if (pair < T) {
                const float rw = (STAGE == STAGE_DOWN) ? g.topk_w[pair] : 1.0f;
#pragma unroll
                for (int t = 0; t < RT; ++t) {
                    const int n0 = (rt0 + t) * TILE_ROWS + 4 * g4;
                    f32x4 o;
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[r] = acc[t][j][r] * g.in_scale * se[n0 + r] * rw;
                    *reinterpret_cast<f32x4*>(yslab + (size_t)pair * g.n_out + n0) = o;
                }
            }
        }
    }
}

template <int STAGE, int NW, int RT, int BM, int OCC>
static void launch_fp8_prefill_cfg(const Fp8GemmArgs& g, int ksplit, hipStream_t s) {
    const dim3 grid(g.n_out / (NW * RT * 16), g.cap / BM, ksplit);
    hipLaunchKernelGGL((fp8_prefill_kernel<STAGE, NW, RT, BM, OCC>), grid, dim3(NW * 64), 0, s, g);
}

// shapes (weight rows x token rows, waves, workgroups per CU):
//   N512 512 x 128, 8 waves, 1 per CU   (n_out % 512 == 0)
//   N128 128 x 128, 4 waves (2 tiles each), 2 per CU
//   T256 256 x 64, 4 waves, 2 per CU    (blocks of 64)
//   T128 128 x 64, 4 waves (2 tiles each), 2 per CU
enum Fp8Shape { F8_N512, F8_N128, F8_T256, F8_T128 };

static Fp8Shape fp8_shape(int n_out, int block_size) {
    if (block_size == 64) return n_out % 256 == 0 ? F8_T256 : F8_T128;
    return n_out % 512 == 0 ? F8_N512 : F8_N128;
}

bool fp8_prefill_supported(int n_out, int k_in, int block_size) {
    return (block_size == 64 || block_size % 128 == 0) && n_out % 128 == 0 && k_in % FP8_KCHUNK == 0;
}

// K slices of the large-batch DOWN (1 to 4): the smallest split whose grid,
// in rounds of resident workgroups of 1/ks of K, takes at least 15 % fewer
// rounds than the smallest split before it, with at least 8 K steps per slice
int fp8_down_split(int T, int E, int n_out, int k_in, int block_size) {
    if (!fp8_prefill_supported(n_out, k_in, block_size) || T <= 0) return 1;
    const int steps = k_in / FP8_KCHUNK;
    const Fp8Shape sh = fp8_shape(n_out, block_size);
    const int bn = sh == F8_N512 ? 512 : (sh == F8_T256 ? 256 : 128);
    const int bm = block_size == 64 ? 64 : 128;
    const int slots = sh == F8_N512 ? 256 : 512;
    const long mt = ((long)T + (long)std::min(T, E) * (bm / 2) + bm - 1) / bm;
    const long wgs = (long)(n_out / bn) * mt;
    auto rounds = [&](int ks) { return (double)((wgs * ks + slots - 1) / slots) / ks; };
    int best = 1;
    double best_t = rounds(1);
    for (int ks = 2; ks <= 4; ++ks) {
        if (steps / ks < 8) break;
        const double t = rounds(ks);
        if (t < 0.85 * best_t) best = ks, best_t = t;
    }
    return best;
}

template <int STAGE>
static void launch_fp8_prefill_s(const Fp8GemmArgs& g, int ksplit, hipStream_t s) {
    switch (fp8_shape(g.n_out, g.block_size)) {
        case F8_N512: launch_fp8_prefill_cfg<STAGE, 8, 4, 128, 1>(g, ksplit, s); break;
        case F8_N128: launch_fp8_prefill_cfg<STAGE, 4, 2, 128, 2>(g, ksplit, s); break;
        case F8_T256: launch_fp8_prefill_cfg<STAGE, 4, 4, 64, 2>(g, ksplit, s); break;
        default: launch_fp8_prefill_cfg<STAGE, 4, 2, 64, 2>(g, ksplit, s); break;
    }
}

// ---------------------------------------------------------------------------
// DOWN of one token with the top-k weighted sum folded in (the E4M3 twin of
// the int8 / int4 one-token kernel).  Slot b is block b of the sorted order:
// its expert's weights start streaming at once, while one wave reads which
// pairs sit in which block (one_token.hpp); the real H code rows are then
// staged in LDS, and one workgroup per 16 output columns streams the 16-row
// tile of every used slot, NW waves splitting the 2 KiB chunks (wave w takes
// chunks w, w + NW, ...), DEPTH chunks per slot in flight.  B column c of slot
// b carries the block's c-th real row, so a pair's product is one column of
// its slot's result; the waves' partial sums of those columns are added in
// LDS in wave order, scaled as the DOWN epilogue scales a routed row (a2, the
// column's weight scale, the pair's routed weight) and summed over the pairs
// in slot order, written as one output row in the activation type: no
// per-pair fp32 rows, no combine launch.  A pair missing from the sorted
// order, or one whose block names no valid expert, adds nothing.
// ---------------------------------------------------------------------------
template <bool BF16, int TK, int NW, int DEPTH>
__global__ __launch_bounds__(NW * 64) void fp8_down_combine_kernel(Fp8GemmArgs g) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    __shared__ OneTokenPlan<TK> pl;
    __shared__ f32x4 red[NW][TK][TK][4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int tile = blockIdx.x;
    const int K = g.k_in;
    const int C = K / FP8_KCHUNK;

    int eb[TK];
    one_token_experts<TK>(g.expert_ids, g.cap, g.block_size, g.E, eb);
    const size_t expert_bytes = (size_t)g.n_out * K;
    const uint8_t* wt[TK];
#pragma unroll
    for (int b = 0; b < TK; ++b)
        wt[b] = g.w + (size_t)eb[b] * expert_bytes + (size_t)tile * C * FP8_CHUNK_BYTES + lane * 16;

    const int nw = wave < C ? (C - 1 - wave) / NW + 1 : 0;
    const int clast = wave < C ? wave + (nw - 1) * NW : C - 1;
    u32x8 wv[DEPTH][TK];
    auto wload = [&](int i, int slot) {
        const size_t off = (size_t)min(wave + NW * i, clast) * FP8_CHUNK_BYTES;
#pragma unroll
        for (int b = 0; b < TK; ++b) wv[slot][b] = cat8(ldg128_stream(wt[b] + off), ldg128_stream(wt[b] + off + 1024));
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

    // stage the real H code rows (rows past them read as code 0)
    const int xrow_b = K + 16;
    const int kp = K / 16;  // 16-byte pieces per row
    for (int q = tid; q < TK * kp; q += NW * 64) {
        const int r = q / kp, pc = q - r * kp;
        const int p = pl.pos[r];
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (p >= 0) v = ldg128(g.a + (size_t)p * K + 16 * pc);
        *reinterpret_cast<u32x4*>(lds + (size_t)r * xrow_b + 16 * pc) = v;
    }
    const uint8_t* xr[TK];  // this lane's B row of each slot
#pragma unroll
    for (int b = 0; b < TK; ++b)
        xr[b] = lds + (size_t)(pl.row0[b] + min(lane & 15, max(pl.cnt[b], 1) - 1)) * xrow_b + 32 * (lane >> 4);
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
            const uint8_t* xc = xr[b] + (size_t)c * FP8_KCHUNK;
            const u32x8 bv = cat8(*reinterpret_cast<const u32x4*>(xc), *reinterpret_cast<const u32x4*>(xc + 16));
            acc[b] = mfma_e4m3(wv[u][b], bv, acc[b]);
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
            const float* se = g.s + (size_t)min(max(g.expert_ids[b], 0), g.E - 1) * g.n_out + row;
            const float rw = g.topk_w[j];
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = o[i] * g.in_scale * se[i] * rw;
            res += o;
        }
        u32x2 st;
        st[0] = (uint32_t)f32_to_act<BF16>(res[0]) | ((uint32_t)f32_to_act<BF16>(res[1]) << 16);
        st[1] = (uint32_t)f32_to_act<BF16>(res[2]) | ((uint32_t)f32_to_act<BF16>(res[3]) << 16);
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(g.out) + row) = st;
    }
}

static size_t fp8_down_combine_lds(int topk, int k_in) { return (size_t)topk * ((size_t)k_in + 16); }

// one token, top-k up to 4, 32 or more 2 KiB chunks per tile, the H code rows in LDS
bool fp8_down_combine_supported(int M, int topk, int n_out, int k_in) {
    return M == 1 && topk >= 1 && topk <= 4 && k_in % FP8_KCHUNK == 0 && k_in / FP8_KCHUNK >= 32 &&
           n_out % TILE_ROWS == 0 && fp8_down_combine_lds(topk, k_in) <= 128 * 1024;
}

template <bool BF16, int TK>
static void launch_fp8_down_combine_tk(const Fp8GemmArgs& g, hipStream_t s) {
    constexpr int NW = 16, DEPTH = TK <= 2 ? 3 : 2;
    auto kern = fp8_down_combine_kernel<BF16, TK, NW, DEPTH>;
    const size_t dyn = fp8_down_combine_lds(TK, g.k_in);
    if (dyn > 64 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)dyn);
    hipLaunchKernelGGL(kern, dim3(g.n_out / TILE_ROWS), dim3(NW * 64), dyn, s, g);
}

template <bool BF16>
static void launch_fp8_down_combine_b(const Fp8GemmArgs& g, hipStream_t s) {
    switch (g.topk) {
        case 1: launch_fp8_down_combine_tk<BF16, 1>(g, s); break;
        case 2: launch_fp8_down_combine_tk<BF16, 2>(g, s); break;
        case 3: launch_fp8_down_combine_tk<BF16, 3>(g, s); break;
        default: launch_fp8_down_combine_tk<BF16, 4>(g, s); break;
    }
}

void launch_fp8_down_combine(bool bf16, const Fp8GemmArgs& g, hipStream_t s) {
    if (bf16) launch_fp8_down_combine_b<true>(g, s);
    else launch_fp8_down_combine_b<false>(g, s);
}

int launch_gemm_fp8(int stage, const Fp8GemmArgs& g, hipStream_t s) {
    if (fp8_prefill_supported(g.n_out, g.k_in, g.block_size)) {
        const int ks = stage == STAGE_DOWN ? fp8_down_split(g.M * g.topk, g.E, g.n_out, g.k_in, g.block_size) : 1;
        if (stage == STAGE_GATE_UP) launch_fp8_prefill_s<STAGE_GATE_UP>(g, 1, s);
        else if (stage == STAGE_DOWN) launch_fp8_prefill_s<STAGE_DOWN>(g, ks, s);
        else launch_fp8_prefill_s<STAGE_RAW>(g, 1, s);
        return ks;
    }
    if (stage == STAGE_GATE_UP) launch_fp8_decode_r<STAGE_GATE_UP>(g, s);
    else if (stage == STAGE_DOWN) launch_fp8_decode_r<STAGE_DOWN>(g, s);
    else launch_fp8_decode_r<STAGE_RAW>(g, s);
    return 1;
}

}  // namespace wq

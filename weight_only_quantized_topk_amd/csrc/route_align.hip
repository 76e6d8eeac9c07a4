// route_align.hip -- moe_route (router softmax + top-k) and moe_align (token
// sort and pad per expert) for gfx950.
//
// moe_route: one 64-lane wave per token (the top-k and softmax steps are in
// route_common.hpp).
//
// moe_align: one 1024-thread workgroup; each of its 16 waves sorts a
// contiguous run of the pairs.  (1) per-run per-expert counts (inside a wave,
// lanes with the same expert are found with one ballot per expert-id bit);
// (2) padded exclusive scan over experts, expert_ids and pad/tail sentinels
// written by the expert's own thread, and each run's first write position per
// expert; (3) a stable scatter along each run, a pair ranked by a popcount of
// the lower lanes holding its expert.  No atomic decides an order, so the
// output is the unique stable one.
// moe_route_align: for batches up to 16 tokens one 1024-thread workgroup does
// both, the expert ids staying in LDS between the two (one launch instead of
// two, the same outputs).
// (The token sort is the moe_align_block_size step of "Marlin moe integration",
// nm-vllm PR 266, review thread on its kernel and its block size of 16.)
#include "common.hpp"
#include "launch.hpp"
#include "route_common.hpp"

#include <algorithm>

namespace wq {

__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int M, int E, int topk,
                                                    int renormalize, float* __restrict__ w_out,
                                                    int32_t* __restrict__ ids_out) {
    const int lane = threadIdx.x & 63;
    const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (m >= M) return;
    route_token(logits + (size_t)m * E, E, topk, renormalize, lane, w_out + (size_t)m * topk,
                ids_out + (size_t)m * topk, nullptr);
}

void launch_route(const float* logits, int M, int E, int topk, int renormalize, float* w, int32_t* ids,
                  hipStream_t s) {
    hipLaunchKernelGGL(route_kernel, dim3((M + 3) / 4), dim3(256), 0, s, logits, M, E, topk, renormalize, w, ids);
}

// ---------------------------------------------------------------------------
constexpr int ALIGN_THREADS = 1024;
constexpr int ALIGN_WAVES = ALIGN_THREADS / 64;
// the fused route + align kernel serves batches up to 16 tokens (one per wave:
// more tokens per wave made it slower than the separate kernels, which spread
// the tokens over many compute units)
constexpr int ROUTE_ALIGN_MAX_M = 16;
constexpr int ROUTE_ALIGN_MAX_T = 1024;

// the align steps for one 1024-thread workgroup; ids may point to global or
// LDS memory; smem holds E * (1 + ALIGN_WAVES) ints.
// Wave w owns the contiguous run of pairs [w L, (w + 1) L).  (1) Each wave
// counts its run per expert (64 pairs a step: the lanes holding one expert
// are found with one ballot per expert-id bit, the group's lowest lane adds
// the group size to the wave's row of the table).  (2) One thread per expert
// adds its column, pads it, and the padded counts are scanned over experts;
// the column is then turned into each wave's first write position for that
// expert (the expert's offset plus the counts of the runs before).  (3) Each
// wave walks its run again and writes pair i at its expert's running
// position plus its rank among the step's lanes with that expert.  Runs are in
// pair order and ranks are by lane, so the result is the unique stable order,
// and the waves need no synchronisation between steps.
__device__ __forceinline__ void align_body(const int32_t* ids, int T, int E, int BS, int nbits,
                                           int32_t* __restrict__ sorted, int32_t* __restrict__ expert_ids,
                                           int32_t* __restrict__ ntpp, int cap, int* smem) {
    int* tab = smem;                     // [ALIGN_WAVES][E] counts per run, then write positions
    __shared__ int wsum[ALIGN_WAVES];
    __shared__ int total_s;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int L = ((T + ALIGN_WAVES - 1) / ALIGN_WAVES + 63) / 64 * 64;  // pairs per run
    const int r0 = wave * L;
    const int r1 = min(T, r0 + L);
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    // the lanes of this step holding the same (valid) expert as this lane
    auto peers_of = [&](int e, bool valid) {
        uint64_t peers = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = valid && ((e >> b) & 1);
            const uint64_t m = __ballot(bit);
            peers &= bit ? m : ~m;
        }
        return peers;
    };

    for (int k = tid; k < ALIGN_WAVES * E; k += ALIGN_THREADS) tab[k] = 0;
    __syncthreads();
    int* row = tab + wave * E;
    // the run, 64 pairs a step
    auto walk = [&](auto step) {
        for (int i0 = r0; i0 < r1; i0 += 64) {
            const int i = i0 + lane;
            step(i, (i < r1) ? ids[i] : -1);
        }
    };
    walk([&](int, int e) {
        const bool valid = (e >= 0 && e < E);
        const uint64_t peers = peers_of(e, valid);
        if (valid && (peers & lt_mask) == 0) row[e] += __popcll(peers);
    });
    __syncthreads();

    // exclusive scan of the padded counts (E <= 1024: one expert per thread)
    int c_e = 0;
    if (tid < E)
        for (int w = 0; w < ALIGN_WAVES; ++w) c_e += tab[w * E + tid];
    const int p_e = (c_e + BS - 1) / BS * BS;
    int incl = p_e;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int wave_off = 0;
    for (int w = 0; w < wave; ++w) wave_off += wsum[w];
    const int o_e = wave_off + incl - p_e;
    if (tid == ALIGN_THREADS - 1) total_s = wave_off + incl;
    if (tid < E) {
        int pos = o_e;  // first write position of each run for this expert
        for (int w = 0; w < ALIGN_WAVES; ++w) {
            const int c = tab[w * E + tid];
            tab[w * E + tid] = pos;
            pos += c;
        }
        for (int b = o_e / BS; b < (o_e + p_e) / BS; ++b) expert_ids[b] = tid;
        for (int p = o_e + c_e; p < o_e + p_e; ++p) sorted[p] = T;
    }
    __syncthreads();
    const int total = total_s;
    if (tid == 0) *ntpp = total;
    for (int p = total + tid; p < cap; p += ALIGN_THREADS) sorted[p] = T;
    for (int b = total / BS + tid; b < cap / BS; b += ALIGN_THREADS) expert_ids[b] = -1;

    // stable scatter, each wave along its own run
    walk([&](int i, int e) {
        const bool valid = (e >= 0 && e < E);
        const uint64_t peers = peers_of(e, valid);
        if (valid) {
            sorted[row[e] + __popcll(peers & lt_mask)] = i;
            if ((peers & lt_mask) == 0) row[e] += __popcll(peers);  // after every lane of the group read it
        }
    });
}

__global__ __launch_bounds__(ALIGN_THREADS) void align_kernel(const int32_t* __restrict__ ids, int T, int E, int BS,
                                                              int nbits, int32_t* __restrict__ sorted,
                                                              int32_t* __restrict__ expert_ids,
                                                              int32_t* __restrict__ ntpp, int cap) {
    extern __shared__ int smem[];
    align_body(ids, T, E, BS, nbits, sorted, expert_ids, ntpp, cap, smem);
}

// moe_route + moe_align for small batches in one workgroup: its 16 waves route
// the tokens (one wave per token), the expert ids stay in LDS for the align steps
__global__ __launch_bounds__(ALIGN_THREADS) void route_align_kernel(const float* __restrict__ logits, int M, int E,
                                                                    int topk, int renormalize,
                                                                    float* __restrict__ w_out,
                                                                    int32_t* __restrict__ ids_out, int BS, int nbits,
                                                                    int32_t* __restrict__ sorted,
                                                                    int32_t* __restrict__ expert_ids,
                                                                    int32_t* __restrict__ ntpp, int cap) {
    extern __shared__ int smem[];
    int* sids = smem + E * (1 + ALIGN_WAVES);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    for (int m = wave; m < M; m += ALIGN_WAVES)
        route_token(logits + (size_t)m * E, E, topk, renormalize, lane, w_out + (size_t)m * topk,
                    ids_out + (size_t)m * topk, sids + m * topk);
    __syncthreads();
    align_body(sids, M * topk, E, BS, nbits, sorted, expert_ids, ntpp, cap, smem);
}

// ---------------------------------------------------------------------------
// moe_route + moe_align for the smallest batches (at most 64 pairs over at
// most 64 experts): one wave per token routes it (as route_kernel does, so
// the weights are the same bits), and after the only barrier wave 0 sorts
// the pairs alone -- lane i holds pair i, lane e expert e: ranks and counts by
// shuffles, the padded offsets by a wave scan -- with no further block-wide
// synchronisation (the 1024-thread align took 7-8 us for one token).
// ---------------------------------------------------------------------------
constexpr int ROUTE_ALIGN_WAVE_MAX = 64;  // pairs and experts

__global__ __launch_bounds__(1024) void route_align_wave_kernel(const float* __restrict__ logits, int M, int E,
                                                                int topk, int renormalize, float* __restrict__ w_out,
                                                                int32_t* __restrict__ ids_out, int BS,
                                                                int32_t* __restrict__ sorted,
                                                                int32_t* __restrict__ expert_ids,
                                                                int32_t* __restrict__ ntpp, int cap) {
    __shared__ int sids[ROUTE_ALIGN_WAVE_MAX];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    for (int m = wave; m < M; m += nw)
        route_token(logits + (size_t)m * E, E, topk, renormalize, lane, w_out + (size_t)m * topk,
                    ids_out + (size_t)m * topk, sids + m * topk);
    __syncthreads();
    if (wave != 0) return;
    align_wave(sids, M * topk, E, BS, cap, lane, sorted, expert_ids, ntpp);
}

// Routing, sort and the act-order gather of a small batch in one launch.
// Workgroup p routes and sorts the whole batch itself into LDS (rank-counting
// top-k, one wave per token, then align_wave: the same arithmetic as
// route_align_wave_kernel, so the same arrays), the first workgroup also
// writes the routing arrays, and then workgroup p writes row p of the
// gathered activations: x of the pair's token in its expert's input-channel
// order (a pad row as zeros), which the gate/up GEMM reads by sorted position.
// For at most 16 tokens, 64 pairs, 64 experts and a capacity of at most
// FR_MAX_CAP rows.
__global__ __launch_bounds__(256) void route_align_gather_kernel(
    const float* __restrict__ logits, int M, int E, int topk, int renormalize, float* __restrict__ w_out,
    int32_t* __restrict__ ids_out, int BS, int32_t* __restrict__ sorted_out, int32_t* __restrict__ expert_ids_out,
    int32_t* __restrict__ ntpp_out, int cap, const uint16_t* __restrict__ x, const int32_t* __restrict__ perm,
    int k_in, uint16_t* __restrict__ a1) {
    __shared__ int s_sorted[FR_MAX_CAP];
    __shared__ int s_blocks[FR_MAX_CAP / 16];
    __shared__ int s_ids[FR_MAX_PAIRS];
    __shared__ float s_w[FR_MAX_PAIRS];
    __shared__ int s_ntpp;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int T = M * topk;
    for (int m = wave; m < M; m += 4)
        route_token_rank(logits + (size_t)m * E, E, topk, renormalize, lane, s_w + m * topk, s_ids + m * topk, nullptr);
    __syncthreads();
    if (wave == 0) align_wave(s_ids, T, E, BS, cap, lane, s_sorted, s_blocks, &s_ntpp);
    __syncthreads();
    if (blockIdx.x == 0) {
        for (int i = threadIdx.x; i < T; i += 256) {
            w_out[i] = s_w[i];
            ids_out[i] = s_ids[i];
        }
        for (int i = threadIdx.x; i < cap; i += 256) sorted_out[i] = s_sorted[i];
        for (int i = threadIdx.x; i < cap / BS; i += 256) expert_ids_out[i] = s_blocks[i];
        if (threadIdx.x == 0) *ntpp_out = s_ntpp;
    }
    const int p = blockIdx.x;
    if (p >= s_ntpp) return;
    const int pair = s_sorted[p];
    uint16_t* dst = a1 + (size_t)p * k_in;
    if (pair >= T) {
        for (int k = threadIdx.x * 8; k < k_in; k += 256 * 8) *reinterpret_cast<u32x4*>(dst + k) = u32x4{0u, 0u, 0u, 0u};
        return;
    }
    const uint16_t* src = x + (size_t)(pair / topk) * k_in;
    const int32_t* pe = perm + (size_t)s_blocks[p / BS] * k_in;
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

bool route_gather_supported(int M, int topk, int E, int cap, int BS) {
    return M >= 1 && M <= ROUTE_ALIGN_MAX_M && M * topk <= FR_MAX_PAIRS && E <= 64 && cap <= FR_MAX_CAP &&
           cap % BS == 0;
}

void launch_route_align_gather(const float* logits, int M, int E, int topk, int renormalize, float* w, int32_t* ids,
                               int BS, int32_t* sorted, int32_t* expert_ids, int32_t* ntpp, int cap,
                               const uint16_t* x, const int32_t* perm, int k_in, uint16_t* a1, hipStream_t s) {
    hipLaunchKernelGGL(route_align_gather_kernel, dim3(cap), dim3(256), 0, s, logits, M, E, topk, renormalize, w, ids,
                       BS, sorted, expert_ids, ntpp, cap, x, perm, k_in, a1);
}

static int id_bits(int E) {
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    return nbits;
}

void launch_align(const int32_t* ids, int T, int E, int BS, int32_t* sorted, int32_t* expert_ids, int32_t* ntpp,
                  int cap, hipStream_t s) {
    const size_t lds = sizeof(int) * (size_t)E * (1 + ALIGN_WAVES);
    if (lds > 65536)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&align_kernel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(align_kernel, dim3(1), dim3(ALIGN_THREADS), lds, s, ids, T, E, BS, id_bits(E), sorted,
                       expert_ids, ntpp, cap);
}

// ---------------------------------------------------------------------------
// Routing of a dense layer (one expert, top-1): what moe_align produces for
// topk_ids = 0 -- the rows in order, pads (id M) up to the capacity, expert 0
// for every block, M rounded up to the block size -- and unit routed weights.
__global__ __launch_bounds__(256) void identity_route_kernel(int M, int cap, int BS, int32_t* __restrict__ sorted,
                                                             int32_t* __restrict__ expert_ids,
                                                             int32_t* __restrict__ ntpp, float* __restrict__ w) {
    const int stride = (int)(gridDim.x * blockDim.x);
    for (int i = (int)(blockIdx.x * blockDim.x + threadIdx.x); i < cap; i += stride) {
        sorted[i] = i < M ? i : M;
        if (i < M) w[i] = 1.0f;
        if (i % BS == 0) expert_ids[i / BS] = 0;
        if (i == 0) *ntpp = (M + BS - 1) / BS * BS;
    }
}

void launch_identity_route(int M, int cap, int BS, int32_t* sorted, int32_t* expert_ids, int32_t* ntpp, float* w,
                           hipStream_t s) {
    const int blocks = std::max(1, std::min(1024, (cap + 255) / 256));
    hipLaunchKernelGGL(identity_route_kernel, dim3(blocks), dim3(256), 0, s, M, cap, BS, sorted, expert_ids, ntpp, w);
}

bool route_align_fused(int M, int topk) { return M <= ROUTE_ALIGN_MAX_M && M * topk <= ROUTE_ALIGN_MAX_T; }

void launch_route_align(const float* logits, int M, int E, int topk, int renormalize, float* w, int32_t* ids, int BS,
                        int32_t* sorted, int32_t* expert_ids, int32_t* ntpp, int cap, hipStream_t s) {
    if (M * topk <= ROUTE_ALIGN_WAVE_MAX && E <= ROUTE_ALIGN_WAVE_MAX) {
        const int waves = std::min(M, ALIGN_WAVES);
        hipLaunchKernelGGL(route_align_wave_kernel, dim3(1), dim3(64 * waves), 0, s, logits, M, E, topk, renormalize, w,
                           ids, BS, sorted, expert_ids, ntpp, cap);
        return;
    }
    const size_t lds = sizeof(int) * ((size_t)E * (1 + ALIGN_WAVES) + (size_t)M * topk);
    if (lds > 65536)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&route_align_kernel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(route_align_kernel, dim3(1), dim3(ALIGN_THREADS), lds, s, logits, M, E, topk, renormalize, w,
                       ids, BS, id_bits(E), sorted, expert_ids, ntpp, cap);
}

}  // namespace wq

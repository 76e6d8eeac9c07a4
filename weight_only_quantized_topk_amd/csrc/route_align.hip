// route_align.hip -- moe_route (router softmax + top-k) and moe_align (token
// sort and pad per expert) for gfx950.
//
// moe_route: one 64-lane wave per token.  Each lane holds up to 16 logits
// (E <= 1024).  Top-k is k rounds of a wave-wide arg-max over the experts not
// yet chosen, comparing (larger logit, then smaller expert index) as one
// 64-bit value, reduced within rows of 16 lanes by DPP; up to 64
// experts, each expert's rank in that order is counted directly instead (E
// steps of a few instructions, against topk chains of shuffle reductions).  The slot
// weights are exp(l_j - max) / sum, evaluated in double with the sum taken in
// ascending slot order, rounded once to float.
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

#include <algorithm>

namespace wq {

constexpr int ROUTE_MAX_PER_LANE = 16;  // E <= 1024

// A logit as an unsigned key in the order of the floats: -0 and +0 equal, and
// every NaN below every number (so the order is total and the top-k always
// names topk distinct experts)
__device__ __forceinline__ uint32_t order_key(float v) {
    if (v != v) return 0u;
    const uint32_t b = __float_as_uint(v + 0.0f);  // -0 -> +0
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// the logit of a key (a NaN for key 0; -0 comes back as +0)
__device__ __forceinline__ float key_value(uint32_t k) {
    if (k == 0u) return __uint_as_float(0x7fc00000u);
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// a candidate expert as one unsigned 64-bit value, larger = better: the key
// above, then the smaller expert index (its complement in the low half); 0
// stands for no candidate (every real one has a low half >= ~1023)
__device__ __forceinline__ uint64_t cand(uint32_t key, int e) { return ((uint64_t)key << 32) | (uint32_t)~e; }

// larger of a lane's candidate and its partner's under a DPP lane pattern
template <int CTRL>
__device__ __forceinline__ uint64_t cand_max_dpp(uint64_t c) {
    const int hi = (int)(uint32_t)(c >> 32), lo = (int)(uint32_t)c;
    const uint64_t o = ((uint64_t)(uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, 0xF, 0xF, false) << 32) |
                       (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, 0xF, 0xF, false);
    return o > c ? o : c;
}

// the largest candidate of the wave, in every lane: within each row of 16
// lanes by DPP (swap neighbours, swap pairs, mirror in 8, mirror in 16: each
// step pairs every lane with one holding the other half of its group), then
// across the rows by two shuffles
__device__ __forceinline__ uint64_t wave_max_cand(uint64_t c) {
    c = cand_max_dpp<0xB1>(c);   // quad_perm [1,0,3,2]
    c = cand_max_dpp<0x4E>(c);   // quad_perm [2,3,0,1]
    c = cand_max_dpp<0x141>(c);  // row_half_mirror
    c = cand_max_dpp<0x140>(c);  // row_mirror
#pragma unroll
    for (int off = 16; off < 64; off <<= 1) {
        const uint64_t o = ((uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)(c >> 32), off, 64) << 32) |
                           (uint32_t)__shfl_xor((int)(uint32_t)c, off, 64);
        c = o > c ? o : c;
    }
    return c;
}

// E <= 64: lane e holds logit e; its rank is the number of experts ahead of it
// in the order above, and the experts ranked below topk are the slots, in rank
// order.  Counting costs E compares per lane, so it serves up to 64 experts
__device__ __forceinline__ void route_token_rank(const float* __restrict__ l, int E, int topk, int renormalize,
                                                 int lane, float* __restrict__ w_row, int32_t* __restrict__ ids_row,
                                                 int* lds_ids) {
    const bool live = lane < E;
    const float v = live ? l[lane] : 0.0f;
    const uint32_t key = order_key(v);
    // expert i's key is read from its lane into a scalar register (a uniform
    // lane index) and compared by every lane without branches
    int rank = 0;
    auto count = [&](int i) {
        const uint32_t ki = (uint32_t)__builtin_amdgcn_readlane((int)key, i);
        rank += (ki > key || (ki == key && i < lane)) ? 1 : 0;
    };
    int i = 0;
    for (; i + 4 <= E; i += 4) {
        count(i);
        count(i + 1);
        count(i + 2);
        count(i + 3);
    }
    for (; i < E; ++i) count(i);
    const bool sel = live && rank < topk;
    // the slot-j expert's lane
    auto slot_lane = [&](int j) { return __builtin_ctzll(__ballot(live && rank == j)); };
    const double vd = (double)v;
    const double mu = __shfl(vd, slot_lane(0), 64);
    const double ex = sel ? exp(vd - mu) : 0.0;
    double denom = 0.0;
    if (renormalize) {
        for (int j = 0; j < topk; ++j) denom += __shfl(ex, slot_lane(j), 64);  // ascending slot order
    } else {
        double part = live ? exp(vd - mu) : 0.0;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
        denom = part;
    }
    if (sel) {
        w_row[rank] = (float)(ex / denom);
        ids_row[rank] = lane;
        if (lds_ids) lds_ids[rank] = lane;
    }
}

// routes token row `l` (E logits) with one wave; lane j < topk writes slot j's
// weight and expert to w_row[j] / ids_row[j] (and to lds_ids[j] if given)
__device__ __forceinline__ void route_token(const float* __restrict__ l, int E, int topk, int renormalize, int lane,
                                            float* __restrict__ w_row, int32_t* __restrict__ ids_row,
                                            int* lds_ids) {
    if (E <= 64) return route_token_rank(l, E, topk, renormalize, lane, w_row, ids_row, lds_ids);
    float v[ROUTE_MAX_PER_LANE];
    uint32_t key[ROUTE_MAX_PER_LANE];
    uint32_t avail = 0;  // bit i: slot i of this lane holds a not-yet-chosen expert
#pragma unroll
    for (int i = 0; i < ROUTE_MAX_PER_LANE; ++i) {
        const int e = lane + 64 * i;
        v[i] = (e < E) ? l[e] : 0.0f;
        key[i] = order_key(v[i]);
        if (e < E) avail |= 1u << i;
    }
    float sel_v = 0.0f;  // lane j < topk ends up holding slot j's logit
    int sel_e = 0;
    for (int j = 0; j < topk; ++j) {
        // lane-local best candidate (0: none), then the wave-wide maximum
        uint64_t c = 0;
#pragma unroll
        for (int i = 0; i < ROUTE_MAX_PER_LANE; ++i) {
            const uint64_t ci = ((avail >> i) & 1u) ? cand(key[i], lane + 64 * i) : 0;
            c = ci > c ? ci : c;
        }
        c = wave_max_cand(c);
        const int be = (int)~(uint32_t)c;
        if ((be & 63) == lane) avail &= ~(1u << (be >> 6));
        if (lane == j) {
            sel_v = key_value((uint32_t)(c >> 32));
            sel_e = be;
        }
    }
    const double mu = (double)__shfl(sel_v, 0, 64);
    const double ex = (lane < topk) ? exp((double)sel_v - mu) : 0.0;
    double denom = 0.0;
    if (renormalize) {
        for (int j = 0; j < topk; ++j) denom += __shfl(ex, j, 64);
    } else {
        double part = 0.0;
#pragma unroll
        for (int i = 0; i < ROUTE_MAX_PER_LANE; ++i)
            if (lane + 64 * i < E) part += exp((double)v[i] - mu);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
        denom = part;
    }
    if (lane < topk) {
        w_row[lane] = (float)(ex / denom);
        ids_row[lane] = sel_e;
        if (lds_ids) lds_ids[lane] = sel_e;
    }
}

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
    const int T = M * topk;
    const int my_e = lane < T ? sids[lane] : -1;  // pair lane's expert
    int rank = 0, cnt = 0;                         // rank among its expert's pairs; count of expert `lane`
    for (int i = 0; i < T; ++i) {
        const int ei = __shfl(my_e, i, 64);
        rank += (i < lane && ei == my_e) ? 1 : 0;
        cnt += (ei == lane) ? 1 : 0;
    }
    const int c_e = lane < E ? cnt : 0;
    const int p_e = (c_e + BS - 1) / BS * BS;
    int incl = p_e;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
    }
    const int o_e = incl - p_e;
    const int total = __shfl(incl, 63, 64);
    if (lane < E) {
        for (int b = o_e / BS; b < (o_e + p_e) / BS; ++b) expert_ids[b] = lane;
        for (int p = o_e + c_e; p < o_e + p_e; ++p) sorted[p] = T;
    }
    const int base = __shfl(o_e, my_e < 0 ? 0 : my_e, 64);
    if (lane < T) sorted[base + rank] = lane;
    for (int p = total + lane; p < cap; p += 64) sorted[p] = T;
    for (int b = total / BS + lane; b < cap / BS; b += 64) expert_ids[b] = -1;
    if (lane == 0) *ntpp = total;
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

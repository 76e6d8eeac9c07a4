// route_common.hpp -- the routing and one-wave sort steps as device functions,
// shared by the routing kernels and the small-batch GEMM that routes a batch
// itself (one launch for route, sort and gate/up).
//
// Top-k: one 64-lane wave per token.  Each lane holds up to 16 logits
// (E <= 1024); k rounds of a wave-wide arg-max over the experts not yet
// chosen, comparing (larger logit, then smaller expert index) as one 64-bit
// value, reduced within rows of 16 lanes by DPP; up to 64 experts each
// expert's rank in that order is counted directly instead (E steps of a few
// instructions, against topk chains of shuffle reductions).  The slot weights
// are exp(l_j - max) / sum, evaluated in double with the sum taken in
// ascending slot order, rounded once to float.
// (The fused_moe interface the kernels plug into: "Marlin moe integration",
// nm-vllm PR 266, review comment on the fused_moe interface.)
#pragma once

#include "common.hpp"

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

// The padded sort of at most 64 pairs over at most 64 experts by one wave
// (lane i holds pair i's expert, sids in LDS): ranks among the pairs of the
// same expert and per-expert counts by shuffles, the padded offsets by a wave
// scan; writes sorted_token_ids, expert_ids (-1 past the used blocks) and the
// padded total, as moe_align does.  The output pointers may be global or LDS.
__device__ __forceinline__ void align_wave(const int* sids, int T, int E, int BS, int cap, int lane,
                                           int32_t* sorted, int32_t* expert_ids, int32_t* ntpp) {
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

}  // namespace wq

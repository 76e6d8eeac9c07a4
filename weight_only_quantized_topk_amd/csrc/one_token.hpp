// one_token.hpp -- where one token's top-k pairs sit in the sorted order, for
// the DOWN kernels that fold the top-k weighted sum into the GEMM.
//
// With one token the top-k pairs are the whole batch, and the alignment puts
// each chosen expert's pairs at the head of one block of sorted_token_ids, in
// expert order: the used blocks are the first ones, at most top-k of them.  A
// kernel can therefore start streaming the weights of block b's expert
// (expert_ids[b], b < top-k) before it has read the sorted order at all, and
// read the rest -- which pairs sit in which block -- while those loads are in
// flight.  A slot is a block; a block holding several real rows (a token's
// top-k naming an expert twice) gives each of them its own MFMA B column.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wq {

template <int TK>
struct OneTokenPlan {
    int cnt[TK];   // real rows of block b (0: slot unused)
    int row0[TK];  // first staged row of block b
    int pos[TK];   // sorted position of staged row q (-1: none, staged as zeros)
    int slot[TK];  // pair j -> block (-1: the pair is not in the sorted order)
    int col[TK];   // pair j -> its B column within the block
};

// block b's expert for addressing before the plan is known: clamped into
// [0, E), so an unused slot still names real memory
template <int TK>
__device__ __forceinline__ void one_token_experts(const int32_t* __restrict__ expert_ids, int cap, int BS, int E,
                                                  int (&eb)[TK]) {
    const int nbc = cap / BS;
#pragma unroll
    for (int b = 0; b < TK; ++b) eb[b] = min(max(expert_ids[min(b, nbc - 1)], 0), E - 1);
}

// run by one whole wave: lane b * TK + c examines position c of block b; a
// real row is a pair index below TK in a used block whose expert is valid
template <int TK>
__device__ __forceinline__ void one_token_plan(OneTokenPlan<TK>& pl, const int32_t* __restrict__ sorted,
                                               const int32_t* __restrict__ expert_ids,
                                               const int32_t* __restrict__ ntpp_p, int cap, int BS, int E,
                                               int lane) {
    static_assert(TK * TK <= 64, "one lane per (block, row)");
    const int ntpp = min(*ntpp_p, cap);
    const int nb = ntpp / BS;
    const int b = lane / TK, c = lane % TK;
    int v = -1, p = 0;
    bool real = false;
    if (lane < TK * TK && b < nb) {
        p = b * BS + c;
        v = sorted[p];
        const int e = expert_ids[b];
        real = v >= 0 && v < TK && e >= 0 && e < E;
    }
    const uint64_t m = __ballot(real);
    const int q = __popcll(m & ((1ull << lane) - 1));  // staged row: rank among the real rows
    const int first = __popcll(m & ((1ull << (b * TK)) - 1));
    if (lane < TK) {
        pl.slot[lane] = -1;
        pl.pos[lane] = -1;
    }
    // one wave's LDS stores complete in program order: the entries below replace the defaults
    if (real) {
        pl.pos[q] = p;
        pl.slot[v] = b;
        pl.col[v] = q - first;
    }
    if (lane < TK * TK && c == 0) {
        pl.row0[b] = first;
        pl.cnt[b] = __popcll((m >> (b * TK)) & ((1ull << TK) - 1));
    }
}

}  // namespace wq

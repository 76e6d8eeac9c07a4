/*
 * oracle.c -- plain, slow CPU oracle for the weight-only-quantized top-k MoE
 * layer and the 2:4-sparse W4A16 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this library.  It shares no
 * code, header, table or constant with the GPU library, and it never sees a
 * packed weight layout: it reads the canonical logical tensors produced by the
 * seeded generator (integer codes, scales, group indices, keep positions).
 *
 * Arithmetic: every 16-bit input value arrives as the float32 that holds it
 * exactly.  Dequantisation is code * scale in float32 (exact: a code of at most
 * 8 bits times a 16-bit float needs at most 19 significand bits).  Every sum is
 * accumulated in double, in ascending index order; nothing is blocked, fused or
 * reordered.
 *
 * Passages followed (the pages print no formula; each step is the plain
 * definition of what the threads describe):
 *  - "[Kernel] W8A16 Int8 inside FusedMoE" (vLLM PR 7415), opening
 *    description: symmetric per-column, per-expert int8 weights, cast to the
 *    activation type and multiplied by their scale before the matmul.
 *  - "Marlin moe integration" (nm-vllm PR 266), opening description and the
 *    review thread: 4-bit GPTQ weights with group-128 scales, with and without
 *    act-order; the token sort that pads each expert's tokens to blocks of 16.
 *  - "Add GPTQ Marlin 2:4 sparse structured support" (vLLM PR 4790), opening
 *    description: 2:4 structured sparsity, 4-bit values, group size 128.
 *  - "[Kernel] W8A16 Int8 inside FusedMoE", opening description and its
 *    "How to convert models to ExpertsInt8?" answer: the int8 weights and
 *    their scales are produced from the 16-bit checkpoint when the model loads
 *    (orc_quant_w8).
 * The router (softmax + top-k), SiLU-and-mul between the two projections and
 * the top-k-weighted sum are the standard fused-MoE steps those threads plug
 * their kernels into; the pages name them only through the fused_moe
 * interface, so the plain readings used here are listed in the design notes.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_EXPORT __attribute__((visibility("default")))

/* flag an argument error from inside a parallel loop */
#define SET_BAD(flag)                 \
    do {                              \
        _Pragma("omp atomic write")   \
        (flag) = 1;                   \
    } while (0)

/* ------------------------------------------------------------------------ */
/* Router: softmax over the expert logits, keep the top k.                   */
/* ------------------------------------------------------------------------ */
/*
 * For each token m: choose k experts by repeated arg-max over the experts not
 * yet chosen; a strictly larger logit wins, so equal logits go to the lower
 * expert index.  Slot 0 holds the largest logit.  Selecting on logits equals
 * selecting on softmax probabilities (softmax is monotone).
 * Weights: with mu = the largest logit of the row,
 *   renormalize = 1: w_j = exp(l_j - mu) / sum_{j' < k} exp(l_j' - mu)
 *   renormalize = 0: w_j = exp(l_j - mu) / sum_{e < E} exp(l_e - mu)
 * computed in double and rounded once to float.
 * Returns 0, or -1 on bad arguments.
 */
ORC_EXPORT int orc_route(const float* logits, int64_t M, int E, int topk, int renormalize,
                         float* topk_weights, int32_t* topk_ids)
{
    if (M < 0 || E <= 0 || topk <= 0 || topk > E) return -1;
    char* chosen = (char*)malloc((size_t)E);
    double* ex = (double*)malloc(sizeof(double) * (size_t)topk);
    if (!chosen || !ex) { free(chosen); free(ex); return -1; }
    for (int64_t m = 0; m < M; ++m) {
        const float* l = logits + m * E;
        memset(chosen, 0, (size_t)E);
        for (int j = 0; j < topk; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (chosen[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e;
            }
            chosen[best] = 1;
            topk_ids[m * topk + j] = best;
        }
        const double mu = (double)l[topk_ids[m * topk]];
        double denom = 0.0;
        for (int j = 0; j < topk; ++j) {
            ex[j] = exp((double)l[topk_ids[m * topk + j]] - mu);
            if (renormalize) denom += ex[j];
        }
        if (!renormalize)
            for (int e = 0; e < E; ++e) denom += exp((double)l[e] - mu);
        for (int j = 0; j < topk; ++j) topk_weights[m * topk + j] = (float)(ex[j] / denom);
    }
    free(chosen);
    free(ex);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Token sort and pad per expert (moe_align_block_size).                      */
/* ------------------------------------------------------------------------ */
/*
 * The flattened (token, slot) index is i = m * topk + j, its expert e_i.
 *   c_e = number of i with e_i = e
 *   p_e = ceil(c_e / BS) * BS         (an expert with no token gets no block)
 *   o_e = sum_{e' < e} p_e'
 *   sorted_token_ids[o_e + r] = the r-th such i in ascending order, r < c_e;
 *   the pad slots [o_e + c_e, o_e + p_e) and everything from sum p_e up to the
 *   capacity hold the sentinel T = M * topk;
 *   expert_ids[b] = e for every block b of expert e's segment, -1 past the end;
 *   *num_tokens_post_padded = sum_e p_e.
 * Capacity: the largest possible sum_e p_e, T + min(E, T) * (BS - 1), rounded
 * up to a multiple of BS.
 */
ORC_EXPORT int64_t orc_align_capacity(int64_t T, int E, int BS)
{
    if (T < 0 || E <= 0 || BS <= 0) return -1;
    int64_t nz = T < (int64_t)E ? T : (int64_t)E;
    int64_t cap = T + nz * (int64_t)(BS - 1);
    return (cap + BS - 1) / BS * BS;
}

ORC_EXPORT int orc_align(const int32_t* topk_ids, int64_t T, int E, int BS,
                         int32_t* sorted_token_ids, int32_t* expert_ids, int32_t* num_tokens_post_padded,
                         int64_t capacity)
{
    if (T < 0 || E <= 0 || BS <= 0 || capacity < orc_align_capacity(T, E, BS) || capacity % BS) return -1;
    int64_t* count = (int64_t*)calloc((size_t)E, sizeof(int64_t));
    int64_t* offset = (int64_t*)calloc((size_t)E, sizeof(int64_t));
    int64_t* cursor = (int64_t*)calloc((size_t)E, sizeof(int64_t));
    if (!count || !offset || !cursor) { free(count); free(offset); free(cursor); return -1; }
    for (int64_t i = 0; i < T; ++i) {
        int32_t e = topk_ids[i];
        if (e < 0 || e >= E) { free(count); free(offset); free(cursor); return -1; }
        count[e] += 1;
    }
    int64_t total = 0;
    for (int e = 0; e < E; ++e) {
        offset[e] = total;
        total += (count[e] + BS - 1) / BS * BS;
    }
    for (int64_t p = 0; p < capacity; ++p) sorted_token_ids[p] = (int32_t)T;
    for (int64_t b = 0; b < capacity / BS; ++b) expert_ids[b] = -1;
    for (int e = 0; e < E; ++e) cursor[e] = offset[e];
    for (int64_t i = 0; i < T; ++i) sorted_token_ids[cursor[topk_ids[i]]++] = (int32_t)i;
    for (int e = 0; e < E; ++e) {
        int64_t p_e = (count[e] + BS - 1) / BS * BS;
        for (int64_t b = offset[e] / BS; b < (offset[e] + p_e) / BS; ++b) expert_ids[b] = e;
    }
    *num_tokens_post_padded = (int32_t)total;
    free(count);
    free(offset);
    free(cursor);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Weight-only dequantisation.                                               */
/* ------------------------------------------------------------------------ */
/*
 * A quantised weight matrix of one expert is W[r, k] = q[r, k] * s[g(k), r]
 * for output row r and input channel k, with q the integer code and s the
 * scale of input-channel group g(k).  g(k) = g_idx[k] when act-order is used
 * (channels quantised in a permuted order), otherwise k / (k_in / G) for G
 * groups (G = 1: one scale per output column, the per-column case).
 */
static inline int group_of(const int32_t* g_idx, int k, int k_in, int G)
{
    return g_idx ? g_idx[k] : k / (k_in / G);
}

static inline float dequant(int8_t q, float s)
{
    return (float)q * s; /* exact in float32 */
}

/* y[r] = sum_k x[k] * W[r, k], accumulated in double in ascending k */
static double dot_dequant(const float* x, const int8_t* q_row, const float* s_e, const int32_t* g_e,
                          int r, int n_out, int k_in, int G)
{
    double acc = 0.0;
    for (int k = 0; k < k_in; ++k) {
        float w = dequant(q_row[k], s_e[(int64_t)group_of(g_e, k, k_in, G) * n_out + r]);
        acc += (double)x[k] * (double)w;
    }
    return acc;
}

static inline double silu(double a) { return a / (1.0 + exp(-a)); }

/* ------------------------------------------------------------------------ */
/* MoE layer, stage by stage.                                                */
/* ------------------------------------------------------------------------ */
/*
 * Row set: rows[0..nrows) are the tokens to evaluate (NULL: all M tokens).
 * Per evaluated (token m, slot j), r = row_index * topk + j, e = topk_ids[m,j]:
 *   gu[r, n]   = sum_k x[m,k] * W1[e, n, k]          n < 2N (gate rows [0,N),
 *                                                     up rows [N,2N))
 *   h[r, n]    = silu(gu[r, n]) * gu[r, N + n]       silu(a) = a / (1 + e^-a)
 *   y[r, c]    = sum_n h[r, n] * W2[e, c, n]
 *   out[row,c] = sum_j topk_weights[m,j] * y[row*topk + j, c]   (ascending j)
 * w1q [E,2N,K] int8, s1 [E,G1,2N], g1 [E,K] or NULL;
 * w2q [E,K,N] int8,  s2 [E,G2,K],  g2 [E,N] or NULL.
 */
ORC_EXPORT int orc_moe_up(int64_t M, int K, int N, int E, int topk,
                          const float* x, const int32_t* topk_ids,
                          const int8_t* w1q, const float* s1, const int32_t* g1, int G1,
                          const int64_t* rows, int64_t nrows,
                          double* gu /* [nrows*topk, 2N] or NULL */, double* h /* [nrows*topk, N] */)
{
    if (!rows) nrows = M;
    const int n_out = 2 * N;
    if (G1 <= 0 || K % G1) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int64_t rr = 0; rr < nrows; ++rr) {
        for (int j = 0; j < topk; ++j) {
            const int64_t m = rows ? rows[rr] : rr;
            if (m < 0 || m >= M) { SET_BAD(bad); continue; }
            const int e = topk_ids[m * topk + j];
            if (e < 0 || e >= E) { SET_BAD(bad); continue; }
            const int64_t r = rr * topk + j;
            const int8_t* q_e = w1q + (int64_t)e * n_out * K;
            const float* s_e = s1 + (int64_t)e * G1 * n_out;
            const int32_t* g_e = g1 ? g1 + (int64_t)e * K : NULL;
            const float* xm = x + m * K;
            for (int n = 0; n < N; ++n) {
                double gate = dot_dequant(xm, q_e + (int64_t)n * K, s_e, g_e, n, n_out, K, G1);
                double up = dot_dequant(xm, q_e + (int64_t)(N + n) * K, s_e, g_e, N + n, n_out, K, G1);
                if (gu) {
                    gu[r * n_out + n] = gate;
                    gu[r * n_out + N + n] = up;
                }
                h[r * N + n] = silu(gate) * up;
            }
        }
    }
    return bad ? -1 : 0;
}

ORC_EXPORT int orc_moe_down(int64_t M, int K, int N, int E, int topk,
                            const int32_t* topk_ids,
                            const int8_t* w2q, const float* s2, const int32_t* g2, int G2,
                            const int64_t* rows, int64_t nrows,
                            const double* h /* [nrows*topk, N] */, double* y /* [nrows*topk, K] */)
{
    if (!rows) nrows = M;
    if (G2 <= 0 || N % G2) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int64_t rr = 0; rr < nrows; ++rr) {
        for (int j = 0; j < topk; ++j) {
            const int64_t m = rows ? rows[rr] : rr;
            if (m < 0 || m >= M) { SET_BAD(bad); continue; }
            const int e = topk_ids[m * topk + j];
            if (e < 0 || e >= E) { SET_BAD(bad); continue; }
            const int64_t r = rr * topk + j;
            const int8_t* q_e = w2q + (int64_t)e * K * N;
            const float* s_e = s2 + (int64_t)e * G2 * K;
            const int32_t* g_e = g2 ? g2 + (int64_t)e * N : NULL;
            const double* hr = h + r * N;
            for (int c = 0; c < K; ++c) {
                const int8_t* q_row = q_e + (int64_t)c * N;
                double acc = 0.0;
                for (int n = 0; n < N; ++n) {
                    float w = dequant(q_row[n], s_e[(int64_t)group_of(g_e, n, N, G2) * K + c]);
                    acc += hr[n] * (double)w;
                }
                y[r * K + c] = acc;
            }
        }
    }
    return bad ? -1 : 0;
}

ORC_EXPORT int orc_moe_combine(int64_t M, int K, int topk, const float* topk_weights,
                               const int64_t* rows, int64_t nrows,
                               const double* y /* [nrows*topk, K] */, double* out /* [nrows, K] */)
{
    if (!rows) nrows = M;
    for (int64_t rr = 0; rr < nrows; ++rr) {
        const int64_t m = rows ? rows[rr] : rr;
        if (m < 0 || m >= M) return -1;
        for (int c = 0; c < K; ++c) {
            double acc = 0.0;
            for (int j = 0; j < topk; ++j)
                acc += (double)topk_weights[m * topk + j] * y[(rr * topk + j) * K + c];
            out[rr * K + c] = acc;
        }
    }
    return 0;
}

/* The whole layer for already-routed tokens: up -> down -> weighted sum. */
ORC_EXPORT int orc_moe_layer(int64_t M, int K, int N, int E, int topk,
                             const float* x, const float* topk_weights, const int32_t* topk_ids,
                             const int8_t* w1q, const float* s1, const int32_t* g1, int G1,
                             const int8_t* w2q, const float* s2, const int32_t* g2, int G2,
                             const int64_t* rows, int64_t nrows,
                             double* gu, double* h, double* y, double* out)
{
    if (!rows) nrows = M;
    double* h_own = NULL;
    double* y_own = NULL;
    if (!h) h = h_own = (double*)malloc(sizeof(double) * (size_t)(nrows * topk) * (size_t)N);
    if (!y) y = y_own = (double*)malloc(sizeof(double) * (size_t)(nrows * topk) * (size_t)K);
    int rc = (!h || !y) ? -1 : 0;
    if (!rc) rc = orc_moe_up(M, K, N, E, topk, x, topk_ids, w1q, s1, g1, G1, rows, nrows, gu, h);
    if (!rc) rc = orc_moe_down(M, K, N, E, topk, topk_ids, w2q, s2, g2, G2, rows, nrows, h, y);
    if (!rc) rc = orc_moe_combine(M, K, topk, topk_weights, rows, nrows, y, out);
    free(h_own);
    free(y_own);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* 2:4-sparse W4A16 linear layer.                                            */
/* ------------------------------------------------------------------------ */
/*
 * W [N, K] keeps 2 of every 4 consecutive input channels.  Kept code t of
 * group b in row n sits at channel k = 4b + idx[n, 2b+t] with value
 * vals[n, 2b+t] * s[k / gs, n]; every other channel of the group is zero.
 *   y[m, n] = sum over kept k of x[m, k] * W[n, k]
 * (the same as the dense product with zeros at the pruned positions).
 * vals, idx [N, K/2]; s [K/gs, N] (gs = K: one scale per output column).
 */
ORC_EXPORT int orc_sparse24(int64_t M, int K, int N, const float* x,
                            const int8_t* vals, const uint8_t* idx, const float* s, int gs,
                            const int64_t* rows, int64_t nrows, double* y /* [nrows, N] */)
{
    if (!rows) nrows = M;
    if (K % 4 || gs <= 0 || K % gs) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int64_t rr = 0; rr < nrows; ++rr) {
        for (int n = 0; n < N; ++n) {
            const int64_t m = rows ? rows[rr] : rr;
            if (m < 0 || m >= M) { SET_BAD(bad); continue; }
            const float* xm = x + m * K;
            double acc = 0.0;
            for (int b = 0; b < K / 4; ++b) {
                for (int t = 0; t < 2; ++t) {
                    const int64_t v = (int64_t)n * (K / 2) + 2 * b + t;
                    if (idx[v] > 3) { SET_BAD(bad); continue; }
                    const int k = 4 * b + idx[v];
                    float w = dequant(vals[v], s[(int64_t)(k / gs) * N + n]);
                    acc += (double)xm[k] * (double)w;
                }
            }
            y[rr * N + n] = acc;
        }
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* ExpertsInt8 quantization at load time ("[Kernel] W8A16 Int8 inside        */
/* FusedMoE", opening description: symmetric per-column per-expert int8,     */
/* scales extracted at startup).  The pages state no formula or rounding;     */
/* the plain reading: per row (one expert's output column) of k weights,      */
/*   s32 = max_k |w| / 127           (float32, one correctly rounded divide)  */
/*   s   = s32 rounded to the 16-bit activation type, nearest-even (stored)   */
/*   q_k = w_k / s (float32 divide) rounded half-to-even, clamped to +-127    */
/* so that q * s, the weight the GEMM uses, is the nearest int8 multiple of   */
/* the stored scale; a row whose stored scale is 0 gets q = 0.                */
/* ------------------------------------------------------------------------ */

/* nearest value with p significant bits and minimum exponent emin (the
 * subnormal step is 2^(emin - p + 1)), ties to even; |x| beyond the largest
 * finite value of the format becomes infinite.  Double arithmetic is exact
 * here: x is a float32, the step a power of two. */
static double round_sig(double x, int p, int emin, double maxv)
{
    if (x == 0.0 || !isfinite(x)) return x;
    int e = ilogb(x);
    if (e < emin) e = emin;
    const double step = ldexp(1.0, e - (p - 1));
    double r = nearbyint(x / step) * step; /* default rounding mode: nearest-even */
    if (fabs(r) > maxv) r = copysign(INFINITY, x);
    return r;
}
static float round_bf16(float x) { return (float)round_sig(x, 8, -126, 0x1.fep127); }
static float round_f16(float x) { return (float)round_sig(x, 11, -14, 65504.0); }

ORC_EXPORT int orc_quant_w8(int64_t rows, int k, const float* w, int bf16, int8_t* q, float* s)
{
    if (rows < 0 || k <= 0) return -1;
    int bad = 0;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const float* wr = w + r * k;
        float mx = 0.0f;
        for (int i = 0; i < k; ++i) {
            if (!isfinite(wr[i])) { SET_BAD(bad); }
            const float a = fabsf(wr[i]);
            if (a > mx) mx = a;
        }
        const float s32 = mx / 127.0f;
        const float sr = bf16 ? round_bf16(s32) : round_f16(s32);
        s[r] = sr;
        for (int i = 0; i < k; ++i) {
            int v = 0;
            if (sr != 0.0f) {
                const float t = wr[i] / sr;
                v = (int)nearbyintf(t);
                if (v > 127) v = 127;
                if (v < -127) v = -127;
            }
            q[r * k + i] = (int8_t)v;
        }
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* FP8 W8A8 MoE layer: the comparison method of the ExpertsInt8 latency      */
/* table ("[Kernel] W8A16 Int8 inside FusedMoE", latency table rows "FP8     */
/* (MoE quant-only)", and the review thread naming it use_fp8_w8a8: weights  */
/* and activations both in 8-bit floating point).  The pages give no scheme;  */
/* the reading followed here:                                                 */
/*  - FP8 format: OCP E4M3 -- sign, 4 exponent bits with bias 7, 3 mantissa   */
/*    bits, no infinities, exponent 15 with mantissa 7 is NaN; largest finite */
/*    448, smallest normal 2^-6, subnormals (m/8) 2^-6.                       */
/*  - Weights: E4M3 codes, one float32 scale per expert and output column:    */
/*    W[e, r, k] = dec(c[e, r, k]) * sw[e, r].                               */
/*  - Activations: one static float32 scale per tensor (a1 for the layer      */
/*    input, a2 for the intermediate H), quantised as                        */
/*    q = enc(v / a)  with v / a a float32 division, enc = nearest E4M3 value */
/*    after clamping to [-448, 448] (saturating), ties to the even mantissa,  */
/*    the sign kept on zero; dequantised as dec(q) * a.  H is rounded to      */
/*    float32 before its division (the kernel holds H in float32).            */
/*  - The layer is the W8A16 one with these dequantised operands: gate/up     */
/*    over dequantised x, SiLU(gate) * up, quantise H, down, weighted sum.    */
/* ------------------------------------------------------------------------ */
ORC_EXPORT double orc_e4m3_decode(uint8_t c)
{
    const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    const double v = e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* nearest E4M3 code to a finite v (saturating at +-448, ties to even) */
ORC_EXPORT uint8_t orc_e4m3_encode(double v)
{
    const uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs(v);
    if (a > 448.0) a = 448.0;
    /* 4 significant bits, exponents down to -6; exact in double (a is a
     * float32 value, the step a power of two); 448 is representable, so the
     * clamped value never rounds past it */
    const double r = round_sig(a, 4, -6, 448.0);
    if (r == 0.0) return sign;
    int e = ilogb(r);
    if (e < -6) return sign | (uint8_t)(r / ldexp(1.0, -9)); /* subnormal: r = m 2^-9 */
    const int m = (int)((r / ldexp(1.0, e) - 1.0) * 8.0);
    return sign | (uint8_t)((e + 7) << 3) | (uint8_t)m;
}

/* values of n codes */
ORC_EXPORT int orc_fp8_decode(int64_t n, const uint8_t* q, double* v)
{
    if (n < 0) return -1;
    for (int64_t i = 0; i < n; ++i) v[i] = orc_e4m3_decode(q[i]);
    return 0;
}

/* codes of v / scale (float32 division) for n values */
ORC_EXPORT int orc_fp8_quant(int64_t n, const float* v, float scale, uint8_t* q)
{
    if (n < 0 || !(scale > 0.0f)) return -1;
    for (int64_t i = 0; i < n; ++i) {
        if (!isfinite(v[i])) return -1;
        const float t = v[i] / scale;
        q[i] = orc_e4m3_encode((double)t);
    }
    return 0;
}

/*
 * The FP8 W8A8 layer for already-routed tokens (rows: evaluated tokens, NULL
 * for all M).  x [M,K] (float32 values of the 16-bit activations),
 * w1 [E,2N,K] and w2 [E,K,N] E4M3 codes, sw1 [E,2N], sw2 [E,K] float32.
 * Outputs per evaluated (token, slot) r: optionally gu [r, 2N] (the gate/up
 * projections of the quantised input), hq [r, N] (the codes of H); y [r, K]
 * unweighted down projections; out [row, K] the weighted sum (ascending j).
 */
ORC_EXPORT int orc_fp8_moe_layer(int64_t M, int K, int N, int E, int topk,
                                 const float* x, const float* topk_weights, const int32_t* topk_ids,
                                 const uint8_t* w1, const float* sw1, const uint8_t* w2, const float* sw2,
                                 float a1, float a2, const int64_t* rows, int64_t nrows,
                                 double* gu, uint8_t* hq, double* y_out, double* out)
{
    if (!rows) nrows = M;
    if (!(a1 > 0.0f) || !(a2 > 0.0f) || K <= 0 || N <= 0 || E <= 0 || topk <= 0) return -1;
    const int n_out = 2 * N;
    double* y = y_out ? y_out : (double*)malloc(sizeof(double) * (size_t)(nrows * topk) * (size_t)K);
    if (!y) return -1;
    double dec[256]; /* the value of every code, looked up in the loops below */
    for (int c = 0; c < 256; ++c) dec[c] = orc_e4m3_decode((uint8_t)c);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int64_t rr = 0; rr < nrows; ++rr) {
        for (int j = 0; j < topk; ++j) {
            const int64_t m = rows ? rows[rr] : rr;
            if (m < 0 || m >= M) { SET_BAD(bad); continue; }
            const int e = topk_ids[m * topk + j];
            if (e < 0 || e >= E) { SET_BAD(bad); continue; }
            const int64_t r = rr * topk + j;
            double* xd = (double*)malloc(sizeof(double) * (size_t)K);
            double* hd = (double*)malloc(sizeof(double) * (size_t)N);
            if (!xd || !hd) { free(xd); free(hd); SET_BAD(bad); continue; }
            /* the layer input, quantised and dequantised */
            for (int k = 0; k < K; ++k) {
                const float t = x[m * K + k] / a1;
                xd[k] = dec[orc_e4m3_encode((double)t)] * (double)a1;
            }
            const uint8_t* c1 = w1 + (int64_t)e * n_out * K;
            for (int n = 0; n < N; ++n) {
                double gate = 0.0, up = 0.0;
                for (int k = 0; k < K; ++k)
                    gate += xd[k] * (dec[c1[(int64_t)n * K + k]] * (double)sw1[(int64_t)e * n_out + n]);
                for (int k = 0; k < K; ++k)
                    up += xd[k] * (dec[c1[(int64_t)(N + n) * K + k]] * (double)sw1[(int64_t)e * n_out + N + n]);
                if (gu) {
                    gu[r * n_out + n] = gate;
                    gu[r * n_out + N + n] = up;
                }
                const double h = silu(gate) * up;
                const float t = (float)h / a2;
                const uint8_t c = orc_e4m3_encode((double)t);
                if (hq) hq[r * N + n] = c;
                hd[n] = dec[c] * (double)a2;
            }
            const uint8_t* c2 = w2 + (int64_t)e * K * N;
            for (int cc = 0; cc < K; ++cc) {
                double acc = 0.0;
                for (int n = 0; n < N; ++n)
                    acc += hd[n] * (dec[c2[(int64_t)cc * N + n]] * (double)sw2[(int64_t)e * K + cc]);
                y[r * K + cc] = acc;
            }
            free(xd);
            free(hd);
        }
    }
    int rc = bad ? -1 : 0;
    if (!rc) rc = orc_moe_combine(M, K, topk, topk_weights, rows, nrows, y, out);
    if (!y_out) free(y);
    return rc;
}

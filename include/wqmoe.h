/*
 * wqmoe.h -- C ABI of libwqmoe.so: the fused Mixture-of-Experts layer with
 * weight-only quantized experts, and the 2:4-sparse W4A16 linear layer, for
 * AMD Instinct MI355X (gfx950).
 *
 * Hot-path calls (asynchronous on the caller's HIP stream, no allocation, no
 * host synchronisation, no device-to-host read):
 *   moe_route             router softmax + top-k
 *   moe_align             token sort and pad per expert
 *   moe_route_align       both in one call (one kernel for small batches)
 *   moe_route_gate_up     route + sort + the GATE_UP GEMM (one kernel for the smallest batches)
 *   moe_w4a16_gemm        grouped GEMM, int4 GPTQ-style weights, fp16 activations
 *   moe_w8a16_gemm        grouped GEMM, int8 per-column weights, bf16/fp16 activations
 *   sparse24_w4a16_gemm   2:4-sparse int4 dense linear layer, fp16 activations
 *   sparse24_w8a16_gemm   the same with 8-bit kept codes
 *   moe_fp8_w8a8_gemm     grouped GEMM with FP8 (E4M3) weights and activations
 * Beside them: dense_w4a16_gemm / dense_w8a16_gemm (one quantized weight
 * matrix, the same kernels with one expert) and wq_quantize_w8 (the int8
 * weights and scales from a 16-bit checkpoint on the device, at load time).
 * Off the hot path (host memory in and out): the packers that turn canonical
 * quantized tensors into the device layout these kernels read.
 *
 * The hot path receives weights that are already quantized and just runs the
 * kernels; quantisation and repacking live outside it ("Marlin moe
 * integration", nm-vllm PR 266, review comments on what the hot-path function
 * should receive).
 *
 * Conventions
 *  - Pointers named d_* or documented "device" are device memory on the
 *    current HIP device; all others are host memory.  Every device pointer must
 *    be 16-byte aligned.  Row-major layouts throughout.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *  - Ownership: the caller allocates and frees everything, workspaces
 *    included (except for moe_w8a16_gemm_noalloc, whose workspace is a device
 *    array inside the library).  The library keeps no other state than a
 *    thread-local error text and that array's device address per GPU.
 *  - Errors: arguments are validated on the host before anything is launched.
 *    A failing call launches nothing and returns a non-zero status; the text of
 *    the last error on this thread is returned by wq_last_error().  No call
 *    aborts or throws across this boundary.
 *  - Activation dtype codes: WQ_F16 = IEEE half, WQ_BF16 = bfloat16.  Scales
 *    must be in the activation dtype (scales may be stored otherwise on disk;
 *    conversion belongs to loading, not the hot path -- "Marlin moe
 *    integration", review question on whether scales are guaranteed fp16).
 */
#ifndef WQMOE_H
#define WQMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int wq_status;
#define WQ_OK 0
#define WQ_ERR_INVALID 1      /* null pointer, bad size, capacity/workspace too small, misaligned */
#define WQ_ERR_UNSUPPORTED 2  /* a valid request the library does not implement (dtype, group size, shape) */
#define WQ_ERR_DEVICE 3       /* a device pointer that is not on the current device */
#define WQ_ERR_HIP 4          /* the HIP runtime reported an error at launch */

#define WQ_F16 0
#define WQ_BF16 1

/* Stages of the grouped GEMM (moe_w4a16_gemm / moe_w8a16_gemm). */
#define WQ_STAGE_GATE_UP 0 /* H = silu(A W_gate^T) * (A W_up^T), rows in sorted order       */
#define WQ_STAGE_DOWN 1    /* out[m] = sum_j w[m,j] (H W_down^T)[row of (m,j)]               */
#define WQ_STAGE_RAW 2     /* Z[i] = A[token of i] W^T in fp32, no epilogue (testing)       */

#define WQ_PACK_INTERLEAVE_GATE_UP 1 /* packer flag: n_out = 2N rows = [gate; up], fused stage */

int wq_version(void);
const char* wq_status_string(wq_status s);
const char* wq_last_error(void);

/* ------------------------------------------------------------------------ */
/* moe_route                                                                 */
/* ------------------------------------------------------------------------ */
/*
 * Router softmax and top-k, one token per row of `logits`.
 *   d_logits        device float [M, E], finite values
 *   d_topk_weights  device float [M, topk]  (out)
 *   d_topk_ids      device int32 [M, topk]  (out)
 * Slot order: larger logit first, equal logits -> lower expert index.
 * renormalize = 1: weights are the softmax of the k selected logits (they sum
 * to 1); renormalize = 0: the selected entries of the softmax over all E.
 * exp, sum and divide are evaluated in double and rounded once to float.
 * Limits: 1 <= E <= 1024, 1 <= topk <= min(E, 16), M >= 0 (M = 0 launches nothing).
 * (The fused_moe interface the pages' kernels plug into: "Marlin moe
 * integration", nm-vllm PR 266, review comment on the fused_moe interface.)
 */
wq_status moe_route(const float* d_logits, int M, int E, int topk, int renormalize,
                    float* d_topk_weights, int32_t* d_topk_ids, void* stream);

/* ------------------------------------------------------------------------ */
/* moe_align                                                                 */
/* ------------------------------------------------------------------------ */
/*
 * Sort the T = M*topk (token, slot) pairs by expert and pad each expert's run
 * to a multiple of block_size ("Marlin moe integration", nm-vllm PR 266,
 * review thread on moe_align_block_size_kernel and its hard-coded block of 16).
 * With i = m*topk + j and c_e the number of pairs routed to expert e:
 *   p_e = ceil(c_e / block_size) * block_size, o_e = sum_{e'<e} p_e'
 *   d_sorted_token_ids[o_e + r] = r-th i (ascending) with topk_ids[i] = e,
 *   pad slots and the tail up to `capacity` hold the sentinel T;
 *   d_expert_ids[b] = expert of block b, -1 for blocks past the end;
 *   *d_num_tokens_post_padded = sum_e p_e.
 * The result is unique (stable order), so it is reproducible bit for bit.
 *   d_topk_ids                  device int32 [T], values in [0, E)
 *   d_sorted_token_ids          device int32 [capacity]            (out)
 *   d_expert_ids                device int32 [capacity/block_size] (out)
 *   d_num_tokens_post_padded    device int32 [1]                   (out)
 *   capacity >= moe_align_capacity(M, topk, E, block_size), a multiple of block_size
 * Limits: 1 <= E <= 1024, block_size in {16, 32, 64, 128, 256}, T <= 2^24.
 * Ids outside [0, E) are not detected on the device: such pairs are dropped.
 */
size_t moe_align_capacity(int M, int topk, int E, int block_size);
wq_status moe_align(const int32_t* d_topk_ids, int M, int topk, int E, int block_size,
                    int32_t* d_sorted_token_ids, int32_t* d_expert_ids, int32_t* d_num_tokens_post_padded,
                    size_t capacity, void* stream);

/* ------------------------------------------------------------------------ */
/* moe_route_align                                                           */
/* ------------------------------------------------------------------------ */
/*
 * moe_route followed by moe_align in one call, with the same arguments and the
 * same outputs bit for bit.  Batches of at most 16 tokens (and 1024 pairs) run
 * as a single kernel that keeps the expert ids on chip between the two steps
 * (one launch instead of two on the latency-bound small-batch path); larger
 * batches run the two kernels.  Limits: those of both calls.
 */
wq_status moe_route_align(const float* d_logits, int M, int E, int topk, int renormalize, int block_size,
                          float* d_topk_weights, int32_t* d_topk_ids, int32_t* d_sorted_token_ids,
                          int32_t* d_expert_ids, int32_t* d_num_tokens_post_padded, size_t capacity,
                          void* stream);

/* ------------------------------------------------------------------------ */
/* Grouped GEMMs                                                             */
/* ------------------------------------------------------------------------ */
/*
 * One call runs one projection of every expert over the tokens routed to it,
 * with the weights dequantized in registers and fp32 accumulation:
 *  - int4: GPTQ-style symmetric codes in [-8, 7], one scale per group of 128
 *    input channels (or per output column, group_size = -1), optional
 *    act-order ("Marlin moe integration", nm-vllm PR 266, opening description
 *    and the end-to-end tests with and without act-order);
 *  - int8: symmetric per-expert, per-output-column codes, the weight is
 *    code * scale ("[Kernel] W8A16 Int8 inside FusedMoE", vLLM PR 7415,
 *    opening description).
 * Expert rows are those of d_sorted_token_ids (from moe_align with the same
 * block_size); block_size 64 or a multiple of 128 (with n_out a multiple of 128
 * and k_in a multiple of 64) selects the large-batch kernel, other blocks the
 * small-batch (decode) kernel.  The large-batch kernel addresses the
 * activation rows with 32-bit byte offsets: capacity * k_in * 2 bytes above
 * 4 GiB is rejected with WQ_ERR_UNSUPPORTED (nothing is launched).
 *
 * Stages (A is d_a, W the expert's packed weight of n_out rows, k_in columns):
 *  GATE_UP  d_a = x [M, k_in]; W = w1 packed with WQ_PACK_INTERLEAVE_GATE_UP,
 *           n_out = 2N.  d_out = H [capacity, N] in act dtype, row p of the
 *           sorted order: H[p, n] = silu(g) * u with g, u the gate/up outputs
 *           of row n for the token of sorted_token_ids[p]; pad rows are 0.
 *           With act-order, d_k_perm is the permutation the packer returned
 *           and the workspace holds the permuted activations.
 *  DOWN     d_a = H [capacity, k_in] from GATE_UP (k_in = N); W = w2, n_out =
 *           hidden size.  d_out = out [M, n_out] act dtype:
 *           out[m, c] = sum_{j<topk} topk_weights[m,j] * (H W^T)[p(m,j), c],
 *           summed in fp32 and rounded once.  Needs a workspace for the
 *           per-pair outputs: fp32 [M*topk, n_out], times 2 or 4 when the
 *           large-batch kernel splits k_in to fill the GPU (small M*topk *
 *           n_out); the slices are added in a fixed order, so results do not
 *           vary from run to run.  A large-batch DOWN that does not split
 *           k_in stores each pair's weighted row rounded once to the act
 *           dtype (half that space used) before the fp32 sum.
 *  RAW      d_a = x [M, k_in]; d_out = fp32 [M*topk, n_out]:
 *           Z[i, r] = sum_k x[i/topk, k] * W_{expert(i)}[r, k], packed row order.
 * The workspace size comes from moe_gemm_workspace_bytes() with the call's
 * stage, M, topk, E, n_out, k_in, capacity and act-order flag; pass 0 / NULL if
 * it returns 0.  Calls sharing a workspace must be stream-ordered.
 */
typedef struct wq_moe_gemm_desc {
    size_t struct_size;          /* = sizeof(wq_moe_gemm_desc) */
    int stage;                   /* WQ_STAGE_* */
    int act_dtype;               /* WQ_F16 or WQ_BF16 */
    const void* d_a;
    int M, topk, E, n_out, k_in;
    const void* d_w_packed;      /* from wq_pack_w4 / wq_pack_w8 */
    const void* d_scales;        /* packed scales from the same packer call, act dtype */
    int group_size;              /* int4: 128 or -1; int8: -1 */
    const int32_t* d_k_perm;     /* int4 act-order GATE_UP/RAW: [E, k_in], else NULL */
    const int32_t* d_sorted_token_ids;
    const int32_t* d_expert_ids;
    const int32_t* d_num_tokens_post_padded;
    size_t capacity;
    int block_size;
    const float* d_topk_weights; /* DOWN only: [M, topk] */
    void* d_out;
    void* d_workspace;
    size_t workspace_bytes;
} wq_moe_gemm_desc;

size_t moe_gemm_workspace_bytes(int stage, int M, int topk, int E, int n_out, int k_in, size_t capacity,
                                int act_order);
wq_status moe_w4a16_gemm(const wq_moe_gemm_desc* d, void* stream);
wq_status moe_w8a16_gemm(const wq_moe_gemm_desc* d, void* stream);

/*
 * moe_route_gate_up: moe_route_align followed by the GATE_UP stage of
 * moe_w4a16_gemm (wbits = 4) or moe_w8a16_gemm (wbits = 8), in one call.  For
 * batches of at most 16 (token, slot) pairs over at most 64 experts, blocks of
 * 16 or 32 rows, a capacity of at most 1024 rows and no act-order permutation,
 * it is one launch: every workgroup of the small-batch GEMM ranks and sorts the
 * batch itself (the decode step's route -> sort -> gate/up chain of "Marlin moe
 * integration", nm-vllm PR 266, with the fused_moe interface of its review
 * thread).  With act-order (int4 with d_k_perm): one token (within the
 * limits above, n_out a multiple of 64, k_in at most 16384 and a multiple of
 * 8) is also one launch, each workgroup gathering the token's row in its
 * expert's channel order into LDS; for at most 16 tokens, 64 pairs, 64 experts
 * and a capacity of at most 1024 rows, the routing launch also gathers the
 * permuted activation rows into the workspace, one launch fewer than the two
 * calls.  Otherwise it runs the two calls' launches in order.  The outputs are
 * those of the two calls, bit for bit.
 *   d_logits [M, E] float32, renormalize: as moe_route_align
 *   d_topk_weights [M, topk] float32, d_topk_ids [M, topk] int32: written
 *   d: a GATE_UP descriptor (stage WQ_STAGE_GATE_UP) whose d_sorted_token_ids,
 *      d_expert_ids (capacity / block_size) and d_num_tokens_post_padded are
 *      written here (cast away const: they are outputs of this call), with
 *      capacity >= moe_align_capacity(M, topk, E, block_size) and topk <= 16;
 *      every other field as for the GEMM call
 * Errors: those of moe_route_align and of the GEMM call; WQ_ERR_INVALID for
 * another stage or wbits.  M = 0 writes the empty sort and launches no GEMM.
 */
wq_status moe_route_gate_up(const float* d_logits, int renormalize, float* d_topk_weights, int32_t* d_topk_ids,
                            const wq_moe_gemm_desc* d, int wbits, void* stream);

/*
 * moe_w8a16_gemm_noalloc -- for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): moe_w8a16_gemm with the same descriptor, kernels and results,
 * whose workspace is a device array inside the library instead of the
 * caller's buffer.  d->d_workspace must be NULL and d->workspace_bytes 0; the
 * caller still passes every input and output.
 *  - The array holds WQ_NOALLOC_SCRATCH_BYTES (64 MiB) on every GPU the
 *    library is loaded on, until the process ends.  A call whose
 *    moe_gemm_workspace_bytes() exceeds it returns WQ_ERR_UNSUPPORTED and
 *    launches nothing (64 MiB covers the DOWN stage of the Mixtral-8x7B shape
 *    up to 512 tokens and of the DeepSeek-V2 shape up to 512 tokens; GATE_UP
 *    and RAW of int8 weights need none).
 *  - No hipMalloc, hipFree or other allocation, no memset: the DOWN stage
 *    writes every scratch element it later reads.
 *  - All calls on one GPU share its array: calls that overlap in time on one
 *    GPU (different streams, or host threads without stream ordering) race on
 *    it.  Calls on one stream are ordered and safe.
 */
#define WQ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
wq_status moe_w8a16_gemm_noalloc(const wq_moe_gemm_desc* d, void* stream);

/* ------------------------------------------------------------------------ */
/* FP8 W8A8 grouped GEMM                                                     */
/* ------------------------------------------------------------------------ */
/*
 * The comparison method of the ExpertsInt8 latency table ("[Kernel] W8A16
 * Int8 inside FusedMoE", vLLM PR 7415: rows "FP8 (MoE quant-only)", and the
 * review thread naming it use_fp8_w8a8): weights and activations both in OCP
 * FP8 E4M3 (no infinities, 0x7F / 0xFF = NaN, largest finite 448), one float32
 * weight scale per expert and output column, one static float32 scale per
 * activation tensor (a1 for the layer input, a2 for H).  A value v is
 * quantised to the E4M3 code nearest to v / a (float32 division) after
 * clamping to +-448, ties to even.  Same descriptor as moe_w8a16_gemm, read
 * as follows:
 *  GATE_UP  d_a = x [M, k_in] in act_dtype, quantised with in_scale = a1 into
 *           the workspace; W = wq_pack_fp8 output with
 *           WQ_PACK_INTERLEAVE_GATE_UP, n_out = 2N; d_out = H codes uint8
 *           [capacity, N]: H[p, n] = code of silu(g) * u / out_scale (out_scale
 *           = a2) with g, u = in_scale * scale[row] * (x codes . weight codes),
 *           pad rows code 0.
 *  DOWN     d_a = H codes uint8 [capacity, k_in] from GATE_UP, in_scale = a2;
 *           d_out = out [M, n_out] act_dtype, the routed-weight sum of
 *           in_scale * scale[c] * (H codes . weight codes) in ascending slot
 *           order, fp32, rounded once; out_scale unused.
 *  RAW      d_a = x as for GATE_UP; d_out = fp32 [M*topk, n_out] (testing).
 *  d_scales float32 [E, n_out] from wq_pack_fp8 (packed row order);
 *  group_size -1; d_k_perm NULL; in_scale (and for GATE_UP out_scale) finite
 *  and > 0; the workspace (moe_fp8_gemm_workspace_bytes) is scratch for the
 *  x codes (GATE_UP / RAW) or the fp32 per-pair rows of DOWN.  One token
 *  (M == 1) on the small-batch kernel: GATE_UP quantises x inside the GEMM
 *  (k_in <= 32768), and DOWN with top-k <= 4 and k_in >= 4096 adds the
 *  top-k rows inside the GEMM (the H code rows in LDS, topk * (k_in + 16)
 *  bytes <= 128 KiB); neither then uses the workspace.
 * Blocks of 64 or a multiple of 128 (n_out % 128 == 0) take the large-batch
 * kernel (v_mfma_scale_f32_16x16x128_f8f6f4, token rows in LDS), which
 * refuses more than 4 GiB of activation codes; other blocks the small-batch
 * kernel.  Limits: k_in % 128 == 0, n_out % 16 (32 for GATE_UP) == 0.
 */
size_t moe_fp8_gemm_workspace_bytes(int stage, int M, int topk, int E, int n_out, int k_in);
wq_status moe_fp8_w8a8_gemm(const wq_moe_gemm_desc* d, float in_scale, float out_scale, void* stream);

/* ------------------------------------------------------------------------ */
/* 2:4-sparse W4A16 linear layer                                             */
/* ------------------------------------------------------------------------ */
/*
 * y[m, n] = sum_k x[m, k] W[n, k] with W [N, K] keeping 2 of every 4
 * consecutive input channels, int4 codes in [-8, 7] and one fp16 scale per
 * group of 128 input channels, or per output column with group_size = -1
 * ("Add GPTQ Marlin 2:4 sparse structured support", vLLM PR 4790, opening
 * description: group size 128 or -1 (channel-wise), 4-bit).
 *   d_x [M, K] fp16, d_y [M, N] fp16 (fp32 accumulation, rounded once)
 *   d_vals, d_meta, d_scales: from wq_pack_sparse24 with the same group_size
 * Limits: K % 256 == 0, N % 16 == 0, group_size 128 or -1, act_dtype == WQ_F16.
 * sparse24_w8a16_gemm: the same with 8-bit kept codes in [-128, 127] (the
 * pages' 8-bit variant of the 2:4 support), packed with bits = 8.
 */
wq_status sparse24_w8a16_gemm(const void* d_x, int M, int K, int N, const void* d_vals, const void* d_meta,
                              const void* d_scales, int group_size, void* d_y, int act_dtype, void* stream);
wq_status sparse24_w4a16_gemm(const void* d_x, int M, int K, int N, const void* d_vals, const void* d_meta,
                              const void* d_scales, int group_size, void* d_y, int act_dtype, void* stream);

/* ------------------------------------------------------------------------ */
/* Dense single-expert W4A16 / W8A16 linear layer                            */
/* ------------------------------------------------------------------------ */
/*
 * y[m, n] = sum_k x[m, k] W[n, k] for one weight matrix W [N, K] (the dense
 * GPTQ-Marlin case the MoE kernel was derived from -- "Marlin moe
 * integration", nm-vllm PR 266, review thread: the MoE file compared against
 * csrc/quantization/gptq_marlin/gptq_marlin.cu -- and the GEMV/GEMM mix picked
 * by batch-size heuristics of "[WIP] AWQ Faster Kernels", vLLM issue 3289).
 * 1..128 rows without act-order run one small-batch kernel (GEMV-like up to 2
 * rows, then token tiles of 16, 32 or 64 rows shared by 8 weight tiles);
 * beyond that (or with act-order) the grouped GEMM of this library with one
 * expert and top-1: up to 24 rows the small-batch kernel, up to 192 the
 * large-batch kernel with 64-row tiles, above that 128-row tiles; fp32
 * accumulation, rounded once to the activation type.
 *   d_x [M, K] act dtype; d_y [M, N] act dtype
 *   d_w_packed, d_scales: wq_pack_w4 / wq_pack_w8 output for E = 1, n_out = N,
 *     k_in = K (no gate/up interleave); int4 group_size 128 or -1, int8 -1
 *   d_k_perm: int4 act-order permutation from wq_pack_w4 ([1, K]) or NULL
 *   d_workspace: dense_gemm_workspace_bytes(M, K, N, act_order) bytes, 256-byte
 *     aligned (the routing arrays, the act-order gather, fp32 partial sums);
 *     0 bytes (NULL allowed) for 1..128 rows without act-order: one
 *     small-batch kernel (1..2 rows staged in LDS whole when they fit 96 KiB,
 *     else the tokens of each K chunk staged in LDS and shared by the 8
 *     weight tiles of a workgroup)
 * Limits: int4 K % 128 == 0 and fp16 activations; int8 K % 64 == 0; N % 16 ==
 * 0; above 24 rows (large-batch kernel) at most 4 GiB of activation rows
 * including the block padding (else WQ_ERR_UNSUPPORTED).  Asynchronous on `stream`; calls sharing a workspace must be
 * stream-ordered.
 */
size_t dense_gemm_workspace_bytes(int M, int K, int N, int act_order);
wq_status dense_w4a16_gemm(const void* d_x, int M, int K, int N, const void* d_w_packed, const void* d_scales,
                           int group_size, const int32_t* d_k_perm, void* d_y, int act_dtype, void* d_workspace,
                           size_t workspace_bytes, void* stream);
wq_status dense_w8a16_gemm(const void* d_x, int M, int K, int N, const void* d_w_packed, const void* d_scales,
                           void* d_y, int act_dtype, void* d_workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* ExpertsInt8 quantization at load time                                     */
/* ------------------------------------------------------------------------ */
/*
 * Produces the int8 weights and per-column scales of the W8A16 path from the
 * 16-bit checkpoint on the GPU ("[Kernel] W8A16 Int8 inside FusedMoE", vLLM
 * PR 7415, opening description: symmetric per-column per-expert int8 with
 * scales extracted at startup; its "How to convert models to ExpertsInt8?"
 * answer: quantization on the fly).  For each of `rows` rows of k weights
 * (row = one expert's output column, rows = E * n_out):
 *   s = round_to_dtype(max_k |w| / 127)      float32 division, nearest-even
 *   q = clamp(round_half_even(w / s), -127, 127), float32 division; q = 0
 *       where s == 0
 *   d_w      [rows, k] 16-bit (dtype: WQ_BF16 or WQ_F16), 16-byte aligned
 *   d_q      int8 [rows, k], 8-byte aligned: the canonical codes wq_pack_w8
 *            takes (copied to host)
 *   d_scales uint16 [rows]: the dtype's bit patterns, i.e. the [E, 1, n_out]
 *            scales wq_pack_w8 takes
 * Limits: k % 8 == 0; finite inputs (NaN or infinity give unspecified codes).
 * Device memory, all of it owned by the caller; asynchronous on `stream`.
 */
wq_status wq_quantize_w8(const void* d_w, int64_t rows, int k, int dtype, int8_t* d_q, uint16_t* d_scales,
                         void* stream);

/* ------------------------------------------------------------------------ */
/* Offline packers (host memory; not on the hot path)                        */
/* ------------------------------------------------------------------------ */
/*
 * Canonical inputs (per expert e, row r of n_out, input channel k of k_in):
 *   q        int8   [E, n_out, k_in]  codes (int4: [-8, 7]; int8: [-128, 127])
 *   scales   uint16 [E, G, n_out]     16-bit float bit patterns (G = k_in /
 *                                     group_size, or 1 for per-column scales)
 *   g_idx    int32  [E, k_in] or NULL act-order group of each input channel;
 *                                     every group must hold exactly group_size
 *                                     channels
 *   row_perm int32  [E, n_rows] or NULL  output-row order to produce: packed
 *                                     row p holds canonical row row_perm[e][p]
 *                                     (with WQ_PACK_INTERLEAVE_GATE_UP, n_rows
 *                                     = n_out/2 and the same order applies to
 *                                     the gate and the up half).  Used to fold
 *                                     the next projection's act-order input
 *                                     permutation into this one's outputs.
 * Outputs:
 *   packed        wq_pack_w4_bytes() / wq_pack_w8_bytes() bytes
 *   scales_packed uint16 [E, G, n_out] in packed row order
 *   k_perm        int32 [E, k_in] (only with g_idx): packed input position k'
 *                 holds canonical channel k_perm[e][k'] (stable sort by g_idx).
 *                 Pass it as d_k_perm to the GATE_UP stage; for a DOWN weight
 *                 pass it as row_perm when packing the GATE_UP weight instead.
 * Limits: n_out % 16 == 0 (% 32 with interleave), int4 k_in % 128 == 0, int8
 * k_in % 64 == 0.
 */
size_t wq_pack_w4_bytes(int E, int n_out, int k_in);
size_t wq_pack_w8_bytes(int E, int n_out, int k_in);
wq_status wq_pack_w4(int E, int n_out, int k_in, const int8_t* q, const uint16_t* scales, int group_size,
                     const int32_t* g_idx, const int32_t* row_perm, int flags,
                     void* packed, uint16_t* scales_packed, int32_t* k_perm);
wq_status wq_pack_w8(int E, int n_out, int k_in, const int8_t* q, const uint16_t* scales,
                     const int32_t* row_perm, int flags, void* packed, uint16_t* scales_packed);

/*
 * FP8 packer: codes uint8 [E, n_out, k_in] (E4M3, no NaN), scales float32
 * [E, n_out] -> packed (wq_pack_fp8_bytes: E * n_out * k_in bytes, tiles of 16
 * rows x 128 channels, 2 KiB each) and scales_packed float32 [E, n_out] in packed row
 * order; row_perm and flags as for wq_pack_w8.  Limits: n_out % 16 == 0 (% 32
 * with interleave), k_in % 128 == 0.
 */
size_t wq_pack_fp8_bytes(int E, int n_out, int k_in);
wq_status wq_pack_fp8(int E, int n_out, int k_in, const uint8_t* codes, const float* scales,
                      const int32_t* row_perm, int flags, void* packed, float* scales_packed);

/*
 * 2:4 sparse canonical input: vals int8 [N, K/2] (kept codes, in [-8, 7] for
 * bits = 4, any int8 for bits = 8; two per group of 4 along K, ascending
 * position), idx uint8 [N, K/2] (their positions 0..3 inside the group,
 * strictly ascending per pair), scales uint16 [G, N] with G = K/128
 * (group_size 128) or 1 (group_size -1).  Outputs: vals_packed
 * (wq_pack_sparse24_vals_bytes: N*K/4 bytes for 4-bit, N*K/2 for 8-bit),
 * meta_packed (wq_pack_sparse24_meta_bytes), scales_packed uint16 [G, N].
 */
size_t wq_pack_sparse24_vals_bytes(int N, int K, int bits);
size_t wq_pack_sparse24_meta_bytes(int N, int K);
wq_status wq_pack_sparse24(int N, int K, int bits, int group_size, const int8_t* vals, const uint8_t* idx,
                           const uint16_t* scales, void* vals_packed, void* meta_packed, uint16_t* scales_packed);

#ifdef __cplusplus
}
#endif
#endif /* WQMOE_H */

// launch.hpp -- internal launchers shared between the kernel translation units
// and the C ABI layer.  Arguments are validated by the caller (abi.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace wq {

constexpr int STAGE_GATE_UP = 0;
constexpr int STAGE_DOWN = 1;
constexpr int STAGE_RAW = 2;

// Packed weight geometry: tiles of 16 output rows; a chunk of one tile holds
// 64 lanes x 16 bytes = 1 KiB and spans KCHUNK input channels.
constexpr int TILE_ROWS = 16;
constexpr int CHUNK_BYTES = 1024;
template <int WBITS>
struct WFmt {
    static constexpr int KCHUNK = WBITS == 4 ? 128 : 64;
};

void launch_route(const float* logits, int M, int E, int topk, int renormalize, float* w, int32_t* ids,
                  hipStream_t s);
void launch_align(const int32_t* ids, int T, int E, int BS, int32_t* sorted, int32_t* expert_ids, int32_t* ntpp,
                  int cap, hipStream_t s);
// route + align in one kernel (batches of at most 16 tokens and 1024 pairs)
bool route_align_fused(int M, int topk);
void launch_route_align(const float* logits, int M, int E, int topk, int renormalize, float* w, int32_t* ids, int BS,
                        int32_t* sorted, int32_t* expert_ids, int32_t* ntpp, int cap, hipStream_t s);

struct GemmArgs {
    const uint16_t* a;        // activations (x, gathered x, or H), 16-bit
    const uint8_t* w;         // packed weights, all experts
    const uint16_t* s;        // packed scales, all experts
    const int32_t* sorted;    // sorted_token_ids
    const int32_t* expert_ids;
    const int32_t* ntpp;
    const float* topk_w;      // DOWN
    void* out;                // H (act) / Y (f32, or act with y_act) / Z (f32)
    int M, topk, E, n_out, k_in;
    int block_size;
    int groups;               // scale groups along k_in (1 = per column)
    int a_direct;             // 1: A row = sorted position; 0: A row = token of the pair
    int cap;
    int y_act;                // large-batch DOWN without a K split: Y rows in the activation type
};

// ---------------------------------------------------------------------------
// FP8 (OCP E4M3) W8A8 grouped GEMM.  Packed weights: per expert, tiles of 16
// output rows x 128 input channels = 2 KiB; lane l's 32-byte MFMA operand (row
// l % 16, channels [32 (l / 16), +32) of the chunk) is split in two 16-byte
// halves at bytes 16 l and 1024 + 16 l; one float32 scale per packed row.
// Activations are E4M3 codes (x quantised by launch_fp8_quant, H by the
// GATE_UP epilogue).
// ---------------------------------------------------------------------------
constexpr int FP8_KCHUNK = 128;
constexpr int FP8_CHUNK_BYTES = 2048;

struct Fp8GemmArgs {
    const uint8_t* a;         // E4M3 rows: quantised x (GATE_UP / RAW) or H (DOWN)
    const uint8_t* w;         // packed E4M3 weights, all experts
    const float* s;           // per-row weight scales [E, n_out] in packed row order
    const int32_t* sorted;
    const int32_t* expert_ids;
    const int32_t* ntpp;
    const float* topk_w;      // DOWN
    void* out;                // H codes (uint8) / Y or Z (f32)
    int M, topk, E, n_out, k_in;
    int block_size;
    int a_direct;             // 1: A row = sorted position (H); 0: A row = token of the pair (x)
    int cap;
    float in_scale;           // scale of the A operand's codes (a1 for x, a2 for H)
    float out_scale;          // GATE_UP: scale H is quantised with (a2)
    const uint16_t* x16;      // GATE_UP of one token: its 16-bit row, quantised in the kernel (a unused); else null
    int x_bf16;               // x16's type: 1 bf16, 0 fp16
};

// GATE_UP of one token on the small-batch kernel: x quantised inside the GEMM
// (its codes in LDS, k_in bytes), no quantisation launch
constexpr int FP8_FOLD_MAX_K = 32768;
bool fp8_fold_quant_supported(int stage, int M, int n_out, int k_in, int block_size);
// q[r, k] = E4M3 code of x[r, k] / scale (float32 division, clamped to +-448, nearest even)
void launch_fp8_quant(const uint16_t* x, int64_t rows, int k, bool bf16, float scale, uint8_t* q, hipStream_t s);
// grouped E4M3 GEMM, small-batch (weights streamed once per pass of token blocks) or
// large-batch (token tiles in LDS, 16x16x128 MFMAs); returns the K slices DOWN wrote
bool fp8_prefill_supported(int n_out, int k_in, int block_size);
int fp8_down_split(int T, int E, int n_out, int k_in, int block_size);
int launch_gemm_fp8(int stage, const Fp8GemmArgs& g, hipStream_t s);
// DOWN of one token with the top-k sum folded in: g.out is the [1, n_out]
// output row in the activation type, no fp32 rows and no combine launch
bool fp8_down_combine_supported(int M, int topk, int n_out, int k_in);
void launch_fp8_down_combine(bool bf16, const Fp8GemmArgs& g, hipStream_t s);

// small-batch path: one workgroup per (expert, 16 or 32 weight rows), split-K
// across its waves, all of the expert's 16-row token blocks per pass
void launch_gemm_decode(int wbits, bool bf16, int stage, const GemmArgs& g, hipStream_t s);

// The small-batch GATE_UP launch that routes and sorts the batch itself (one
// launch for moe_route_align + GATE_UP): the logits, the softmax mode and the
// routing arrays it writes (topk weights and ids, sorted_token_ids,
// expert_ids, num_tokens_post_padded; g.sorted / g.expert_ids / g.ntpp are
// not read).
struct RouteArgs {
    const float* logits = nullptr;
    int renormalize = 0;
    float* w_out = nullptr;
    int32_t* ids_out = nullptr;
    int32_t* sorted_out = nullptr;
    int32_t* expert_ids_out = nullptr;
    int32_t* ntpp_out = nullptr;
    const int32_t* perm = nullptr;  // act-order, one token: the experts' k_in permutations
};
constexpr int FR_MAX_PAIRS = 64;   // M * topk
constexpr int FR_MAX_CAP = 1024;   // capacity rows held in LDS
// routing, sort and the act-order gather (row p of the gathered activations
// a1 = x of sorted_token_ids[p]'s token permuted by its expert's perm) in one
// launch, for batches within route_gather_supported
bool route_gather_supported(int M, int topk, int E, int cap, int BS);
void launch_route_align_gather(const float* logits, int M, int E, int topk, int renormalize, float* w, int32_t* ids,
                               int BS, int32_t* sorted, int32_t* expert_ids, int32_t* ntpp, int cap,
                               const uint16_t* x, const int32_t* perm, int k_in, uint16_t* a1, hipStream_t s);
// up to 16 pairs over at most 64 experts, blocks of 16 or 32 rows
bool decode_route_supported(int stage, int M, int topk, int E, int cap, int block_size);
// the same launch for one token of an act-order (int4) layer: each workgroup
// gathers the token's row in its expert's channel order into LDS
constexpr int DECODE_AO_MAX_K = 16384;
bool decode_route_ao_supported(int M, int topk, int n_out, int k_in);
void launch_gemm_decode_route(int wbits, bool bf16, const GemmArgs& g, const RouteArgs& ra, hipStream_t s);
// batches of at most 4 tokens: one workgroup per (used block, 16 or 32 weight
// rows), the block's token rows staged in LDS (through the act-order
// permutation perm [E, k_in] when not NULL, GATE_UP / RAW only); DOWN in up
// to max_ks K slices (fp32 slab z of the output at out + z * M*topk*n_out).
// tiny_supported: whether it is the faster kernel for this call;
// tiny_down_slabs: the most K slices its DOWN stage can take (for the
// workspace); launch returns the number of K slices it wrote
bool tiny_supported(int wbits, int stage, int M, int k_in, int groups, int max_ks);
int tiny_down_slabs(int M, int k_in);
// DOWN of one token with the top-k sum folded in: writes the layer output row
// (activation type) directly
bool tiny_down_combine_supported(int wbits, int M, int topk, int n_out, int k_in);
void launch_tiny_down_combine(int wbits, bool bf16, const GemmArgs& g, uint16_t* out, hipStream_t s);
int launch_gemm_tiny(int wbits, bool bf16, int stage, const GemmArgs& g, const int32_t* perm, int max_ks,
                     hipStream_t s);
// large-batch path: 512, 256 or 128 weight rows (dequantized in registers) x
// 128 (or 64) token rows (staged in LDS)
bool prefill_supported(int n_out, int k_in, int block_size);
// the large-batch kernel addresses its activations (rows x k_in 16-bit values)
// with 32-bit byte offsets
bool prefill_fits(size_t rows, int k_in);
// K slices of the large-batch DOWN stage for T = M*topk rows over E experts in
// blocks of block_size rows (1, 2 or 4); the DOWN workspace holds that many
// fp32 slabs of T x n_out.  _max: the largest over the supported block sizes
int prefill_down_split(int T, int E, int n_out, int k_in, int block_size);
int prefill_down_split_max(int T, int E, int n_out, int k_in);
// returns the number of K slices (Y slabs) it wrote
int launch_gemm_prefill(int wbits, bool bf16, int stage, const GemmArgs& g, hipStream_t s);

// the routing arrays of a dense layer (E = 1, top-1): sorted = 0..M-1 then pad
// ids M up to cap, expert 0 per block, ntpp = M rounded up to BS, weights 1
void launch_identity_route(int M, int cap, int BS, int32_t* sorted, int32_t* expert_ids, int32_t* ntpp, float* w,
                           hipStream_t s);

// act-order: A1[p, k'] = x[token(p), perm[expert(p), k']] for sorted rows p
void launch_gather_perm(const uint16_t* x, const int32_t* perm, const int32_t* sorted, const int32_t* expert_ids,
                        const int32_t* ntpp, int M, int topk, int k_in, int block_size, int cap, uint16_t* a1,
                        hipStream_t s);
// out[m, c] = sum_j sum_z Y[z][m*topk + j, c] over top-k slots j and K slices z
// (ascending, fp32), rounded to act; slab z starts at y + z * M*topk*n
void launch_combine_act(const uint16_t* y, int M, int topk, int n, bool bf16, uint16_t* out, hipStream_t s);
void launch_combine(const float* y, int M, int topk, int n, int ksplit, bool bf16, uint16_t* out, hipStream_t s);

// 2:4-sparse linear with 4- or 8-bit kept codes; group_size 128 (scales
// [K/128, N]) or -1 (one scale per output column, [1, N])
void launch_sparse24(int bits, const uint16_t* x, int M, int K, int N, const uint8_t* vals, const uint8_t* meta,
                     const uint16_t* scales, int group_size, uint16_t* y, hipStream_t s);

// dense single-expert linear at 1..4 token rows (rows staged in LDS, at most 96 KiB)
bool dense_decode_supported(int M, int K);
void launch_dense_decode(int wbits, bool bf16, const uint16_t* x, int M, int K, int N, const uint8_t* w,
                         const uint16_t* s, int groups, uint16_t* y, hipStream_t st);

// ExpertsInt8 load-time quantizer: rows of k 16-bit weights -> int8 codes and
// one 16-bit scale per row
void launch_quant_w8(const uint16_t* w, int64_t rows, int k, bool bf16, int8_t* q, uint16_t* s, hipStream_t st);

}  // namespace wq

// abi.cpp -- the C ABI of libwqmoe.so (declared in include/wqmoe.h): argument
// validation, device checks, kernel dispatch, and the offline packers.
//
// Every entry point validates all sizes, pointers and formats on the host
// before the first HIP call, so a rejected call launches nothing and the
// validation itself runs (and is tested) on machines without a GPU.  Device
// pointers must live on the current device: a multi-device process that hands
// a kernel another device's buffer gets WQ_ERR_DEVICE instead of an illegal
// access (the failure reported for moe_align_block_size_kernel on a second
// device in "Marlin moe integration", nm-vllm PR 266, review thread).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "../../include/wqmoe.h"
#include "launch.hpp"

namespace {

thread_local std::string g_last_error;

wq_status fail(wq_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

wq_status ok() {
    g_last_error.clear();
    return WQ_OK;
}

#define WQ_REQUIRE(cond, st, ...)              \
    do {                                       \
        if (!(cond)) return fail(st, __VA_ARGS__); \
    } while (0)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// host-side pointer sanity (no HIP call): non-null and 16-byte aligned
wq_status check_ptr(const void* p, const char* name) {
    WQ_REQUIRE(p != nullptr, WQ_ERR_INVALID, "%s is NULL", name);
    WQ_REQUIRE(aligned16(p), WQ_ERR_INVALID, "%s is not 16-byte aligned", name);
    return WQ_OK;
}

// device check: the pointer is device (or managed) memory of the current device
wq_status check_dev(const void* p, const char* name) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return fail(WQ_ERR_HIP, "hipGetDevice failed");
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
        (void)hipGetLastError();
        return fail(WQ_ERR_DEVICE, "%s is not a HIP allocation", name);
    }
    if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)
        return fail(WQ_ERR_DEVICE, "%s is not device memory", name);
    if (attr.type == hipMemoryTypeDevice && attr.device != cur)
        return fail(WQ_ERR_DEVICE, "%s lives on device %d, current device is %d", name, attr.device, cur);
    return WQ_OK;
}

#define WQ_TRY(expr)                      \
    do {                                  \
        wq_status _st = (expr);           \
        if (_st != WQ_OK) return _st;     \
    } while (0)

wq_status after_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(WQ_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

// ---------------------------------------------------------------------------
// The no-allocation entry point's workspace: one file-scope device array per
// GPU, held from the library's load until the process ends.  Host code never
// uses the array's name as an address (on the host it names a stand-in):
// the device address comes from hipGetSymbolAddress, once per device with that
// device current, and is kept per device.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[WQ_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::atomic<void*> g_scratch_addr[MAX_DEVICES];
std::mutex g_scratch_mu;

// device address of the current device's scratch array
wq_status scratch_for_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return fail(WQ_ERR_HIP, "hipGetDevice failed");
    if (dev < 0 || dev >= MAX_DEVICES) return fail(WQ_ERR_UNSUPPORTED, "device %d >= %d", dev, MAX_DEVICES);
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || p == nullptr) {
                (void)hipGetLastError();
                return fail(WQ_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
            }
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return WQ_OK;
}

bool valid_block_size(int bs) { return bs == 16 || bs == 32 || bs == 64 || bs == 128 || bs == 256; }

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

constexpr int64_t MAX_PAIRS = 1 << 24;

template <class F>
void parallel_for(int n, F f) {
    unsigned hw = std::max(1u, std::min(32u, std::thread::hardware_concurrency()));
    int nt = std::min<int>(n, (int)hw);
    if (nt <= 1) {
        for (int i = 0; i < n; ++i) f(i);
        return;
    }
    std::vector<std::thread> th;
    for (int t = 0; t < nt; ++t)
        th.emplace_back([=]() {
            for (int i = t; i < n; i += nt) f(i);
        });
    for (auto& x : th) x.join();
}

}  // namespace

extern "C" {

int wq_version(void) { return 1; }

const char* wq_status_string(wq_status s) {
    switch (s) {
        case WQ_OK: return "ok";
        case WQ_ERR_INVALID: return "invalid argument";
        case WQ_ERR_UNSUPPORTED: return "unsupported";
        case WQ_ERR_DEVICE: return "wrong device";
        case WQ_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* wq_last_error(void) { return g_last_error.c_str(); }

// ---------------------------------------------------------------------------
size_t moe_align_capacity(int M, int topk, int E, int block_size) {
    if (M < 0 || topk <= 0 || E <= 0 || block_size <= 0) return 0;
    const int64_t T = (int64_t)M * topk;
    const int64_t nz = std::min<int64_t>(T, E);
    const int64_t cap = T + nz * (block_size - 1);
    return (size_t)((cap + block_size - 1) / block_size * block_size);
}

wq_status moe_route(const float* d_logits, int M, int E, int topk, int renormalize, float* d_topk_weights,
                    int32_t* d_topk_ids, void* stream) {
    try {
        WQ_REQUIRE(M >= 0, WQ_ERR_INVALID, "M = %d < 0", M);
        WQ_REQUIRE(E >= 1 && topk >= 1 && topk <= E, WQ_ERR_INVALID, "need 1 <= topk <= E (topk %d, E %d)", topk, E);
        WQ_REQUIRE(E <= 1024, WQ_ERR_UNSUPPORTED, "E = %d > 1024", E);
        WQ_REQUIRE(topk <= 16, WQ_ERR_UNSUPPORTED, "topk = %d > 16", topk);
        WQ_REQUIRE((int64_t)M * topk <= MAX_PAIRS, WQ_ERR_UNSUPPORTED, "M*topk > 2^24");
        if (M == 0) return ok();
        WQ_TRY(check_ptr(d_logits, "logits"));
        WQ_TRY(check_ptr(d_topk_weights, "topk_weights"));
        WQ_TRY(check_ptr(d_topk_ids, "topk_ids"));
        WQ_TRY(check_dev(d_logits, "logits"));
        WQ_TRY(check_dev(d_topk_weights, "topk_weights"));
        WQ_TRY(check_dev(d_topk_ids, "topk_ids"));
        wq::launch_route(d_logits, M, E, topk, renormalize ? 1 : 0, d_topk_weights, d_topk_ids,
                         (hipStream_t)stream);
        return after_launch("moe_route");
    } catch (...) {
        return fail(WQ_ERR_HIP, "moe_route: unexpected exception");
    }
}

wq_status moe_align(const int32_t* d_topk_ids, int M, int topk, int E, int block_size, int32_t* d_sorted_token_ids,
                    int32_t* d_expert_ids, int32_t* d_num_tokens_post_padded, size_t capacity, void* stream) {
    try {
        WQ_REQUIRE(M >= 0 && topk >= 1 && E >= 1, WQ_ERR_INVALID, "bad sizes M %d topk %d E %d", M, topk, E);
        WQ_REQUIRE(E <= 1024, WQ_ERR_UNSUPPORTED, "E = %d > 1024", E);
        WQ_REQUIRE(valid_block_size(block_size), WQ_ERR_UNSUPPORTED, "block_size %d not in {16,32,64,128,256}",
                   block_size);
        WQ_REQUIRE((int64_t)M * topk <= MAX_PAIRS, WQ_ERR_UNSUPPORTED, "M*topk > 2^24");
        const size_t need = moe_align_capacity(M, topk, E, block_size);
        WQ_REQUIRE(capacity >= need, WQ_ERR_INVALID, "capacity %zu < required %zu", capacity, need);
        WQ_REQUIRE(capacity % (size_t)block_size == 0, WQ_ERR_INVALID, "capacity not a multiple of block_size");
        WQ_REQUIRE(capacity <= (size_t)0x7fffffff, WQ_ERR_UNSUPPORTED, "capacity too large");
        if (M > 0) WQ_TRY(check_ptr(d_topk_ids, "topk_ids"));
        WQ_TRY(check_ptr(d_sorted_token_ids, "sorted_token_ids"));
        WQ_TRY(check_ptr(d_expert_ids, "expert_ids"));
        WQ_TRY(check_ptr(d_num_tokens_post_padded, "num_tokens_post_padded"));
        if (M > 0) WQ_TRY(check_dev(d_topk_ids, "topk_ids"));
        WQ_TRY(check_dev(d_sorted_token_ids, "sorted_token_ids"));
        WQ_TRY(check_dev(d_expert_ids, "expert_ids"));
        WQ_TRY(check_dev(d_num_tokens_post_padded, "num_tokens_post_padded"));
        wq::launch_align(d_topk_ids, M * topk, E, block_size, d_sorted_token_ids, d_expert_ids,
                         d_num_tokens_post_padded, (int)capacity, (hipStream_t)stream);
        return after_launch("moe_align");
    } catch (...) {
        return fail(WQ_ERR_HIP, "moe_align: unexpected exception");
    }
}

// the launches of moe_route_align (arguments already validated)
static wq_status launch_routing(const float* d_logits, int M, int E, int topk, int renormalize, int block_size,
                               float* d_topk_weights, int32_t* d_topk_ids, int32_t* d_sorted_token_ids,
                               int32_t* d_expert_ids, int32_t* d_num_tokens_post_padded, size_t capacity,
                               hipStream_t s, const char* who) {
    const int rn = renormalize ? 1 : 0;
    if (M > 0 && wq::route_align_fused(M, topk)) {
        wq::launch_route_align(d_logits, M, E, topk, rn, d_topk_weights, d_topk_ids, block_size, d_sorted_token_ids,
                               d_expert_ids, d_num_tokens_post_padded, (int)capacity, s);
    } else {
        if (M > 0) {
            wq::launch_route(d_logits, M, E, topk, rn, d_topk_weights, d_topk_ids, s);
            WQ_TRY(after_launch(who));
        }
        wq::launch_align(d_topk_ids, M * topk, E, block_size, d_sorted_token_ids, d_expert_ids,
                         d_num_tokens_post_padded, (int)capacity, s);
    }
    return after_launch(who);
}

wq_status moe_route_align(const float* d_logits, int M, int E, int topk, int renormalize, int block_size,
                          float* d_topk_weights, int32_t* d_topk_ids, int32_t* d_sorted_token_ids,
                          int32_t* d_expert_ids, int32_t* d_num_tokens_post_padded, size_t capacity, void* stream) {
    try {
        WQ_REQUIRE(M >= 0, WQ_ERR_INVALID, "M = %d < 0", M);
        WQ_REQUIRE(E >= 1 && topk >= 1 && topk <= E, WQ_ERR_INVALID, "need 1 <= topk <= E (topk %d, E %d)", topk, E);
        WQ_REQUIRE(E <= 1024, WQ_ERR_UNSUPPORTED, "E = %d > 1024", E);
        WQ_REQUIRE(topk <= 16, WQ_ERR_UNSUPPORTED, "topk = %d > 16", topk);
        WQ_REQUIRE(valid_block_size(block_size), WQ_ERR_UNSUPPORTED, "block_size %d not in {16,32,64,128,256}",
                   block_size);
        WQ_REQUIRE((int64_t)M * topk <= MAX_PAIRS, WQ_ERR_UNSUPPORTED, "M*topk > 2^24");
        const size_t need = moe_align_capacity(M, topk, E, block_size);
        WQ_REQUIRE(capacity >= need, WQ_ERR_INVALID, "capacity %zu < required %zu", capacity, need);
        WQ_REQUIRE(capacity % (size_t)block_size == 0, WQ_ERR_INVALID, "capacity not a multiple of block_size");
        WQ_REQUIRE(capacity <= (size_t)0x7fffffff, WQ_ERR_UNSUPPORTED, "capacity too large");
        if (M > 0) {
            WQ_TRY(check_ptr(d_logits, "logits"));
            WQ_TRY(check_ptr(d_topk_weights, "topk_weights"));
            WQ_TRY(check_ptr(d_topk_ids, "topk_ids"));
        }
        WQ_TRY(check_ptr(d_sorted_token_ids, "sorted_token_ids"));
        WQ_TRY(check_ptr(d_expert_ids, "expert_ids"));
        WQ_TRY(check_ptr(d_num_tokens_post_padded, "num_tokens_post_padded"));
        if (M > 0) {
            WQ_TRY(check_dev(d_logits, "logits"));
            WQ_TRY(check_dev(d_topk_weights, "topk_weights"));
            WQ_TRY(check_dev(d_topk_ids, "topk_ids"));
        }
        WQ_TRY(check_dev(d_sorted_token_ids, "sorted_token_ids"));
        WQ_TRY(check_dev(d_expert_ids, "expert_ids"));
        WQ_TRY(check_dev(d_num_tokens_post_padded, "num_tokens_post_padded"));
        return launch_routing(d_logits, M, E, topk, renormalize, block_size, d_topk_weights, d_topk_ids,
                              d_sorted_token_ids, d_expert_ids, d_num_tokens_post_padded, capacity,
                              (hipStream_t)stream, "moe_route_align");
    } catch (...) {
        return fail(WQ_ERR_HIP, "moe_route_align: unexpected exception");
    }
}

// ---------------------------------------------------------------------------
// fp32 slabs of M*topk x n_out the DOWN stage may write (one per K slice)
static int down_slabs(int M, int topk, int E, int n_out, int k_in) {
    return std::max(wq::prefill_down_split_max(M * topk, E, n_out, k_in), wq::tiny_down_slabs(M, k_in));
}

size_t moe_gemm_workspace_bytes(int stage, int M, int topk, int E, int n_out, int k_in, size_t capacity,
                                int act_order) {
    if (M < 0 || topk <= 0 || E <= 0 || n_out <= 0 || k_in <= 0) return 0;
    size_t b = 0;
    if ((stage == WQ_STAGE_GATE_UP || stage == WQ_STAGE_RAW) && act_order) b += round256(capacity * k_in * 2);
    if (stage == WQ_STAGE_DOWN) b += round256((size_t)down_slabs(M, topk, E, n_out, k_in) * M * topk * n_out * sizeof(float));
    return b;
}

// A GATE_UP call that also routes the batch (moe_route_gate_up): the logits
// and the routing outputs; the desc's sorted_token_ids / expert_ids /
// num_tokens_post_padded are then written, not read.
struct RouteRequest {
    const float* logits;
    int renormalize;
    float* topk_weights;
    int32_t* topk_ids;
};

// noalloc: the workspace is the library's scratch array (d_workspace must be
// NULL and workspace_bytes 0; a need above its size is refused)
static wq_status moe_gemm(const wq_moe_gemm_desc* d, int wbits, void* stream, const char* who, bool noalloc = false,
                          const RouteRequest* route = nullptr) {
    WQ_REQUIRE(d != nullptr, WQ_ERR_INVALID, "%s: desc is NULL", who);
    WQ_REQUIRE(d->struct_size >= sizeof(wq_moe_gemm_desc), WQ_ERR_INVALID, "%s: struct_size %zu < %zu", who,
               d->struct_size, sizeof(wq_moe_gemm_desc));
    const int stage = d->stage;
    WQ_REQUIRE(stage == WQ_STAGE_GATE_UP || stage == WQ_STAGE_DOWN || stage == WQ_STAGE_RAW, WQ_ERR_INVALID,
               "%s: bad stage %d", who, stage);
    WQ_REQUIRE(d->act_dtype == WQ_F16 || d->act_dtype == WQ_BF16, WQ_ERR_INVALID, "%s: bad act dtype", who);
    if (wbits == 4) WQ_REQUIRE(d->act_dtype == WQ_F16, WQ_ERR_UNSUPPORTED, "%s: int4 path takes fp16 activations", who);
    WQ_REQUIRE(d->M >= 0 && d->topk >= 1 && d->E >= 1 && d->topk <= d->E, WQ_ERR_INVALID,
               "%s: bad M/topk/E (%d/%d/%d)", who, d->M, d->topk, d->E);
    WQ_REQUIRE(d->E <= 1024, WQ_ERR_UNSUPPORTED, "%s: E > 1024", who);
    WQ_REQUIRE((int64_t)d->M * d->topk <= MAX_PAIRS, WQ_ERR_UNSUPPORTED, "%s: M*topk > 2^24", who);
    WQ_REQUIRE(d->n_out > 0 && d->k_in > 0, WQ_ERR_INVALID, "%s: bad n_out/k_in", who);
    const int kchunk = wbits == 4 ? wq::WFmt<4>::KCHUNK : wq::WFmt<8>::KCHUNK;
    WQ_REQUIRE(d->k_in % kchunk == 0, WQ_ERR_UNSUPPORTED, "%s: k_in %d not a multiple of %d", who, d->k_in, kchunk);
    WQ_REQUIRE(d->n_out % (stage == WQ_STAGE_GATE_UP ? 32 : 16) == 0, WQ_ERR_UNSUPPORTED,
               "%s: n_out %d not a multiple of %d", who, d->n_out, stage == WQ_STAGE_GATE_UP ? 32 : 16);
    if (wbits == 4)
        WQ_REQUIRE(d->group_size == 128 || d->group_size == -1, WQ_ERR_UNSUPPORTED, "%s: group_size %d", who,
                   d->group_size);
    else
        WQ_REQUIRE(d->group_size == -1, WQ_ERR_UNSUPPORTED, "%s: int8 weights take per-column scales (-1)", who);
    WQ_REQUIRE(valid_block_size(d->block_size), WQ_ERR_UNSUPPORTED, "%s: block_size %d", who, d->block_size);
    const size_t need_cap = moe_align_capacity(d->M, d->topk, d->E, d->block_size);
    WQ_REQUIRE(d->capacity >= need_cap && d->capacity % (size_t)d->block_size == 0 &&
                   d->capacity <= (size_t)0x7fffffff,
               WQ_ERR_INVALID, "%s: capacity %zu (need >= %zu, multiple of block_size)", who, d->capacity, need_cap);
    const bool act_order = d->d_k_perm != nullptr;
    WQ_REQUIRE(!act_order || (wbits == 4 && stage != WQ_STAGE_DOWN), WQ_ERR_INVALID,
               "%s: k_perm only applies to int4 GATE_UP/RAW", who);
    if (route) {
        WQ_REQUIRE(stage == WQ_STAGE_GATE_UP, WQ_ERR_INVALID, "%s: routing goes with the GATE_UP stage", who);
        WQ_REQUIRE(d->topk <= 16, WQ_ERR_UNSUPPORTED, "%s: topk = %d > 16", who, d->topk);
    }
    const size_t ws = moe_gemm_workspace_bytes(stage, d->M, d->topk, d->E, d->n_out, d->k_in, d->capacity, act_order);
    if (noalloc) {
        WQ_REQUIRE(d->d_workspace == nullptr && d->workspace_bytes == 0, WQ_ERR_INVALID,
                   "%s: takes no workspace (d_workspace must be NULL, workspace_bytes 0)", who);
        WQ_REQUIRE(ws <= (size_t)WQ_NOALLOC_SCRATCH_BYTES, WQ_ERR_UNSUPPORTED,
                   "%s: needs %zu bytes of workspace, more than the %zu-byte scratch", who, ws,
                   (size_t)WQ_NOALLOC_SCRATCH_BYTES);
    } else {
        WQ_REQUIRE(d->workspace_bytes >= ws, WQ_ERR_INVALID, "%s: workspace %zu < required %zu", who,
                   d->workspace_bytes, ws);
    }
    if (d->M == 0) {
        if (!route) return ok();
        // no tokens: the routing arrays are still written (an empty sort)
        WQ_TRY(check_ptr(d->d_sorted_token_ids, "sorted_token_ids"));
        WQ_TRY(check_ptr(d->d_expert_ids, "expert_ids"));
        WQ_TRY(check_ptr(d->d_num_tokens_post_padded, "num_tokens_post_padded"));
        WQ_TRY(check_dev(d->d_sorted_token_ids, "sorted_token_ids"));
        WQ_TRY(check_dev(d->d_expert_ids, "expert_ids"));
        WQ_TRY(check_dev(d->d_num_tokens_post_padded, "num_tokens_post_padded"));
        return launch_routing(nullptr, 0, d->E, d->topk, route->renormalize, d->block_size, nullptr, nullptr,
                              const_cast<int32_t*>(d->d_sorted_token_ids), const_cast<int32_t*>(d->d_expert_ids),
                              const_cast<int32_t*>(d->d_num_tokens_post_padded), d->capacity, (hipStream_t)stream,
                              who);
    }
    WQ_TRY(check_ptr(d->d_a, "a"));
    WQ_TRY(check_ptr(d->d_w_packed, "w_packed"));
    WQ_TRY(check_ptr(d->d_scales, "scales"));
    WQ_TRY(check_ptr(d->d_sorted_token_ids, "sorted_token_ids"));
    WQ_TRY(check_ptr(d->d_expert_ids, "expert_ids"));
    WQ_TRY(check_ptr(d->d_num_tokens_post_padded, "num_tokens_post_padded"));
    WQ_TRY(check_ptr(d->d_out, "out"));
    if (act_order) WQ_TRY(check_ptr(d->d_k_perm, "k_perm"));
    if (stage == WQ_STAGE_DOWN) WQ_TRY(check_ptr(d->d_topk_weights, "topk_weights"));
    if (ws && !noalloc) WQ_TRY(check_ptr(d->d_workspace, "workspace"));
    if (route) {
        WQ_TRY(check_ptr(route->logits, "logits"));
        WQ_TRY(check_ptr(route->topk_weights, "topk_weights"));
        WQ_TRY(check_ptr(route->topk_ids, "topk_ids"));
        WQ_TRY(check_dev(route->logits, "logits"));
        WQ_TRY(check_dev(route->topk_weights, "topk_weights"));
        WQ_TRY(check_dev(route->topk_ids, "topk_ids"));
    }

    WQ_TRY(check_dev(d->d_a, "a"));
    WQ_TRY(check_dev(d->d_w_packed, "w_packed"));
    WQ_TRY(check_dev(d->d_scales, "scales"));
    WQ_TRY(check_dev(d->d_sorted_token_ids, "sorted_token_ids"));
    WQ_TRY(check_dev(d->d_expert_ids, "expert_ids"));
    WQ_TRY(check_dev(d->d_num_tokens_post_padded, "num_tokens_post_padded"));
    WQ_TRY(check_dev(d->d_out, "out"));
    if (act_order) WQ_TRY(check_dev(d->d_k_perm, "k_perm"));
    if (stage == WQ_STAGE_DOWN) WQ_TRY(check_dev(d->d_topk_weights, "topk_weights"));
    if (ws && !noalloc) WQ_TRY(check_dev(d->d_workspace, "workspace"));
    void* workspace = d->d_workspace;
    if (ws && noalloc) WQ_TRY(scratch_for_current_device(&workspace));

    hipStream_t s = (hipStream_t)stream;
    const bool bf16 = d->act_dtype == WQ_BF16;
    wq::GemmArgs g{};
    g.a = static_cast<const uint16_t*>(d->d_a);
    g.w = static_cast<const uint8_t*>(d->d_w_packed);
    g.s = static_cast<const uint16_t*>(d->d_scales);
    g.sorted = d->d_sorted_token_ids;
    g.expert_ids = d->d_expert_ids;
    g.ntpp = d->d_num_tokens_post_padded;
    g.topk_w = d->d_topk_weights;
    g.out = d->d_out;
    g.M = d->M;
    g.topk = d->topk;
    g.E = d->E;
    g.n_out = d->n_out;
    g.k_in = d->k_in;
    g.block_size = d->block_size;
    g.groups = (wbits == 4 && d->group_size == 128) ? d->k_in / 128 : 1;
    g.a_direct = (stage == WQ_STAGE_DOWN) ? 1 : 0;
    g.cap = (int)d->capacity;

    if (stage == WQ_STAGE_DOWN && wq::tiny_down_combine_supported(wbits, d->M, d->topk, d->n_out, d->k_in)) {
        // one token: the top-k sum is folded into the DOWN kernel
        wq::launch_tiny_down_combine(wbits, bf16, g, static_cast<uint16_t*>(d->d_out), s);
        return after_launch(who);
    }
    const int slabs = stage == WQ_STAGE_DOWN ? down_slabs(d->M, d->topk, d->E, d->n_out, d->k_in) : 1;
    const bool tiny = wq::tiny_supported(wbits, stage, d->M, d->k_in, g.groups, slabs);
    const bool large = !tiny && wq::prefill_supported(d->n_out, d->k_in, d->block_size);
    WQ_REQUIRE(!large || wq::prefill_fits(d->capacity, d->k_in), WQ_ERR_UNSUPPORTED,
               "%s: activations of %zu rows x %d channels exceed 4 GiB (large-batch kernel)", who, d->capacity,
               d->k_in);
    bool gathered = false;  // the act-order rows already gathered by the routing launch
    if (route) {
        // one launch: the small-batch kernel routes and sorts the batch itself,
        // and for one token of an act-order layer each workgroup also gathers
        // the token's row in its expert's channel order
        const bool fold = !tiny && !large &&
                          wq::decode_route_supported(stage, d->M, d->topk, d->E, (int)d->capacity, d->block_size) &&
                          (!act_order || wq::decode_route_ao_supported(d->M, d->topk, d->n_out, d->k_in));
        if (fold) {
            wq::RouteArgs ra;
            ra.logits = route->logits;
            ra.renormalize = route->renormalize ? 1 : 0;
            ra.w_out = route->topk_weights;
            ra.ids_out = route->topk_ids;
            // the desc's routing arrays are outputs of this call
            ra.sorted_out = const_cast<int32_t*>(d->d_sorted_token_ids);
            ra.expert_ids_out = const_cast<int32_t*>(d->d_expert_ids);
            ra.ntpp_out = const_cast<int32_t*>(d->d_num_tokens_post_padded);
            ra.perm = act_order ? d->d_k_perm : nullptr;
            wq::launch_gemm_decode_route(wbits, bf16, g, ra, s);
            return after_launch(who);
        }
        if (act_order && !tiny &&
            wq::route_gather_supported(d->M, d->topk, d->E, (int)d->capacity, d->block_size)) {
            // one launch routes, sorts and gathers the act-order rows
            uint16_t* a1 = static_cast<uint16_t*>(workspace);
            wq::launch_route_align_gather(route->logits, d->M, d->E, d->topk, route->renormalize ? 1 : 0,
                                          route->topk_weights, route->topk_ids,
                                          d->block_size, const_cast<int32_t*>(d->d_sorted_token_ids),
                                          const_cast<int32_t*>(d->d_expert_ids),
                                          const_cast<int32_t*>(d->d_num_tokens_post_padded), (int)d->capacity, g.a,
                                          d->d_k_perm, d->k_in, a1, s);
            WQ_TRY(after_launch(who));
            g.a = a1;
            g.a_direct = 1;
            gathered = true;
        } else {
            WQ_TRY(launch_routing(route->logits, d->M, d->E, d->topk, route->renormalize, d->block_size,
                                  route->topk_weights, route->topk_ids, const_cast<int32_t*>(d->d_sorted_token_ids),
                                  const_cast<int32_t*>(d->d_expert_ids),
                                  const_cast<int32_t*>(d->d_num_tokens_post_padded), d->capacity, s, who));
        }
    }
    if (act_order && !tiny && !gathered) {
        uint16_t* a1 = static_cast<uint16_t*>(workspace);
        wq::launch_gather_perm(g.a, d->d_k_perm, g.sorted, g.expert_ids, g.ntpp, d->M, d->topk, d->k_in,
                               d->block_size, g.cap, a1, s);
        WQ_TRY(after_launch(who));
        g.a = a1;
        g.a_direct = 1;
    }
    float* y = nullptr;
    if (stage == WQ_STAGE_DOWN) {
        y = static_cast<float*>(workspace);
        g.out = y;
        // a large-batch DOWN that does not split K writes each pair's routed
        // row rounded once to the activation type (half the bytes of the
        // per-pair rows each way); split slices keep fp32 partial sums
        g.y_act = (large && wq::prefill_down_split(d->M * d->topk, d->E, d->n_out, d->k_in, d->block_size) == 1)
                      ? 1 : 0;
    }
    int ksplit = 1;
    if (tiny) ksplit = wq::launch_gemm_tiny(wbits, bf16, stage, g, act_order ? d->d_k_perm : nullptr, slabs, s);
    else if (large) ksplit = wq::launch_gemm_prefill(wbits, bf16, stage, g, s);
    else wq::launch_gemm_decode(wbits, bf16, stage, g, s);
    WQ_TRY(after_launch(who));
    if (stage == WQ_STAGE_DOWN) {
        if (g.y_act) {
            WQ_REQUIRE(ksplit == 1, WQ_ERR_HIP, "%s: DOWN split K after all", who);
            wq::launch_combine_act(reinterpret_cast<const uint16_t*>(y), d->M, d->topk, d->n_out, bf16,
                                   static_cast<uint16_t*>(d->d_out), s);
        } else {
            wq::launch_combine(y, d->M, d->topk, d->n_out, ksplit, bf16, static_cast<uint16_t*>(d->d_out), s);
        }
        WQ_TRY(after_launch(who));
    }
    return ok();
}

wq_status moe_w4a16_gemm(const wq_moe_gemm_desc* d, void* stream) {
    try {
        return moe_gemm(d, 4, stream, "moe_w4a16_gemm");
    } catch (...) {
        return fail(WQ_ERR_HIP, "moe_w4a16_gemm: unexpected exception");
    }
}

wq_status moe_w8a16_gemm(const wq_moe_gemm_desc* d, void* stream) {
    try {
        return moe_gemm(d, 8, stream, "moe_w8a16_gemm");
    } catch (...) {
        return fail(WQ_ERR_HIP, "moe_w8a16_gemm: unexpected exception");
    }
}

wq_status moe_route_gate_up(const float* d_logits, int renormalize, float* d_topk_weights, int32_t* d_topk_ids,
                            const wq_moe_gemm_desc* d, int wbits, void* stream) {
    try {
        WQ_REQUIRE(wbits == 4 || wbits == 8, WQ_ERR_INVALID, "moe_route_gate_up: wbits %d not 4 or 8", wbits);
        const RouteRequest rr{d_logits, renormalize, d_topk_weights, d_topk_ids};
        return moe_gemm(d, wbits, stream, "moe_route_gate_up", false, &rr);
    } catch (...) {
        return fail(WQ_ERR_HIP, "moe_route_gate_up: unexpected exception");
    }
}

wq_status moe_w8a16_gemm_noalloc(const wq_moe_gemm_desc* d, void* stream) {
    try {
        return moe_gemm(d, 8, stream, "moe_w8a16_gemm_noalloc", true);
    } catch (...) {
        return fail(WQ_ERR_HIP, "moe_w8a16_gemm_noalloc: unexpected exception");
    }
}

// ---------------------------------------------------------------------------
// FP8 (E4M3) W8A8 grouped GEMM
// ---------------------------------------------------------------------------
static int fp8_down_slabs(int M, int topk, int E, int n_out, int k_in) {
    const int T = M * topk;
    return std::max(wq::fp8_down_split(T, E, n_out, k_in, 64), wq::fp8_down_split(T, E, n_out, k_in, 128));
}

size_t moe_fp8_gemm_workspace_bytes(int stage, int M, int topk, int E, int n_out, int k_in) {
    if (M < 0 || topk <= 0 || E <= 0 || n_out <= 0 || k_in <= 0) return 0;
    if (stage == WQ_STAGE_GATE_UP || stage == WQ_STAGE_RAW) return round256((size_t)M * k_in);  // x codes
    if (stage == WQ_STAGE_DOWN)
        return round256((size_t)fp8_down_slabs(M, topk, E, n_out, k_in) * M * topk * n_out * sizeof(float));
    return 0;
}

static wq_status fp8_gemm(const wq_moe_gemm_desc* d, float in_scale, float out_scale, void* stream) {
    const char* who = "moe_fp8_w8a8_gemm";
    WQ_REQUIRE(d != nullptr, WQ_ERR_INVALID, "%s: desc is NULL", who);
    WQ_REQUIRE(d->struct_size >= sizeof(wq_moe_gemm_desc), WQ_ERR_INVALID, "%s: struct_size %zu < %zu", who,
               d->struct_size, sizeof(wq_moe_gemm_desc));
    const int stage = d->stage;
    WQ_REQUIRE(stage == WQ_STAGE_GATE_UP || stage == WQ_STAGE_DOWN || stage == WQ_STAGE_RAW, WQ_ERR_INVALID,
               "%s: bad stage %d", who, stage);
    WQ_REQUIRE(d->act_dtype == WQ_F16 || d->act_dtype == WQ_BF16, WQ_ERR_INVALID, "%s: bad act dtype", who);
    WQ_REQUIRE(d->M >= 0 && d->topk >= 1 && d->E >= 1 && d->topk <= d->E, WQ_ERR_INVALID,
               "%s: bad M/topk/E (%d/%d/%d)", who, d->M, d->topk, d->E);
    WQ_REQUIRE(d->E <= 1024, WQ_ERR_UNSUPPORTED, "%s: E > 1024", who);
    WQ_REQUIRE((int64_t)d->M * d->topk <= MAX_PAIRS, WQ_ERR_UNSUPPORTED, "%s: M*topk > 2^24", who);
    WQ_REQUIRE(d->n_out > 0 && d->k_in > 0, WQ_ERR_INVALID, "%s: bad n_out/k_in", who);
    WQ_REQUIRE(d->k_in % wq::FP8_KCHUNK == 0, WQ_ERR_UNSUPPORTED, "%s: k_in %d not a multiple of %d", who, d->k_in,
               wq::FP8_KCHUNK);
    WQ_REQUIRE(d->n_out % (stage == WQ_STAGE_GATE_UP ? 32 : 16) == 0, WQ_ERR_UNSUPPORTED,
               "%s: n_out %d not a multiple of %d", who, d->n_out, stage == WQ_STAGE_GATE_UP ? 32 : 16);
    WQ_REQUIRE(d->group_size == -1, WQ_ERR_UNSUPPORTED, "%s: FP8 weights take per-column scales (-1)", who);
    WQ_REQUIRE(d->d_k_perm == nullptr, WQ_ERR_INVALID, "%s: no act-order for FP8 weights", who);
    WQ_REQUIRE(std::isfinite(in_scale) && in_scale > 0.0f, WQ_ERR_INVALID, "%s: in_scale must be finite and > 0",
               who);
    WQ_REQUIRE(stage != WQ_STAGE_GATE_UP || (std::isfinite(out_scale) && out_scale > 0.0f), WQ_ERR_INVALID,
               "%s: out_scale must be finite and > 0", who);
    WQ_REQUIRE(valid_block_size(d->block_size), WQ_ERR_UNSUPPORTED, "%s: block_size %d", who, d->block_size);
    const size_t need_cap = moe_align_capacity(d->M, d->topk, d->E, d->block_size);
    WQ_REQUIRE(d->capacity >= need_cap && d->capacity % (size_t)d->block_size == 0 &&
                   d->capacity <= (size_t)0x7fffffff,
               WQ_ERR_INVALID, "%s: capacity %zu (need >= %zu, multiple of block_size)", who, d->capacity, need_cap);
    const size_t ws = moe_fp8_gemm_workspace_bytes(stage, d->M, d->topk, d->E, d->n_out, d->k_in);
    WQ_REQUIRE(d->workspace_bytes >= ws, WQ_ERR_INVALID, "%s: workspace %zu < required %zu", who, d->workspace_bytes,
               ws);
    const bool large = wq::fp8_prefill_supported(d->n_out, d->k_in, d->block_size);
    // the large-batch kernel addresses its activation codes with 32-bit byte offsets
    const size_t a_rows = stage == WQ_STAGE_DOWN ? d->capacity : (size_t)d->M;
    WQ_REQUIRE(!large || a_rows * (size_t)d->k_in <= (size_t)0xffffffffu, WQ_ERR_UNSUPPORTED,
               "%s: activations of %zu rows x %d codes exceed 4 GiB (large-batch kernel)", who, a_rows, d->k_in);
    if (d->M == 0) return ok();
    WQ_TRY(check_ptr(d->d_a, "a"));
    WQ_TRY(check_ptr(d->d_w_packed, "w_packed"));
    WQ_TRY(check_ptr(d->d_scales, "scales"));
    WQ_TRY(check_ptr(d->d_sorted_token_ids, "sorted_token_ids"));
    WQ_TRY(check_ptr(d->d_expert_ids, "expert_ids"));
    WQ_TRY(check_ptr(d->d_num_tokens_post_padded, "num_tokens_post_padded"));
    WQ_TRY(check_ptr(d->d_out, "out"));
    if (stage == WQ_STAGE_DOWN) WQ_TRY(check_ptr(d->d_topk_weights, "topk_weights"));
    WQ_TRY(check_ptr(d->d_workspace, "workspace"));
    WQ_TRY(check_dev(d->d_a, "a"));
    WQ_TRY(check_dev(d->d_w_packed, "w_packed"));
    WQ_TRY(check_dev(d->d_scales, "scales"));
    WQ_TRY(check_dev(d->d_sorted_token_ids, "sorted_token_ids"));
    WQ_TRY(check_dev(d->d_expert_ids, "expert_ids"));
    WQ_TRY(check_dev(d->d_num_tokens_post_padded, "num_tokens_post_padded"));
    WQ_TRY(check_dev(d->d_out, "out"));
    if (stage == WQ_STAGE_DOWN) WQ_TRY(check_dev(d->d_topk_weights, "topk_weights"));
    WQ_TRY(check_dev(d->d_workspace, "workspace"));

    hipStream_t s = (hipStream_t)stream;
    const bool bf16 = d->act_dtype == WQ_BF16;
    wq::Fp8GemmArgs g{};
    g.w = static_cast<const uint8_t*>(d->d_w_packed);
    g.s = static_cast<const float*>(d->d_scales);
    g.sorted = d->d_sorted_token_ids;
    g.expert_ids = d->d_expert_ids;
    g.ntpp = d->d_num_tokens_post_padded;
    g.topk_w = d->d_topk_weights;
    g.out = d->d_out;
    g.M = d->M;
    g.topk = d->topk;
    g.E = d->E;
    g.n_out = d->n_out;
    g.k_in = d->k_in;
    g.block_size = d->block_size;
    g.cap = (int)d->capacity;
    g.in_scale = in_scale;
    g.out_scale = out_scale;
    if (stage == WQ_STAGE_DOWN) {
        g.a = static_cast<const uint8_t*>(d->d_a);  // H codes in sorted order
        g.a_direct = 1;
        if (wq::fp8_down_combine_supported(d->M, d->topk, d->n_out, d->k_in)) {
            wq::launch_fp8_down_combine(bf16, g, s);  // g.out: the output row
            return after_launch(who);
        }
        g.out = d->d_workspace;                     // fp32 Y slabs
    } else if (wq::fp8_fold_quant_supported(stage, d->M, d->n_out, d->k_in, d->block_size)) {
        g.x16 = static_cast<const uint16_t*>(d->d_a);  // quantised inside the GEMM
        g.x_bf16 = bf16 ? 1 : 0;
        g.a_direct = 0;
    } else {
        uint8_t* xq = static_cast<uint8_t*>(d->d_workspace);
        wq::launch_fp8_quant(static_cast<const uint16_t*>(d->d_a), d->M, d->k_in, bf16, in_scale, xq, s);
        WQ_TRY(after_launch(who));
        g.a = xq;
        g.a_direct = 0;
    }
    const int ks = wq::launch_gemm_fp8(stage, g, s);
    WQ_TRY(after_launch(who));
    if (stage == WQ_STAGE_DOWN) {
        wq::launch_combine(static_cast<const float*>(d->d_workspace), d->M, d->topk, d->n_out, ks, bf16,
                           static_cast<uint16_t*>(d->d_out), s);
        WQ_TRY(after_launch(who));
    }
    return ok();
}

wq_status moe_fp8_w8a8_gemm(const wq_moe_gemm_desc* d, float in_scale, float out_scale, void* stream) {
    try {
        return fp8_gemm(d, in_scale, out_scale, stream);
    } catch (...) {
        return fail(WQ_ERR_HIP, "moe_fp8_w8a8_gemm: unexpected exception");
    }
}

static wq_status sparse24_gemm(int bits, const void* d_x, int M, int K, int N, const void* d_vals, const void* d_meta,
                               const void* d_scales, int group_size, void* d_y, int act_dtype, void* stream,
                               const char* who) {
    WQ_REQUIRE(M >= 0 && K > 0 && N > 0, WQ_ERR_INVALID, "%s: bad sizes M %d K %d N %d", who, M, K, N);
    WQ_REQUIRE(act_dtype == WQ_F16, WQ_ERR_UNSUPPORTED, "%s: fp16 activations only", who);
    WQ_REQUIRE(group_size == 128 || group_size == -1, WQ_ERR_UNSUPPORTED, "%s: group_size %d (128 or -1)", who,
               group_size);
    WQ_REQUIRE(K % 256 == 0, WQ_ERR_UNSUPPORTED, "%s: K %d not a multiple of 256", who, K);
    WQ_REQUIRE(N % 16 == 0, WQ_ERR_UNSUPPORTED, "%s: N %d not a multiple of 16", who, N);
    WQ_REQUIRE((M + 15) / 16 <= 65535, WQ_ERR_UNSUPPORTED, "%s: M too large", who);
    if (M == 0) return ok();
    WQ_TRY(check_ptr(d_x, "x"));
    WQ_TRY(check_ptr(d_vals, "vals"));
    WQ_TRY(check_ptr(d_meta, "meta"));
    WQ_TRY(check_ptr(d_scales, "scales"));
    WQ_TRY(check_ptr(d_y, "y"));
    WQ_TRY(check_dev(d_x, "x"));
    WQ_TRY(check_dev(d_vals, "vals"));
    WQ_TRY(check_dev(d_meta, "meta"));
    WQ_TRY(check_dev(d_scales, "scales"));
    WQ_TRY(check_dev(d_y, "y"));
    wq::launch_sparse24(bits, static_cast<const uint16_t*>(d_x), M, K, N, static_cast<const uint8_t*>(d_vals),
                        static_cast<const uint8_t*>(d_meta), static_cast<const uint16_t*>(d_scales), group_size,
                        static_cast<uint16_t*>(d_y), (hipStream_t)stream);
    return after_launch(who);
}

wq_status sparse24_w4a16_gemm(const void* d_x, int M, int K, int N, const void* d_vals, const void* d_meta,
                              const void* d_scales, int group_size, void* d_y, int act_dtype, void* stream) {
    try {
        return sparse24_gemm(4, d_x, M, K, N, d_vals, d_meta, d_scales, group_size, d_y, act_dtype, stream,
                             "sparse24_w4a16_gemm");
    } catch (...) {
        return fail(WQ_ERR_HIP, "sparse24_w4a16_gemm: unexpected exception");
    }
}

wq_status sparse24_w8a16_gemm(const void* d_x, int M, int K, int N, const void* d_vals, const void* d_meta,
                              const void* d_scales, int group_size, void* d_y, int act_dtype, void* stream) {
    try {
        return sparse24_gemm(8, d_x, M, K, N, d_vals, d_meta, d_scales, group_size, d_y, act_dtype, stream,
                             "sparse24_w8a16_gemm");
    } catch (...) {
        return fail(WQ_ERR_HIP, "sparse24_w8a16_gemm: unexpected exception");
    }
}

// ---------------------------------------------------------------------------
// Dense single-expert linear.  1..4 rows (without act-order): one small-batch
// kernel with the rows staged in LDS, no workspace.  Otherwise the grouped
// kernels with E = 1 and top-1 on identity routing written into the workspace,
// the DOWN stage with unit routed weights (rows gathered by token, not by
// sorted position: x has M rows), the combine rounding the fp32 result to the
// activation type.
// ---------------------------------------------------------------------------
namespace {
struct DenseLayout {
    int bs, ks;
    size_t cap, off_sorted, off_eids, off_ntpp, off_w, off_a1, off_y, total;
};

// batch-size dispatch of the grouped path (above 128 rows, or with act-order;
// up to 128 rows without act-order one dense kernel runs, no workspace): the
// small-batch kernel (blocks of 16 rows) up to 24 rows, the large-batch kernel
// with 64-row tiles up to 192 (one expert gives few token tiles: 128-row tiles
// left the GPU part idle, Yi-34B shape int4 M = 128 0.114 -> 0.091 ms, M = 192
// 0.114 -> 0.106 ms; at 256 rows and above they are faster), 128-row tiles above
int dense_block_size(int M, int N, int K) {
    const int bs = M <= 24 ? 16 : (M <= 192 ? 64 : 128);
    return (bs == 16 || wq::prefill_supported(N, K, bs)) ? bs : 16;
}

DenseLayout dense_layout(int M, int K, int N, bool act_order) {
    DenseLayout L{};
    L.bs = dense_block_size(M, N, K);
    L.cap = moe_align_capacity(M, 1, 1, L.bs);
    L.ks = (L.bs == 16) ? 1 : wq::prefill_down_split(M, 1, N, K, L.bs);
    size_t o = 0;
    L.off_sorted = o;
    o += round256(L.cap * 4);
    L.off_eids = o;
    o += round256(L.cap / L.bs * 4);
    L.off_ntpp = o;
    o += 256;
    L.off_w = o;
    o += round256((size_t)M * 4);
    L.off_a1 = o;
    if (act_order) o += round256(L.cap * (size_t)K * 2);
    L.off_y = o;
    o += round256((size_t)L.ks * M * N * sizeof(float));
    L.total = o;
    return L;
}

wq_status dense_gemm(int wbits, const void* d_x, int M, int K, int N, const void* d_w, const void* d_scales,
                     int group_size, const int32_t* d_k_perm, void* d_y, int act_dtype, void* d_ws, size_t ws_bytes,
                     void* stream, const char* who) {
    WQ_REQUIRE(M >= 0 && K > 0 && N > 0, WQ_ERR_INVALID, "%s: bad sizes M %d K %d N %d", who, M, K, N);
    WQ_REQUIRE(M <= MAX_PAIRS, WQ_ERR_UNSUPPORTED, "%s: M > 2^24", who);
    WQ_REQUIRE(act_dtype == WQ_F16 || act_dtype == WQ_BF16, WQ_ERR_INVALID, "%s: bad act dtype", who);
    if (wbits == 4) WQ_REQUIRE(act_dtype == WQ_F16, WQ_ERR_UNSUPPORTED, "%s: int4 path takes fp16 activations", who);
    const int kchunk = wbits == 4 ? wq::WFmt<4>::KCHUNK : wq::WFmt<8>::KCHUNK;
    WQ_REQUIRE(K % kchunk == 0, WQ_ERR_UNSUPPORTED, "%s: K %d not a multiple of %d", who, K, kchunk);
    WQ_REQUIRE(N % 16 == 0, WQ_ERR_UNSUPPORTED, "%s: N %d not a multiple of 16", who, N);
    if (wbits == 4)
        WQ_REQUIRE(group_size == 128 || group_size == -1, WQ_ERR_UNSUPPORTED, "%s: group_size %d", who, group_size);
    const bool act_order = d_k_perm != nullptr;
    const size_t need = dense_gemm_workspace_bytes(M, K, N, act_order);
    WQ_REQUIRE(ws_bytes >= need, WQ_ERR_INVALID, "%s: workspace %zu < required %zu", who, ws_bytes, need);
    if (M == 0) return ok();
    WQ_TRY(check_ptr(d_x, "x"));
    WQ_TRY(check_ptr(d_w, "w_packed"));
    WQ_TRY(check_ptr(d_scales, "scales"));
    WQ_TRY(check_ptr(d_y, "y"));
    if (act_order) WQ_TRY(check_ptr(d_k_perm, "k_perm"));  // read with 128-bit loads by the gather
    WQ_TRY(check_dev(d_x, "x"));
    WQ_TRY(check_dev(d_w, "w_packed"));
    WQ_TRY(check_dev(d_scales, "scales"));
    WQ_TRY(check_dev(d_y, "y"));
    if (act_order) WQ_TRY(check_dev(d_k_perm, "k_perm"));
    hipStream_t s = (hipStream_t)stream;
    const bool bf16 = act_dtype == WQ_BF16;
    const int groups = (wbits == 4 && group_size == 128) ? K / 128 : 1;
    if (need == 0) {  // 1..4 rows: one kernel, no workspace
        wq::launch_dense_decode(wbits, bf16, static_cast<const uint16_t*>(d_x), M, K, N,
                                static_cast<const uint8_t*>(d_w), static_cast<const uint16_t*>(d_scales), groups,
                                static_cast<uint16_t*>(d_y), s);
        return after_launch(who);
    }
    WQ_TRY(check_ptr(d_ws, "workspace"));
    WQ_TRY(check_dev(d_ws, "workspace"));
    WQ_REQUIRE(reinterpret_cast<uintptr_t>(d_ws) % 256 == 0, WQ_ERR_INVALID, "%s: workspace not 256-byte aligned",
               who);

    const DenseLayout L = dense_layout(M, K, N, act_order);
    WQ_REQUIRE(L.bs == 16 || wq::prefill_fits(L.cap, K), WQ_ERR_UNSUPPORTED,
               "%s: activations of %d rows x %d channels exceed 4 GiB (large-batch kernel)", who, M, K);
    uint8_t* ws = static_cast<uint8_t*>(d_ws);
    int32_t* sorted = reinterpret_cast<int32_t*>(ws + L.off_sorted);
    int32_t* eids = reinterpret_cast<int32_t*>(ws + L.off_eids);
    int32_t* ntpp = reinterpret_cast<int32_t*>(ws + L.off_ntpp);
    float* tw = reinterpret_cast<float*>(ws + L.off_w);
    float* y = reinterpret_cast<float*>(ws + L.off_y);
    wq::launch_identity_route(M, (int)L.cap, L.bs, sorted, eids, ntpp, tw, s);
    WQ_TRY(after_launch(who));

    wq::GemmArgs g{};
    g.a = static_cast<const uint16_t*>(d_x);
    g.w = static_cast<const uint8_t*>(d_w);
    g.s = static_cast<const uint16_t*>(d_scales);
    g.sorted = sorted;
    g.expert_ids = eids;
    g.ntpp = ntpp;
    g.topk_w = tw;
    g.out = y;
    g.M = M;
    g.topk = 1;
    g.E = 1;
    g.n_out = N;
    g.k_in = K;
    g.block_size = L.bs;
    g.groups = groups;
    g.a_direct = 0;  // x row = token of the pair (x has M rows, no pad rows)
    g.cap = (int)L.cap;
    if (act_order) {
        uint16_t* a1 = reinterpret_cast<uint16_t*>(ws + L.off_a1);
        wq::launch_gather_perm(g.a, d_k_perm, sorted, eids, ntpp, M, 1, K, L.bs, g.cap, a1, s);
        WQ_TRY(after_launch(who));
        g.a = a1;
        g.a_direct = 1;
    }
    int ks = 1;
    if (L.bs != 16) ks = wq::launch_gemm_prefill(wbits, bf16, wq::STAGE_DOWN, g, s);
    else wq::launch_gemm_decode(wbits, bf16, wq::STAGE_DOWN, g, s);
    WQ_TRY(after_launch(who));
    wq::launch_combine(y, M, 1, N, ks, bf16, static_cast<uint16_t*>(d_y), s);
    return after_launch(who);
}
}  // namespace

size_t dense_gemm_workspace_bytes(int M, int K, int N, int act_order) {
    if (M < 0 || K <= 0 || N <= 0 || M > MAX_PAIRS) return 0;
    if (M == 0) return 0;
    if (!act_order && wq::dense_decode_supported(M, K)) return 0;  // the single-kernel small-batch path
    return dense_layout(M, K, N, act_order != 0).total;
}

wq_status dense_w4a16_gemm(const void* d_x, int M, int K, int N, const void* d_w_packed, const void* d_scales,
                           int group_size, const int32_t* d_k_perm, void* d_y, int act_dtype, void* d_workspace,
                           size_t workspace_bytes, void* stream) {
    try {
        return dense_gemm(4, d_x, M, K, N, d_w_packed, d_scales, group_size, d_k_perm, d_y, act_dtype, d_workspace,
                          workspace_bytes, stream, "dense_w4a16_gemm");
    } catch (...) {
        return fail(WQ_ERR_HIP, "dense_w4a16_gemm: unexpected exception");
    }
}

wq_status dense_w8a16_gemm(const void* d_x, int M, int K, int N, const void* d_w_packed, const void* d_scales,
                           void* d_y, int act_dtype, void* d_workspace, size_t workspace_bytes, void* stream) {
    try {
        return dense_gemm(8, d_x, M, K, N, d_w_packed, d_scales, -1, nullptr, d_y, act_dtype, d_workspace,
                          workspace_bytes, stream, "dense_w8a16_gemm");
    } catch (...) {
        return fail(WQ_ERR_HIP, "dense_w8a16_gemm: unexpected exception");
    }
}

// ---------------------------------------------------------------------------
wq_status wq_quantize_w8(const void* d_w, int64_t rows, int k, int dtype, int8_t* d_q, uint16_t* d_scales,
                         void* stream) {
    try {
        WQ_REQUIRE(rows >= 0 && k > 0, WQ_ERR_INVALID, "quantize_w8: bad sizes rows %lld k %d", (long long)rows, k);
        WQ_REQUIRE(dtype == WQ_F16 || dtype == WQ_BF16, WQ_ERR_INVALID, "quantize_w8: bad dtype %d", dtype);
        WQ_REQUIRE(k % 8 == 0, WQ_ERR_UNSUPPORTED, "quantize_w8: k %d not a multiple of 8", k);
        WQ_REQUIRE((rows + 3) / 4 <= 0x7fffffffLL, WQ_ERR_UNSUPPORTED, "quantize_w8: too many rows");
        if (rows == 0) return ok();
        WQ_TRY(check_ptr(d_w, "w"));
        WQ_TRY(check_ptr(d_q, "q"));
        WQ_TRY(check_ptr(d_scales, "scales"));
        WQ_TRY(check_dev(d_w, "w"));
        WQ_TRY(check_dev(d_q, "q"));
        WQ_TRY(check_dev(d_scales, "scales"));
        WQ_REQUIRE(reinterpret_cast<uintptr_t>(d_w) % 16 == 0 && reinterpret_cast<uintptr_t>(d_q) % 8 == 0,
                   WQ_ERR_INVALID, "quantize_w8: w must be 16-byte and q 8-byte aligned");
        wq::launch_quant_w8(static_cast<const uint16_t*>(d_w), rows, k, dtype == WQ_BF16, d_q, d_scales,
                            (hipStream_t)stream);
        return after_launch("wq_quantize_w8");
    } catch (...) {
        return fail(WQ_ERR_HIP, "quantize_w8: unexpected exception");
    }
}

// ---------------------------------------------------------------------------
// Offline packers
// ---------------------------------------------------------------------------
size_t wq_pack_w4_bytes(int E, int n_out, int k_in) {
    if (E <= 0 || n_out <= 0 || k_in <= 0 || n_out % 16 || k_in % 128) return 0;
    return (size_t)E * n_out * k_in / 2;
}

size_t wq_pack_w8_bytes(int E, int n_out, int k_in) {
    if (E <= 0 || n_out <= 0 || k_in <= 0 || n_out % 16 || k_in % 64) return 0;
    return (size_t)E * n_out * k_in;
}

// canonical row held by packed row p of expert e
static inline int logical_row(int p, int n_out, bool interleave, const int32_t* perm_e) {
    if (!interleave) return perm_e ? perm_e[p] : p;
    const int t = p / 16, j = t / 2, half = t % 2, within = p % 16;
    int lr = 16 * j + within;
    if (perm_e) lr = perm_e[lr];
    return half * (n_out / 2) + lr;
}

static wq_status check_row_perm(int E, int n, const int32_t* perm) {
    if (!perm) return WQ_OK;
    std::vector<char> seen((size_t)n);
    for (int e = 0; e < E; ++e) {
        std::fill(seen.begin(), seen.end(), 0);
        for (int i = 0; i < n; ++i) {
            const int32_t v = perm[(size_t)e * n + i];
            WQ_REQUIRE(v >= 0 && v < n && !seen[v], WQ_ERR_INVALID, "row_perm of expert %d is not a permutation", e);
            seen[v] = 1;
        }
    }
    return WQ_OK;
}

wq_status wq_pack_w4(int E, int n_out, int k_in, const int8_t* q, const uint16_t* scales, int group_size,
                     const int32_t* g_idx, const int32_t* row_perm, int flags, void* packed, uint16_t* scales_packed,
                     int32_t* k_perm) {
    try {
        WQ_REQUIRE(E > 0 && n_out > 0 && k_in > 0, WQ_ERR_INVALID, "pack_w4: bad sizes");
        const bool il = (flags & WQ_PACK_INTERLEAVE_GATE_UP) != 0;
        WQ_REQUIRE(n_out % (il ? 32 : 16) == 0, WQ_ERR_UNSUPPORTED, "pack_w4: n_out %d", n_out);
        WQ_REQUIRE(k_in % 128 == 0, WQ_ERR_UNSUPPORTED, "pack_w4: k_in %d not a multiple of 128", k_in);
        WQ_REQUIRE(group_size == 128 || group_size == -1, WQ_ERR_UNSUPPORTED, "pack_w4: group_size %d", group_size);
        WQ_REQUIRE(q && scales && packed && scales_packed, WQ_ERR_INVALID, "pack_w4: NULL buffer");
        WQ_REQUIRE(!g_idx || (group_size == 128 && k_perm), WQ_ERR_INVALID,
                   "pack_w4: act-order needs group_size 128 and a k_perm output");
        const int G = group_size == -1 ? 1 : k_in / group_size;
        WQ_TRY(check_row_perm(E, il ? n_out / 2 : n_out, row_perm));
        const int rows_perm = il ? n_out / 2 : n_out;
        // input-channel order: stable sort by group
        std::vector<int32_t> sig((size_t)E * k_in);
        for (int e = 0; e < E; ++e) {
            int32_t* s = sig.data() + (size_t)e * k_in;
            if (!g_idx) {
                for (int k = 0; k < k_in; ++k) s[k] = k;
                continue;
            }
            const int32_t* gi = g_idx + (size_t)e * k_in;
            std::vector<int> cnt(G, 0);
            for (int k = 0; k < k_in; ++k) {
                WQ_REQUIRE(gi[k] >= 0 && gi[k] < G, WQ_ERR_INVALID, "pack_w4: g_idx out of range (expert %d)", e);
                cnt[gi[k]]++;
            }
            for (int gg = 0; gg < G; ++gg)
                WQ_REQUIRE(cnt[gg] == group_size, WQ_ERR_UNSUPPORTED,
                           "pack_w4: act-order group %d of expert %d has %d channels, not %d", gg, e, cnt[gg],
                           group_size);
            std::vector<int> pos(G);
            for (int gg = 0; gg < G; ++gg) pos[gg] = gg * group_size;
            for (int k = 0; k < k_in; ++k) s[pos[gi[k]]++] = k;
        }
        // value range
        for (size_t i = 0, n = (size_t)E * n_out * k_in; i < n; ++i)
            WQ_REQUIRE(q[i] >= -8 && q[i] <= 7, WQ_ERR_INVALID, "pack_w4: code %d out of [-8, 7]", (int)q[i]);
        if (k_perm) std::memcpy(k_perm, sig.data(), sizeof(int32_t) * sig.size());

        const int C = k_in / 128;
        const size_t expert_bytes = (size_t)n_out * k_in / 2;
        uint8_t* out = static_cast<uint8_t*>(packed);
        parallel_for(E * (n_out / 16), [&](int job) {
            const int e = job / (n_out / 16), t = job % (n_out / 16);
            const int32_t* pe = row_perm ? row_perm + (size_t)e * rows_perm : nullptr;
            const int32_t* s = sig.data() + (size_t)e * k_in;
            for (int l = 0; l < 64; ++l) {
                const int p = t * 16 + (l & 15);
                const int lr = logical_row(p, n_out, il, pe);
                const int8_t* qr = q + ((size_t)e * n_out + lr) * k_in;
                for (int c = 0; c < C; ++c) {
                    uint32_t* dst = reinterpret_cast<uint32_t*>(out + (size_t)e * expert_bytes +
                                                                (((size_t)t * C + c) * 64 + l) * 16);
                    for (int st = 0; st < 4; ++st) {
                        uint32_t d = 0;
                        for (int j = 0; j < 8; ++j) {
                            const int kp = 128 * c + 32 * st + 8 * (l >> 4) + j;
                            const uint32_t u = (uint32_t)(qr[s[kp]] + 8);
                            d |= u << (4 * (j >> 1) + 16 * (j & 1));
                        }
                        dst[st] = d;
                    }
                }
            }
            if (t == 0) {
                for (int gg = 0; gg < G; ++gg)
                    for (int pp = 0; pp < n_out; ++pp)
                        scales_packed[((size_t)e * G + gg) * n_out + pp] =
                            scales[((size_t)e * G + gg) * n_out + logical_row(pp, n_out, il, pe)];
            }
        });
        return ok();
    } catch (...) {
        return fail(WQ_ERR_INVALID, "pack_w4: unexpected exception");
    }
}

wq_status wq_pack_w8(int E, int n_out, int k_in, const int8_t* q, const uint16_t* scales, const int32_t* row_perm,
                     int flags, void* packed, uint16_t* scales_packed) {
    try {
        WQ_REQUIRE(E > 0 && n_out > 0 && k_in > 0, WQ_ERR_INVALID, "pack_w8: bad sizes");
        const bool il = (flags & WQ_PACK_INTERLEAVE_GATE_UP) != 0;
        WQ_REQUIRE(n_out % (il ? 32 : 16) == 0, WQ_ERR_UNSUPPORTED, "pack_w8: n_out %d", n_out);
        WQ_REQUIRE(k_in % 64 == 0, WQ_ERR_UNSUPPORTED, "pack_w8: k_in %d not a multiple of 64", k_in);
        WQ_REQUIRE(q && scales && packed && scales_packed, WQ_ERR_INVALID, "pack_w8: NULL buffer");
        const int rows_perm = il ? n_out / 2 : n_out;
        WQ_TRY(check_row_perm(E, rows_perm, row_perm));
        const int C = k_in / 64;
        const size_t expert_bytes = (size_t)n_out * k_in;
        uint8_t* out = static_cast<uint8_t*>(packed);
        parallel_for(E * (n_out / 16), [&](int job) {
            const int e = job / (n_out / 16), t = job % (n_out / 16);
            const int32_t* pe = row_perm ? row_perm + (size_t)e * rows_perm : nullptr;
            for (int l = 0; l < 64; ++l) {
                const int p = t * 16 + (l & 15);
                const int lr = logical_row(p, n_out, il, pe);
                const int8_t* qr = q + ((size_t)e * n_out + lr) * k_in;
                for (int c = 0; c < C; ++c) {
                    uint8_t* dst = out + (size_t)e * expert_bytes + (((size_t)t * C + c) * 64 + l) * 16;
                    for (int st = 0; st < 2; ++st)
                        for (int j = 0; j < 8; ++j)
                            dst[8 * st + j] = (uint8_t)qr[64 * c + 32 * st + 8 * (l >> 4) + j];
                }
            }
            if (t == 0)
                for (int pp = 0; pp < n_out; ++pp)
                    scales_packed[(size_t)e * n_out + pp] = scales[(size_t)e * n_out + logical_row(pp, n_out, il, pe)];
        });
        return ok();
    } catch (...) {
        return fail(WQ_ERR_INVALID, "pack_w8: unexpected exception");
    }
}

size_t wq_pack_fp8_bytes(int E, int n_out, int k_in) {
    if (E <= 0 || n_out <= 0 || k_in <= 0 || n_out % 16 || k_in % wq::FP8_KCHUNK) return 0;
    return (size_t)E * n_out * k_in;
}

// E4M3 codes: tiles of 16 rows x 128 channels (2 KiB).  Lane l's MFMA operand
// is row l % 16, channels [32 (l / 16), +32) of the chunk; its first 16
// channels sit at bytes 16 l of the chunk and the other 16 at 1024 + 16 l, so
// each of a wave's two 128-bit loads reads one contiguous KiB
wq_status wq_pack_fp8(int E, int n_out, int k_in, const uint8_t* codes, const float* scales, const int32_t* row_perm,
                      int flags, void* packed, float* scales_packed) {
    try {
        WQ_REQUIRE(E > 0 && n_out > 0 && k_in > 0, WQ_ERR_INVALID, "pack_fp8: bad sizes");
        const bool il = (flags & WQ_PACK_INTERLEAVE_GATE_UP) != 0;
        WQ_REQUIRE(n_out % (il ? 32 : 16) == 0, WQ_ERR_UNSUPPORTED, "pack_fp8: n_out %d", n_out);
        WQ_REQUIRE(k_in % wq::FP8_KCHUNK == 0, WQ_ERR_UNSUPPORTED, "pack_fp8: k_in %d not a multiple of %d", k_in,
                   wq::FP8_KCHUNK);
        WQ_REQUIRE(codes && scales && packed && scales_packed, WQ_ERR_INVALID, "pack_fp8: NULL buffer");
        for (size_t i = 0, n = (size_t)E * n_out * k_in; i < n; ++i)
            WQ_REQUIRE((codes[i] & 0x7f) != 0x7f, WQ_ERR_INVALID, "pack_fp8: NaN code at %zu", i);
        for (size_t i = 0, n = (size_t)E * n_out; i < n; ++i)
            WQ_REQUIRE(std::isfinite(scales[i]), WQ_ERR_INVALID, "pack_fp8: non-finite scale at %zu", i);
        const int rows_perm = il ? n_out / 2 : n_out;
        WQ_TRY(check_row_perm(E, rows_perm, row_perm));
        const int C = k_in / wq::FP8_KCHUNK;
        const size_t expert_bytes = (size_t)n_out * k_in;
        uint8_t* out = static_cast<uint8_t*>(packed);
        parallel_for(E * (n_out / 16), [&](int job) {
            const int e = job / (n_out / 16), t = job % (n_out / 16);
            const int32_t* pe = row_perm ? row_perm + (size_t)e * rows_perm : nullptr;
            for (int l = 0; l < 64; ++l) {
                const int p = t * 16 + (l & 15);
                const uint8_t* qr = codes + ((size_t)e * n_out + logical_row(p, n_out, il, pe)) * k_in;
                for (int c = 0; c < C; ++c)
                    for (int h = 0; h < 2; ++h)
                        std::memcpy(out + (size_t)e * expert_bytes + ((size_t)t * C + c) * 2048 + 1024 * h + 16 * l,
                                    qr + (size_t)wq::FP8_KCHUNK * c + 32 * (l >> 4) + 16 * h, 16);
            }
            if (t == 0)
                for (int pp = 0; pp < n_out; ++pp)
                    scales_packed[(size_t)e * n_out + pp] = scales[(size_t)e * n_out + logical_row(pp, n_out, il, pe)];
        });
        return ok();
    } catch (...) {
        return fail(WQ_ERR_INVALID, "pack_fp8: unexpected exception");
    }
}

size_t wq_pack_sparse24_vals_bytes(int N, int K, int bits) {
    if (N <= 0 || K <= 0 || N % 16 || K % 256 || (bits != 4 && bits != 8)) return 0;
    return (size_t)N * K / 2 * bits / 8;
}

size_t wq_pack_sparse24_meta_bytes(int N, int K) {
    if (N <= 0 || K <= 0 || N % 16 || K % 256) return 0;
    return (size_t)N * K / 8;
}

wq_status wq_pack_sparse24(int N, int K, int bits, int group_size, const int8_t* vals, const uint8_t* idx,
                           const uint16_t* scales, void* vals_packed, void* meta_packed, uint16_t* scales_packed) {
    try {
        WQ_REQUIRE(N > 0 && K > 0, WQ_ERR_INVALID, "pack_sparse24: bad sizes");
        WQ_REQUIRE(bits == 4 || bits == 8, WQ_ERR_UNSUPPORTED, "pack_sparse24: bits %d (4 or 8)", bits);
        WQ_REQUIRE(group_size == 128 || group_size == -1, WQ_ERR_UNSUPPORTED, "pack_sparse24: group_size %d",
                   group_size);
        WQ_REQUIRE(N % 16 == 0 && K % 256 == 0, WQ_ERR_UNSUPPORTED, "pack_sparse24: need N %% 16 == 0, K %% 256 == 0");
        WQ_REQUIRE(vals && idx && scales && vals_packed && meta_packed && scales_packed, WQ_ERR_INVALID,
                   "pack_sparse24: NULL buffer");
        const size_t half = (size_t)N * K / 2;
        for (size_t i = 0; i < half; i += 2) {
            WQ_REQUIRE(bits == 8 || (vals[i] >= -8 && vals[i] <= 7 && vals[i + 1] >= -8 && vals[i + 1] <= 7),
                       WQ_ERR_INVALID, "pack_sparse24: code out of [-8, 7]");
            WQ_REQUIRE(idx[i] < idx[i + 1] && idx[i + 1] <= 3, WQ_ERR_INVALID,
                       "pack_sparse24: keep positions must be ascending in 0..3");
        }
        const int C = K / 256;
        uint8_t* vo = static_cast<uint8_t*>(vals_packed);
        uint8_t* mo = static_cast<uint8_t*>(meta_packed);
        parallel_for(N / 16, [&](int t) {
            for (int l = 0; l < 64; ++l) {
                const int n = t * 16 + (l & 15);
                const int8_t* vr = vals + (size_t)n * (K / 2);
                const uint8_t* ir = idx + (size_t)n * (K / 2);
                for (int c = 0; c < C; ++c) {
                    // lane l's values: 16 bytes (4-bit) or 32 bytes (8-bit) per chunk
                    uint8_t* vd = vo + (((size_t)t * C + c) * 64 + l) * (size_t)(4 * bits);
                    uint16_t* md = reinterpret_cast<uint16_t*>(mo + (((size_t)t * C + c) * 64 + l) * 8);
                    for (int st = 0; st < 4; ++st) {
                        const int g4 = (256 * c + 64 * st + 16 * (l >> 4)) / 4;  // first group of 4 of this lane
                        uint32_t d = 0;
                        uint32_t m = 0;
                        for (int b = 0; b < 4; ++b) {
                            for (int h = 0; h < 2; ++h) {
                                const int j = 2 * b + h;
                                const size_t v = (size_t)2 * (g4 + b) + h;
                                if (bits == 4) d |= (uint32_t)(vr[v] + 8) << (4 * (j >> 1) + 16 * (j & 1));
                                else vd[8 * st + j] = (uint8_t)vr[v];  // two's complement, natural order
                                m |= (uint32_t)ir[v] << (4 * b + 2 * h);
                            }
                        }
                        if (bits == 4) std::memcpy(vd + 4 * st, &d, 4);
                        md[st] = (uint16_t)m;
                    }
                }
            }
        });
        std::memcpy(scales_packed, scales, sizeof(uint16_t) * (size_t)(group_size == -1 ? 1 : K / 128) * N);
        return ok();
    } catch (...) {
        return fail(WQ_ERR_INVALID, "pack_sparse24: unexpected exception");
    }
}

}  // extern "C"

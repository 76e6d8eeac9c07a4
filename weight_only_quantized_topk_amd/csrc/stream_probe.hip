// stream_probe.hip -- the read bandwidth a plain streaming kernel reaches on
// this GPU for a given number of bytes: the practical ceiling against which
// the weight-streaming (small-batch) kernels of the library are read.
//
//   stream_probe [bytes ...]      (default: 58720256 117440512 234881024 352321536 1073741824)
//
// Each size is read R = 7 times by each of four launch shapes (4096 or 8192
// workgroups of 256 threads, 4 or 8 16-byte nontemporal loads in flight per
// thread), every read preceded by a 1 GiB read of another buffer so it starts
// from HBM, and timed with HIP events around the launch alone.  One JSON line
// per size: the best shape's best and median time and bandwidth.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <vector>

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                                        \
    do {                                                                                \
        hipError_t e_ = (x);                                                            \
        if (e_ != hipSuccess) {                                                         \
            std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            std::exit(1);                                                               \
        }                                                                               \
    } while (0)

// thread t reads words t, t + S, t + 2 S, ... (S = threads in the grid), U
// loads issued before they are combined; one xor per thread is written so
// nothing is optimised away
template <int U>
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ p, size_t n, unsigned* __restrict__ out) {
    const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    size_t i = tid;
    for (; i + (size_t)(U - 1) * stride < n; i += (size_t)U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int k = 0; k < U; ++k) v[k] = __builtin_nontemporal_load(p + i + k * stride);
#pragma unroll
        for (int k = 0; k < U; ++k) acc ^= v[k];
    }
    for (; i < n; i += stride) acc ^= p[i];
    out[tid] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

int main(int argc, char** argv) {
    std::vector<size_t> sizes;
    for (int i = 1; i < argc; ++i) sizes.push_back(std::strtoull(argv[i], nullptr, 10));
    if (sizes.empty()) sizes = {58720256ull, 117440512ull, 234881024ull, 352321536ull, 1073741824ull};
    const size_t flush_b = (size_t)1 << 30;
    size_t max_b = 0;
    for (size_t b : sizes) {
        if (b < 16 || b > ((size_t)4 << 30)) {
            std::fprintf(stderr, "sizes must be 16 B .. 4 GiB\n");
            return 2;
        }
        max_b = std::max(max_b, b);
    }
    const int grids[2] = {4096, 8192};
    u32x4 *flush, *data;
    unsigned* out;
    CHECK(hipMalloc(&flush, flush_b));
    CHECK(hipMalloc(&data, max_b));
    CHECK(hipMalloc(&out, (size_t)8192 * 256 * sizeof(unsigned)));
    CHECK(hipMemset(flush, 1, flush_b));
    CHECK(hipMemset(data, 2, max_b));
    hipEvent_t a, b;
    CHECK(hipEventCreate(&a));
    CHECK(hipEventCreate(&b));
    const int R = 7;
    for (size_t bytes : sizes) {
        const size_t n = bytes / 16;
        float best = 1e30f, best_med = 1e30f;
        int best_grid = 0, best_u = 0;
        for (int gi = 0; gi < 2; ++gi) {
            for (int u = 4; u <= 8; u += 4) {
                std::vector<float> t;
                for (int r = 0; r < R; ++r) {
                    hipLaunchKernelGGL(read_kernel<8>, dim3(8192), dim3(256), 0, 0, flush, flush_b / 16, out);
                    CHECK(hipEventRecord(a, 0));
                    if (u == 4) hipLaunchKernelGGL(read_kernel<4>, dim3(grids[gi]), dim3(256), 0, 0, data, n, out);
                    else hipLaunchKernelGGL(read_kernel<8>, dim3(grids[gi]), dim3(256), 0, 0, data, n, out);
                    CHECK(hipEventRecord(b, 0));
                    CHECK(hipEventSynchronize(b));
                    float ms = 0.f;
                    CHECK(hipEventElapsedTime(&ms, a, b));
                    t.push_back(ms);
                }
                std::sort(t.begin(), t.end());
                if (t[R / 2] < best_med) {
                    best_med = t[R / 2];
                    best = t[0];
                    best_grid = grids[gi];
                    best_u = u;
                }
            }
        }
        std::printf("{\"bytes\": %zu, \"grid\": %d, \"loads_in_flight\": %d, \"best_us\": %.2f, \"best_GBps\": %.0f, "
                    "\"median_us\": %.2f, \"median_GBps\": %.0f}\n",
                    bytes, best_grid, best_u, best * 1e3, bytes / (best * 1e-3) / 1e9, best_med * 1e3,
                    bytes / (best_med * 1e-3) / 1e9);
        std::fflush(stdout);
    }
    CHECK(hipDeviceSynchronize());
    CHECK(hipFree(flush));
    CHECK(hipFree(data));
    CHECK(hipFree(out));
    return 0;
}

// Streaming-read ceiling of the GPU: the HBM bandwidth a plain read kernel
// reaches (each thread sums 16-byte loads over a grid-stride loop with U
// independent loads in flight).  Prints one JSON line with the best of a sweep
// of grid sizes (1024..32768 workgroups of 256) and U (4, 8, 16).  A
// calibration aid for the decode roofline: the decode kernels are read
// streams, so this is the practical ceiling their HBM fraction is set against.
#include <hip/hip_runtime.h>

#include <cstdio>

#define CK(x)                                                                                      \
    do {                                                                                           \
        hipError_t e_ = (x);                                                                       \
        if (e_ != hipSuccess) {                                                                    \
            std::fprintf(stderr, "calib_read: %s (line %d)\n", hipGetErrorString(e_), __LINE__);   \
            return 1;                                                                              \
        }                                                                                          \
    } while (0)

template <int U>
__global__ void k_read(const float4 *__restrict__ p, size_t n, float *__restrict__ out)
{
    const size_t tid = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x;
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    float acc = 0.0f;
    size_t i = tid;
    for (; i + (U - 1) * stride < n; i += U * stride) {
        float4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = p[i + u * stride];
#pragma unroll
        for (int u = 0; u < U; ++u) acc += (v[u].x + v[u].y) + (v[u].z + v[u].w);
    }
    for (; i < n; i += stride) {
        const float4 v = p[i];
        acc += (v.x + v.y) + (v.z + v.w);
    }
    out[tid] = acc;     // keeps the loads live
}

template <int U>
static int time_read(const float4 *d, size_t n, float *out, int blocks, double &gbs)
{
    hipEvent_t a, b;
    CK(hipEventCreate(&a));
    CK(hipEventCreate(&b));
    for (int w = 0; w < 2; ++w) hipLaunchKernelGGL(k_read<U>, dim3(blocks), dim3(256), 0, 0, d, n, out);
    CK(hipGetLastError());
    constexpr int R = 10;
    CK(hipEventRecord(a));
    for (int r = 0; r < R; ++r) hipLaunchKernelGGL(k_read<U>, dim3(blocks), dim3(256), 0, 0, d, n, out);
    CK(hipEventRecord(b));
    CK(hipEventSynchronize(b));
    float ms = 0.0f;
    CK(hipEventElapsedTime(&ms, a, b));
    gbs = static_cast<double>(n) * 16.0 * R / (ms * 1e-3) / 1e9;
    CK(hipEventDestroy(a));
    CK(hipEventDestroy(b));
    return 0;
}

int main()
{
    const size_t bytes = static_cast<size_t>(2) << 30;
    const size_t n = bytes / 16;
    constexpr int kMaxBlocks = 32768;
    float4 *d = nullptr;
    float *out = nullptr;
    CK(hipMalloc(&d, bytes));
    CK(hipMemset(d, 0, bytes));
    CK(hipMalloc(&out, sizeof(float) * kMaxBlocks * 256));
    double best = 0.0;
    int best_blocks = 0, best_u = 0;
    for (int blocks = 1024; blocks <= kMaxBlocks; blocks *= 2) {
        double g[3] = {0.0, 0.0, 0.0};
        if (time_read<4>(d, n, out, blocks, g[0]) || time_read<8>(d, n, out, blocks, g[1]) ||
            time_read<16>(d, n, out, blocks, g[2]))
            return 1;
        for (int k = 0; k < 3; ++k)
            if (g[k] > best) {
                best = g[k];
                best_blocks = blocks;
                best_u = 4 << k;
            }
    }
    std::printf("{\"read_GBps\": %.1f, \"bytes\": %zu, \"blocks\": %d, \"threads\": 256, \"loads_in_flight\": %d}\n",
                best, bytes, best_blocks, best_u);
    CK(hipFree(d));
    CK(hipFree(out));
    return 0;
}

// Streaming-read ceiling of the GPU: the HBM bandwidth a plain read kernel
// reaches.  Four access patterns are timed, each thread summing 16-byte
// loads with U independent loads in flight: a grid-stride loop (consecutive
// threads on consecutive chunks, the grid stepping over the whole buffer) and
// per-workgroup contiguous slices, each with plain loads and with
// nontemporal ones (the "nt" bit).  Prints one JSON line with the best over
// grid sizes (1024..32768 workgroups of 256), U (4, 8, 16) and pattern, and
// the best of each pattern.  A calibration aid for the decode roofline: the
// decode kernels are read streams, so this is the practical ceiling their HBM
// fraction is set against.
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

typedef float f32x4 __attribute__((ext_vector_type(4)));

// MODE bit 0: nontemporal loads; bit 1: per-workgroup contiguous slices
// (n a multiple of the grid x 256 x U: the slices hold whole rounds)
template <int U, int MODE>
__global__ void k_read(const f32x4 *__restrict__ p, size_t n, float *__restrict__ out)
{
    constexpr bool NT = MODE & 1, SLICE = MODE & 2;
    const size_t per = SLICE ? n / gridDim.x : n;
    const f32x4 *q = SLICE ? p + blockIdx.x * per : p;
    const size_t first = SLICE ? threadIdx.x : blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x;
    const size_t stride = SLICE ? blockDim.x : static_cast<size_t>(gridDim.x) * blockDim.x;
    float acc = 0.0f;
    size_t i = first;
    for (; i + (U - 1) * stride < per; i += U * stride) {
        f32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = NT ? __builtin_nontemporal_load(q + i + u * stride) : q[i + u * stride];
#pragma unroll
        for (int u = 0; u < U; ++u) acc += (v[u].x + v[u].y) + (v[u].z + v[u].w);
    }
    for (; i < per; i += stride) {
        const f32x4 v = q[i];
        acc += (v.x + v.y) + (v.z + v.w);
    }
    out[blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x] = acc;     // keeps the loads live
}

template <int U, int MODE>
static int time_read(const f32x4 *d, size_t n, float *out, int blocks, double &gbs)
{
    hipEvent_t a, b;
    CK(hipEventCreate(&a));
    CK(hipEventCreate(&b));
    for (int w = 0; w < 2; ++w) hipLaunchKernelGGL((k_read<U, MODE>), dim3(blocks), dim3(256), 0, 0, d, n, out);
    CK(hipGetLastError());
    constexpr int R = 10;
    CK(hipEventRecord(a));
    for (int r = 0; r < R; ++r) hipLaunchKernelGGL((k_read<U, MODE>), dim3(blocks), dim3(256), 0, 0, d, n, out);
    CK(hipEventRecord(b));
    CK(hipEventSynchronize(b));
    float ms = 0.0f;
    CK(hipEventElapsedTime(&ms, a, b));
    gbs = static_cast<double>(n) * 16.0 * R / (ms * 1e-3) / 1e9;
    CK(hipEventDestroy(a));
    CK(hipEventDestroy(b));
    return 0;
}

template <int MODE>
static int sweep(const f32x4 *d, size_t n, float *out, double &best, int &best_blocks, int &best_u)
{
    constexpr int kMaxBlocks = 32768;
    best = 0.0;
    for (int blocks = 1024; blocks <= kMaxBlocks; blocks *= 2) {
        double g[3] = {0.0, 0.0, 0.0};
        if (time_read<4, MODE>(d, n, out, blocks, g[0]) || time_read<8, MODE>(d, n, out, blocks, g[1]) ||
            time_read<16, MODE>(d, n, out, blocks, g[2]))
            return 1;
        for (int k = 0; k < 3; ++k)
            if (g[k] > best) {
                best = g[k];
                best_blocks = blocks;
                best_u = 4 << k;
            }
    }
    return 0;
}

int main()
{
    // 2 GiB: n = 2^27 chunks, a multiple of every grid x 256 x 16 swept
    const size_t bytes = static_cast<size_t>(2) << 30;
    const size_t n = bytes / 16;
    f32x4 *d = nullptr;
    float *out = nullptr;
    CK(hipMalloc(&d, bytes));
    CK(hipMemset(d, 0, bytes));
    CK(hipMalloc(&out, sizeof(float) * 32768 * 256));
    constexpr const char *kName[4] = {"grid_stride", "grid_stride_nt", "slices", "slices_nt"};
    double g[4];
    int blocks[4], u[4];
    if (sweep<0>(d, n, out, g[0], blocks[0], u[0]) || sweep<1>(d, n, out, g[1], blocks[1], u[1]) ||
        sweep<2>(d, n, out, g[2], blocks[2], u[2]) || sweep<3>(d, n, out, g[3], blocks[3], u[3]))
        return 1;
    int k = 0;
    for (int m = 1; m < 4; ++m)
        if (g[m] > g[k]) k = m;
    std::printf("{\"read_GBps\": %.1f, \"bytes\": %zu, \"blocks\": %d, \"threads\": 256, \"loads_in_flight\": %d, "
                "\"pattern\": \"%s\", \"patterns_GBps\": {", g[k], bytes, blocks[k], u[k], kName[k]);
    for (int m = 0; m < 4; ++m) std::printf("%s\"%s\": %.1f", m ? ", " : "", kName[m], g[m]);
    std::printf("}}\n");
    CK(hipFree(d));
    CK(hipFree(out));
    return 0;
}

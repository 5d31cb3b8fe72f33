// Matrix-core ceiling of the GPU: the sustained rate of the three MFMA shapes
// libtq's kernels issue (v_mfma_f32_16x16x32_bf16 in the key compressor,
// v_mfma_f32_16x16x32_f16 in the value accumulation, v_mfma_i32_16x16x64_i8
// in the exact-digit scores).  Each wave runs a long stream of independent
// products (8 accumulators, operands in registers, nothing else in the loop);
// the best over grids of 1, 2, 4 and 8 workgroups of 4 waves per CU is
// printed as one JSON line, next to the published dense peaks.  A
// calibration aid for the compressor's roofline, as the streaming-read
// program is for the decode kernels.  It also times a mix of MFMA-only and
// VALU-only waves on each SIMD, which shows whether the two pipes overlap.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <type_traits>

#define CK(x)                                                                                      \
    do {                                                                                           \
        hipError_t e_ = (x);                                                                       \
        if (e_ != hipSuccess) {                                                                    \
            std::fprintf(stderr, "calib_mfma: %s (line %d)\n", hipGetErrorString(e_), __LINE__);   \
            return 1;                                                                              \
        }                                                                                          \
    } while (0)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kAcc = 8;        // independent accumulators per wave

enum Kind { kBf16 = 0, kF16 = 1, kI8 = 2 };

// operations of one product: 2 M N K
constexpr double kOps[3] = {2.0 * 16 * 16 * 32, 2.0 * 16 * 16 * 32, 2.0 * 16 * 16 * 64};
// published dense peaks (TFLOP/s, TOP/s for int8)
constexpr double kPeak[3] = {2500.0, 2500.0, 5000.0};
constexpr const char *kName[3] = {"bf16_16x16x32", "f16_16x16x32", "i8_16x16x64"};

template <int KIND>
__global__ __launch_bounds__(256) void k_mfma(const uint4 *__restrict__ in, float *__restrict__ out, int iters)
{
    using Acc = typename std::conditional<KIND == kI8, i32x4, f32x4>::type;
    const int lane = threadIdx.x & 63;
    const uint4 a = in[lane], b = in[64 + lane];
    const uint4 c0 = in[lane ^ 1];
    Acc acc[kAcc];
#pragma unroll
    for (int u = 0; u < kAcc; ++u)      // distinct starting values: eight independent chains
        acc[u] = __builtin_bit_cast(Acc, make_uint4(c0.x + u, c0.y, c0.z, c0.w));
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < kAcc; ++u) {
            if constexpr (KIND == kBf16)
                acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                                 __builtin_bit_cast(bf16x8, b), acc[u], 0, 0, 0);
            else if constexpr (KIND == kF16)
                acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                                __builtin_bit_cast(f16x8, b), acc[u], 0, 0, 0);
            else
                acc[u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a),
                                                               __builtin_bit_cast(i32x4, b), acc[u], 0, 0, 0);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int u = 0; u < kAcc; ++u) s += static_cast<float>(acc[u][0] + acc[u][1] + acc[u][2] + acc[u][3]);
    out[blockIdx.x * 256 + threadIdx.x] = s;     // keeps the products live
}

// Whether MFMA and VALU work of different waves on one SIMD overlap:
// 512-thread workgroups (two waves per SIMD, two workgroups per CU); mode 0:
// every wave runs MFMAs, 1: every wave fp32 FMAs (16 independent chains), 2:
// waves 0-3 MFMAs and waves 4-7 FMAs.  With overlap, mode 2 would take about
// max(mode 0, mode 1) / 2; without, (mode 0 + mode 1) / 2.
__global__ __launch_bounds__(512) void k_mix(const uint4 *__restrict__ in, float *__restrict__ out, int mode, int nm, int nv)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const bool mfma = mode == 0 || (mode == 2 && wave < 4);
    float s = 0.0f;
    if (mfma) {
        const uint4 a = in[lane], b = in[64 + lane];
        f32x4 acc[kAcc];
#pragma unroll
        for (int u = 0; u < kAcc; ++u) acc[u] = f32x4{static_cast<float>(u), 0.0f, 0.0f, static_cast<float>(lane)};
        for (int it = 0; it < nm; ++it) {
#pragma unroll
            for (int u = 0; u < kAcc; ++u)
                acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                                 __builtin_bit_cast(bf16x8, b), acc[u], 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kAcc; ++u) s += acc[u][0] + acc[u][3];
    } else {
        float x[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) x[u] = static_cast<float>(in[lane].x & 0xff) * 1e-3f + static_cast<float>(u);
        for (int it = 0; it < nv; ++it) {
#pragma unroll
            for (int u = 0; u < 16; ++u) x[u] = __builtin_fmaf(x[u], 0.999f, 1e-3f);
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) s += x[u];
    }
    out[blockIdx.x * 512 + threadIdx.x] = s;
}

static int time_mix(const uint4 *in, float *out, int cus, double (&ms)[3])
{
    hipEvent_t e0, e1;
    CK(hipEventCreate(&e0));
    CK(hipEventCreate(&e1));
    const int blocks = 2 * cus, nm = 512, nv = 2048;
    for (int mode = 0; mode < 3; ++mode) {
        hipLaunchKernelGGL(k_mix, dim3(blocks), dim3(512), 0, 0, in, out, mode, nm, nv);
        CK(hipGetLastError());
        constexpr int R = 5;
        CK(hipEventRecord(e0));
        for (int r = 0; r < R; ++r) hipLaunchKernelGGL(k_mix, dim3(blocks), dim3(512), 0, 0, in, out, mode, nm, nv);
        CK(hipEventRecord(e1));
        CK(hipEventSynchronize(e1));
        float t = 0.0f;
        CK(hipEventElapsedTime(&t, e0, e1));
        ms[mode] = t / R;
    }
    CK(hipEventDestroy(e0));
    CK(hipEventDestroy(e1));
    return 0;
}

template <int KIND>
static int time_mfma(const uint4 *in, float *out, int blocks, int iters, double &rate)
{
    hipEvent_t e0, e1;
    CK(hipEventCreate(&e0));
    CK(hipEventCreate(&e1));
    hipLaunchKernelGGL(k_mfma<KIND>, dim3(blocks), dim3(256), 0, 0, in, out, iters);
    CK(hipGetLastError());
    constexpr int R = 5;
    CK(hipEventRecord(e0));
    for (int r = 0; r < R; ++r) hipLaunchKernelGGL(k_mfma<KIND>, dim3(blocks), dim3(256), 0, 0, in, out, iters);
    CK(hipEventRecord(e1));
    CK(hipEventSynchronize(e1));
    float ms = 0.0f;
    CK(hipEventElapsedTime(&ms, e0, e1));
    const double ops = static_cast<double>(blocks) * 4 * iters * kAcc * kOps[KIND] * R;
    rate = ops / (ms * 1e-3) / 1e12;
    CK(hipEventDestroy(e0));
    CK(hipEventDestroy(e1));
    return 0;
}

template <int KIND>
static int sweep(const uint4 *in, float *out, int cus, double &best, int &best_blocks)
{
    best = 0.0;
    best_blocks = 0;
    for (int per_cu = 1; per_cu <= 8; per_cu *= 2) {
        double r = 0.0;
        if (time_mfma<KIND>(in, out, cus * per_cu, 2048, r)) return 1;
        if (r > best) {
            best = r;
            best_blocks = cus * per_cu;
        }
    }
    return 0;
}

int main()
{
    int dev = 0, cus = 0;
    CK(hipGetDevice(&dev));
    CK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    uint4 *in = nullptr;
    float *out = nullptr;
    CK(hipMalloc(&in, sizeof(uint4) * 128));
    CK(hipMemset(in, 0x11, sizeof(uint4) * 128));     // small finite operands of every type
    CK(hipMalloc(&out, sizeof(float) * 256 * cus * 8));     // also 512 x 2 cus for the mix
    double rate[3];
    int blocks[3];
    if (sweep<kBf16>(in, out, cus, rate[0], blocks[0]) || sweep<kF16>(in, out, cus, rate[1], blocks[1]) ||
        sweep<kI8>(in, out, cus, rate[2], blocks[2]))
        return 1;
    std::printf("{\"cus\": %d", cus);
    for (int k = 0; k < 3; ++k)
        std::printf(", \"%s\": {\"measured\": %.1f, \"peak\": %.1f, \"frac\": %.3f, \"blocks\": %d}", kName[k], rate[k],
                    kPeak[k], rate[k] / kPeak[k], blocks[k]);
    double mix[3];
    if (time_mix(in, out, cus, mix)) return 1;
    std::printf(", \"unit\": \"TFLOP/s (TOP/s for i8)\", \"mfma_valu_mix_ms\": {\"mfma_only\": %.4f, \"valu_only\": %.4f, "
                "\"half_each\": %.4f, \"if_overlapped\": %.4f, \"if_serial\": %.4f}}\n",
                mix[0], mix[1], mix[2], 0.5 * (mix[0] > mix[1] ? mix[0] : mix[1]), 0.5 * (mix[0] + mix[1]));
    CK(hipFree(in));
    CK(hipFree(out));
    return 0;
}

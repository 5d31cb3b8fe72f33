// Compression of keys into the rotated scalar block formats for gfx950 (the
// comparison the tproger.ru article reports in its section "First
// benchmarks": Q8_0 and Q4_0 with rotation).  x = Pi k, then per 32
// consecutive rotated coordinates one fp16 scale amax / qmax and signed codes
// round_half_even(x / scale) clamped to +-qmax.
//
// One workgroup takes 32 keys.  The keys are staged in LDS as fp32 (exact for
// every input dtype); thread (channel c, key group) accumulates x[key][c] in
// fp64 from the fp64 Pi^T (one coalesced row read serves all its keys), so the
// rotated key is exact to fp64 rounding and the codes match the exact ones
// but for ties.  A block of 32 channels is 32 adjacent lanes: its maximum is a
// 5-step shuffle reduction.  Codes and scales are staged in LDS and stored as
// whole rows.
#include "tq_internal.h"
#include "tq_device.h"

#include <cmath>

namespace tq {
namespace {

constexpr int kThreads = 256;
constexpr int kKeys = 32;

template <typename TIn, int BITS, int D>
__global__ __launch_bounds__(kThreads) void k_compress_keys_block(BlockLaunch a, int64_t n_total)
{
    constexpr int KG = kThreads / D;           // key groups
    constexpr int KPT = kKeys / KG;            // keys per thread
    constexpr int NB = D / 32;
    constexpr int QMAX = BITS == 8 ? 127 : 7;
    constexpr int ROWB = D * BITS / 8;         // code bytes per key
    __shared__ float ks[kKeys][D];
    __shared__ uint8_t cs[kKeys][D];           // one code byte per coordinate (q, or q + 8)
    __shared__ uint16_t ss[kKeys][NB];
    __shared__ const TIn *kp[kKeys];
    const int tid = threadIdx.x;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kKeys;
    const int nk = static_cast<int>(n_total - n0 < kKeys ? n_total - n0 : kKeys);
    if (tid < kKeys) {
        const int64_t n = n0 + (tid < nk ? tid : 0);
        const int64_t t = n % a.T, bh = n / a.T, b = bh / a.H, h = bh - b * a.H;
        kp[tid] = static_cast<const TIn *>(a.k) + b * a.sb + h * a.sh + t * a.st;
    }
    __syncthreads();
    for (int i = tid; i < kKeys * (D / 8); i += kThreads) {
        const int key = i / (D / 8), c8 = i % (D / 8);
        float v[8];
        load8_as_f32(kp[key] + 8 * c8, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) ks[key][8 * c8 + e] = key < nk ? v[e] : 0.0f;
    }
    __syncthreads();
    const int c = tid % D, kg = tid / D;
    double x[KPT];
#pragma unroll
    for (int u = 0; u < KPT; ++u) x[u] = 0.0;
    for (int j = 0; j < D; ++j) {
        const double p = a.pi64T[static_cast<int64_t>(j) * D + c];
#pragma unroll
        for (int u = 0; u < KPT; ++u) x[u] = fma(p, static_cast<double>(ks[kg + KG * u][j]), x[u]);
    }
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
        // block maximum over the 32 lanes of this channel block
        double m = fabs(x[u]);
#pragma unroll
        for (int off = 1; off < 32; off <<= 1) m = fmax(m, __shfl_xor(m, off));
        const uint32_t sh = f64_to_f16_rne(m / QMAX);
        const double sc = static_cast<double>(f16_bits_to_f32(sh));
        int q = 0;
        if (sc > 0.0) {
            const double r = rint(x[u] / sc);
            q = static_cast<int>(r > QMAX ? QMAX : (r < -QMAX ? -QMAX : r));
        }
        const int key = kg + KG * u;
        cs[key][c] = static_cast<uint8_t>(BITS == 8 ? q : q + 8);
        if ((c & 31) == 0) ss[key][c / 32] = static_cast<uint16_t>(sh);
    }
    __syncthreads();
    // whole rows: codes (bytes, or two nibbles per byte, element j at bits 4j..4j+3)
    uint32_t *codes = reinterpret_cast<uint32_t *>(a.out.codes) + n0 * (ROWB / 4);
    for (int i = tid; i < nk * (ROWB / 4); i += kThreads) {
        const int key = i / (ROWB / 4), w = i % (ROWB / 4);
        uint32_t word = 0;
        if constexpr (BITS == 8) {
#pragma unroll
            for (int e = 0; e < 4; ++e) word |= static_cast<uint32_t>(cs[key][4 * w + e]) << (8 * e);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) word |= static_cast<uint32_t>(cs[key][8 * w + e] & 15u) << (4 * e);
        }
        codes[i] = word;
    }
    uint16_t *scales = a.out.scales + n0 * NB;
    for (int i = tid; i < nk * NB; i += kThreads) scales[i] = ss[i / NB][i % NB];
}

template <typename TIn, int BITS>
hipError_t launch_kb_t(const BlockLaunch &a, hipStream_t stream, int64_t n)
{
    const dim3 grid(static_cast<unsigned>((n + kKeys - 1) / kKeys));
    if (a.d == 128) hipLaunchKernelGGL((k_compress_keys_block<TIn, BITS, 128>), grid, dim3(kThreads), 0, stream, a, n);
    else hipLaunchKernelGGL((k_compress_keys_block<TIn, BITS, 256>), grid, dim3(kThreads), 0, stream, a, n);
    return hipGetLastError();
}

template <typename TIn>
hipError_t launch_kb(const BlockLaunch &a, hipStream_t stream, int64_t n)
{
    return a.bits == 8 ? launch_kb_t<TIn, 8>(a, stream, n) : launch_kb_t<TIn, 4>(a, stream, n);
}

}  // namespace

hipError_t launch_compress_keys_block(const BlockLaunch &a, hipStream_t stream)
{
    const int64_t n = static_cast<int64_t>(a.B) * a.H * a.T;
    if (n == 0) return hipSuccess;
    void *tok;
    prof_begin("tq_compress_keys_block", stream, &tok);
    hipError_t e = hipErrorInvalidValue;
    switch (a.dtype) {
    case TQ_F32: e = launch_kb<float>(a, stream, n); break;
    case TQ_BF16: e = launch_kb<bf16_t>(a, stream, n); break;
    case TQ_F16: e = launch_kb<f16_t>(a, stream, n); break;
    }
    prof_end(tok, stream);
    return e;
}

}  // namespace tq

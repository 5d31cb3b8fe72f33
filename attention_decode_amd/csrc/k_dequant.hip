// Explicit key estimates of a packed key cache for gfx950 ("turboquant-pytorch",
// section "What it does": the inverse of the two-stage encoding):
//   k_hat = n Pi^T ( c[idx] + sqrt(pi/2)/m rho S^T (2 s - 1) ),
// whose inner product with a query is the asymmetric score; with m = 0 (first
// stage alone) k_hat = n Pi^T c[idx].  Not on the decode path.
//
// One workgroup takes kKeys consecutive keys.  The rotated-domain estimate
// r_hat = c[idx] + kappa rho S^T sigma is built in LDS (S read row-major, so a
// matrix row is one coalesced read for all keys of the workgroup), then
// k_hat = n Pi^T r_hat with Pi read row-major the same way; thread (channel c,
// key group) keeps the sums of its keys in registers.
#include "tq_internal.h"
#include "tq_device.h"

#include <cmath>

namespace tq {
namespace {

constexpr int kThreads = 256;
constexpr int kKeys = 32;

// code j (width `bits`, LSB-first) of a packed row; reads a second byte only
// when the field crosses into it, so no read passes the end of the row
__device__ __forceinline__ uint32_t code_at(const uint8_t *row, int j, int bits)
{
    const int p = j * bits, b = p >> 3, s = p & 7;
    uint32_t v = row[b] >> s;
    if (s + bits > 8) v |= static_cast<uint32_t>(row[b + 1]) << (8 - s);
    return v & ((1u << bits) - 1u);
}

template <int D>
__global__ __launch_bounds__(kThreads) void k_dequant_keys(DequantLaunch a)
{
    constexpr int KG = kThreads / D;           // key groups (threads per channel)
    constexpr int KPT = kKeys / KG;            // keys per thread
    __shared__ float yr[kKeys][D];             // rotated-domain estimates
    __shared__ float sg[kKeys][D];             // QJL signs as +-1 (m = D rows)
    const int tid = threadIdx.x;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kKeys;
    const int nk = static_cast<int>(a.N - n0 < kKeys ? a.N - n0 : kKeys);
    const int bits = a.bits, M = a.m;
    const int64_t code_bytes = D * bits / 8;
    for (int e = tid; e < kKeys * D; e += kThreads) {
        const int key = e / D, j = e % D;
        float y = 0.0f, sv = 0.0f;
        if (key < nk) {
            y = a.centroids[code_at(a.codes + (n0 + key) * code_bytes, j, bits)];
            if (M > 0) sv = code_at(a.signs + (n0 + key) * (D / 8), j, 1) ? 1.0f : -1.0f;
        }
        yr[key][j] = y;
        sg[key][j] = sv;
    }
    __syncthreads();
    const int c = tid % D, kg = tid / D;
    if (M > 0) {
        // r_hat[key][c] += kappa rho_key sum_i S[i][c] sigma[key][i]
        float acc[KPT];
#pragma unroll
        for (int u = 0; u < KPT; ++u) acc[u] = 0.0f;
        for (int i = 0; i < M; ++i) {
            const float s = a.s[static_cast<int64_t>(i) * D + c];
#pragma unroll
            for (int u = 0; u < KPT; ++u) acc[u] = fmaf(s, sg[kg + KG * u][i], acc[u]);
        }
        float f[KPT];
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
            const int key = kg + KG * u;
            f[u] = key < nk ? a.kappa * a.rnorm[n0 + key] : 0.0f;
        }
        __syncthreads();                       // every thread has read sg and yr
#pragma unroll
        for (int u = 0; u < KPT; ++u) yr[kg + KG * u][c] = fmaf(f[u], acc[u], yr[kg + KG * u][c]);
        __syncthreads();
    }
    // k_hat[key][c] = n_key sum_j Pi[j][c] r_hat[key][j]
    float acc[KPT];
#pragma unroll
    for (int u = 0; u < KPT; ++u) acc[u] = 0.0f;
    for (int j = 0; j < D; ++j) {
        const float p = a.pi[static_cast<int64_t>(j) * D + c];
#pragma unroll
        for (int u = 0; u < KPT; ++u) acc[u] = fmaf(p, yr[kg + KG * u][j], acc[u]);
    }
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
        const int key = kg + KG * u;
        if (key < nk) a.out[(n0 + key) * D + c] = a.knorm[n0 + key] * acc[u];
    }
}

}  // namespace

hipError_t launch_dequant_keys(const DequantLaunch &a, hipStream_t stream)
{
    if (a.N == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>((a.N + kKeys - 1) / kKeys));
    void *tok;
    prof_begin("tq_dequantize_keys", stream, &tok);
    switch (a.d) {
    case 64: hipLaunchKernelGGL(k_dequant_keys<64>, grid, dim3(kThreads), 0, stream, a); break;
    case 128: hipLaunchKernelGGL(k_dequant_keys<128>, grid, dim3(kThreads), 0, stream, a); break;
    case 256: hipLaunchKernelGGL(k_dequant_keys<256>, grid, dim3(kThreads), 0, stream, a); break;
    default: return hipErrorInvalidValue;
    }
    prof_end(tok, stream);
    return hipGetLastError();
}

}  // namespace tq

// Compression of keys into the rotated scalar block formats for gfx950 (the
// comparison the tproger.ru article reports in its section "First
// benchmarks": Q8_0 and Q4_0 with rotation).  x = Pi k, then per 32
// consecutive rotated coordinates one fp16 scale amax / qmax and signed codes
// round_half_even(x / scale) clamped to +-qmax.
//
// One workgroup takes 32 keys.  The keys are staged in LDS as fp64 (exact for
// every input dtype), transposed so that the 32 keys of one input coordinate
// are adjacent; thread (4 channels, key block) accumulates a 4-channel x
// key-block tile of x = Pi k in fp64 from the fp64 Pi^T over j in order (its
// keys come two at a time from 16-byte LDS reads the lanes of a key block
// share), so the rotated key is exact to fp64 rounding and the codes match
// the exact ones but for ties.  A block of 32 channels is 8 adjacent lanes:
// its maximum is a 3-step shuffle reduction.  Codes and scales are staged in
// LDS and stored as whole rows.
#include "tq_internal.h"
#include "tq_device.h"

#include <cmath>

namespace tq {
namespace {

constexpr int kThreads = 256;
constexpr int kKeys = 32;

template <int D>
constexpr size_t block_smem_bytes()
{
    return sizeof(double) * D * kKeys + static_cast<size_t>(kKeys) * D + sizeof(uint16_t) * kKeys * (D / 32);
}

template <typename TIn, int BITS, int D>
__global__ __launch_bounds__(kThreads, 2) void k_compress_keys_block(BlockLaunch a, int64_t n_total)
{
    constexpr int NB = D / 32;
    constexpr int QMAX = BITS == 8 ? 127 : 7;
    constexpr int ROWB = D * BITS / 8;         // code bytes per key
    extern __shared__ __align__(16) unsigned char smem_raw[];
    double *kT = reinterpret_cast<double *>(smem_raw);                                 // [D][kKeys]
    uint8_t (*cs)[D] = reinterpret_cast<uint8_t (*)[D]>(smem_raw + sizeof(double) * D * kKeys);   // code bytes
    uint16_t (*ss)[NB] = reinterpret_cast<uint16_t (*)[NB]>(smem_raw + sizeof(double) * D * kKeys + kKeys * D);
    const int tid = threadIdx.x;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kKeys;
    const int nk = static_cast<int>(n_total - n0 < kKeys ? n_total - n0 : kKeys);
    // staging: thread i loads 8 channels of key i % kKeys (consecutive lanes,
    // consecutive keys: the transposed stores are conflict-free)
    for (int i = tid; i < kKeys * (D / 8); i += kThreads) {
        const int key = i % kKeys, c8 = i / kKeys;
        const int64_t n = n0 + (key < nk ? key : 0);
        const int64_t t = n % a.T, bh = n / a.T, b = bh / a.H, h = bh - b * a.H;
        float v[8];
        load8_as_f32(static_cast<const TIn *>(a.k) + b * a.sb + h * a.sh + t * a.st + 8 * c8, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) kT[(8 * c8 + e) * kKeys + key] = key < nk ? static_cast<double>(v[e]) : 0.0;
    }
    __syncthreads();
    // products: thread (coordinate block cb of CB channels, key block kq of
    // KB keys) accumulates a CB x KB tile of x over j in order: per j, CB
    // entries of Pi^T's row j (one 16-byte-aligned run) and KB keys (shared
    // 16-byte LDS reads), CB KB fmas
    constexpr int CB = 4;                      // channels per thread
    constexpr int NCB = D / CB;                // channel blocks (lanes of a key block)
    constexpr int KB = kKeys * NCB / kThreads; // keys per thread
    static_assert(NCB * (kKeys / KB) == kThreads && KB % 2 == 0, "thread tiling");
    const int cb = tid % NCB, kq = tid / NCB;
    double x[KB][CB];
#pragma unroll
    for (int u = 0; u < KB; ++u)
#pragma unroll
        for (int i = 0; i < CB; ++i) x[u][i] = 0.0;
    const double *prow = a.pi64T + CB * cb;
#pragma unroll 2
    for (int j = 0; j < D; ++j) {
        const double2 p01 = *reinterpret_cast<const double2 *>(prow + static_cast<int64_t>(j) * D);
        const double2 p23 = *reinterpret_cast<const double2 *>(prow + static_cast<int64_t>(j) * D + 2);
        const double p[CB] = {p01.x, p01.y, p23.x, p23.y};
        const double2 *kr = reinterpret_cast<const double2 *>(kT + j * kKeys + kq * KB);
#pragma unroll
        for (int u = 0; u < KB / 2; ++u) {
            const double2 k2 = kr[u];
#pragma unroll
            for (int i = 0; i < CB; ++i) {
                x[2 * u][i] = fma(p[i], k2.x, x[2 * u][i]);
                x[2 * u + 1][i] = fma(p[i], k2.y, x[2 * u + 1][i]);
            }
        }
    }
    // a block of 32 channels is 32 / CB adjacent lanes
#pragma unroll
    for (int u = 0; u < KB; ++u) {
        double m = 0.0;
#pragma unroll
        for (int i = 0; i < CB; ++i) m = fmax(m, fabs(x[u][i]));
#pragma unroll
        for (int off = 1; off < 32 / CB; off <<= 1) m = fmax(m, __shfl_xor(m, off));
        const uint32_t sh = f64_to_f16_rne(m / QMAX);
        const double sc = static_cast<double>(f16_bits_to_f32(sh));
        const int key = kq * KB + u;
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            int q = 0;
            if (sc > 0.0) {
                const double r = rint(x[u][i] / sc);
                q = static_cast<int>(r > QMAX ? QMAX : (r < -QMAX ? -QMAX : r));
            }
            cs[key][CB * cb + i] = static_cast<uint8_t>(BITS == 8 ? q : q + 8);
        }
        if ((cb & (32 / CB - 1)) == 0) ss[key][CB * cb / 32] = static_cast<uint16_t>(sh);
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
    auto kern = a.d == 128 ? k_compress_keys_block<TIn, BITS, 128> : k_compress_keys_block<TIn, BITS, 256>;
    const size_t smem = a.d == 128 ? block_smem_bytes<128>() : block_smem_bytes<256>();
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(smem));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), smem, stream, a, n);
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

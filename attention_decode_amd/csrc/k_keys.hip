// Key compression for gfx950: norm, rotation, Lloyd-Max codes, residual norm
// and QJL signs, packed into the four key planes.  One 256-thread workgroup
// owns a tile of TK = 8192/D keys (32 KB of fp32 in LDS); the dense rotation
// and the QJL projection are fp32 tile products whose second operand (Pi^T or
// S^T) is streamed through LDS in 32-row chunks; the Hadamard rotation is an
// in-place butterfly on the LDS tile.  Method: discosf.com TurboQuant article,
// section "TurboQuant in one sentence", steps 1-3.
#include "tq_internal.h"
#include "tq_device.h"

namespace tq {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 32;   // rows of the streamed operand per LDS stage

template <int D>
struct KeyTile {
    static constexpr int TK = 8192 / D;        // keys per workgroup
    static constexpr int LPR = kThreads / TK;  // lanes per key row (2, 4, 8)
    static constexpr int OC = D / 16;          // outputs per thread in the products
    static constexpr int KR = TK / 16;         // key rows per thread in the products
    static constexpr int LD = D + 1;           // padded LDS row
};

struct KeySmem {
    float *u;         // [TK][D+1]  input -> rotated -> residual
    float *chunk;     // [kChunk][D]
    uint8_t *code8;   // [TK][D]
    uint8_t *sign8;   // [TK][D]
    float *inv_n;     // [TK]
    float *knorm;     // [TK]
    float *rnorm;     // [TK]
    float *cent;      // [256]
    float *bnd;       // [256]
};

// acc[kr][c] += U[ty*KR + kr][j] * Op[j][tx + 16 c] over j, Op streamed from global
template <int D>
__device__ __forceinline__ void tile_product(const KeySmem &s, const float *__restrict__ op,
                                             float (&acc)[KeyTile<D>::KR][KeyTile<D>::OC])
{
    using KT = KeyTile<D>;
    const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
#pragma unroll
    for (int kr = 0; kr < KT::KR; ++kr)
#pragma unroll
        for (int c = 0; c < KT::OC; ++c) acc[kr][c] = 0.0f;
    for (int j0 = 0; j0 < D; j0 += kChunk) {
        __syncthreads();
        // stage rows j0 .. j0+kChunk of the operand (each row D floats)
        const float4 *src = reinterpret_cast<const float4 *>(op + static_cast<size_t>(j0) * D);
        float4 *dst = reinterpret_cast<float4 *>(s.chunk);
        for (int i = tid; i < kChunk * D / 4; i += kThreads) dst[i] = src[i];
        __syncthreads();
#pragma unroll 4
        for (int jj = 0; jj < kChunk; ++jj) {
            float a[KT::KR], b[KT::OC];
#pragma unroll
            for (int kr = 0; kr < KT::KR; ++kr) a[kr] = s.u[(ty * KT::KR + kr) * KT::LD + j0 + jj];
#pragma unroll
            for (int c = 0; c < KT::OC; ++c) b[c] = s.chunk[jj * D + tx + 16 * c];
#pragma unroll
            for (int kr = 0; kr < KT::KR; ++kr)
#pragma unroll
                for (int c = 0; c < KT::OC; ++c) acc[kr][c] = fmaf(a[kr], b[c], acc[kr][c]);
        }
    }
}

template <int D, typename TIn>
__global__ __launch_bounds__(kThreads) void k_compress_keys(KeyLaunch a, int64_t n_total)
{
    using KT = KeyTile<D>;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    KeySmem s;
    {
        unsigned char *p = smem_raw;
        s.u = reinterpret_cast<float *>(p);        p += sizeof(float) * KT::TK * KT::LD;
        s.chunk = reinterpret_cast<float *>(p);    p += sizeof(float) * kChunk * D;
        s.inv_n = reinterpret_cast<float *>(p);    p += sizeof(float) * KT::TK;
        s.knorm = reinterpret_cast<float *>(p);    p += sizeof(float) * KT::TK;
        s.rnorm = reinterpret_cast<float *>(p);    p += sizeof(float) * KT::TK;
        s.cent = reinterpret_cast<float *>(p);     p += sizeof(float) * 256;
        s.bnd = reinterpret_cast<float *>(p);      p += sizeof(float) * 256;
        s.code8 = p;                               p += KT::TK * D;
        s.sign8 = p;
    }
    const int tid = threadIdx.x;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * KT::TK;
    const int L = 1 << a.bits;

    for (int i = tid; i < L; i += kThreads) s.cent[i] = a.centroids[i];
    for (int i = tid; i < L - 1; i += kThreads) s.bnd[i] = a.boundaries[i];

    // ---- 1. load the key tile as fp32 (8 channels per access)
    for (int i = tid; i < KT::TK * D / 8; i += kThreads) {
        const int r = i / (D / 8), j = (i % (D / 8)) * 8;
        const int64_t n = n0 + r;
        float v[8];
        if (n < n_total) {
            const int64_t t = n % a.T, bh = n / a.T;
            const int64_t b = bh / a.H, h = bh % a.H;
            const TIn *src = static_cast<const TIn *>(a.k) + b * a.sb + h * a.sh + t * a.st + j;
            load8_as_f32(src, v);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = 0.0f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) s.u[r * KT::LD + j + e] = v[e];
    }
    __syncthreads();

    // ---- 2. ||k|| in fp64, LPR lanes per row
    {
        const int r = tid / KT::LPR, part = tid % KT::LPR;
        double acc = 0.0;
        for (int j = part; j < D; j += KT::LPR) {
            const double x = s.u[r * KT::LD + j];
            acc = fma(x, x, acc);
        }
#pragma unroll
        for (int off = KT::LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, KT::LPR);
        if (part == 0) {
            const double n = sqrt(acc);
            s.knorm[r] = static_cast<float>(n);
            s.inv_n[r] = (n > 0.0) ? static_cast<float>((a.hadamard ? 1.0 / sqrt(double(D)) : 1.0) / n)
                                   : 0.0f;
        }
    }
    __syncthreads();

    // ---- 3. rotation: y = Pi k / n
    if (!a.hadamard) {
        float acc[KT::KR][KT::OC];
        tile_product<D>(s, a.piT, acc);
        __syncthreads();
        const int tx = tid % 16, ty = tid / 16;
#pragma unroll
        for (int kr = 0; kr < KT::KR; ++kr) {
            const int r = ty * KT::KR + kr;
            const float sc = s.inv_n[r];
#pragma unroll
            for (int c = 0; c < KT::OC; ++c) s.u[r * KT::LD + tx + 16 * c] = acc[kr][c] * sc;
        }
    } else {
        // y = H (D k) / (sqrt(d) n): sign flip, then log2(d) butterfly stages
        for (int i = tid; i < KT::TK * D; i += kThreads) {
            const int r = i / D, j = i % D;
            s.u[r * KT::LD + j] *= a.dsign[j];
        }
        for (int h = 1; h < D; h <<= 1) {
            __syncthreads();
            for (int p = tid; p < KT::TK * D / 2; p += kThreads) {
                const int r = p / (D / 2), q = p % (D / 2);
                const int j = (q / h) * 2 * h + (q % h);
                float *row = s.u + r * KT::LD;
                const float x = row[j], y = row[j + h];
                row[j] = x + y;
                row[j + h] = x - y;
            }
        }
        __syncthreads();
        for (int i = tid; i < KT::TK * D; i += kThreads) {
            const int r = i / D, j = i % D;
            s.u[r * KT::LD + j] *= s.inv_n[r];
        }
    }
    __syncthreads();

    // ---- 4. codes idx = #{boundaries < y}, residual r = y - c[idx], ||r||
    {
        const int r = tid / KT::LPR, part = tid % KT::LPR;
        double acc = 0.0;
        for (int j = part; j < D; j += KT::LPR) {
            const float y = s.u[r * KT::LD + j];
            int pos = 0;
            for (int step = L >> 1; step > 0; step >>= 1)
                if (s.bnd[pos + step - 1] < y) pos += step;
            const float res = y - s.cent[pos];
            s.u[r * KT::LD + j] = res;
            s.code8[r * D + j] = static_cast<uint8_t>(pos);
            acc = fma(double(res), double(res), acc);
        }
#pragma unroll
        for (int off = KT::LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, KT::LPR);
        if (part == 0) s.rnorm[r] = static_cast<float>(sqrt(acc));
    }
    __syncthreads();

    // ---- 5. QJL signs of z = S r
    {
        float acc[KT::KR][KT::OC];
        tile_product<D>(s, a.sT, acc);
        const int tx = tid % 16, ty = tid / 16;
#pragma unroll
        for (int kr = 0; kr < KT::KR; ++kr)
#pragma unroll
            for (int c = 0; c < KT::OC; ++c)
                s.sign8[(ty * KT::KR + kr) * D + tx + 16 * c] = acc[kr][c] >= 0.0f ? 1 : 0;
    }
    __syncthreads();

    // ---- 6. pack and store (rows of consecutive keys are contiguous)
    const int wc = D * a.bits / 32, ws = D / 32;
    uint32_t *codes = reinterpret_cast<uint32_t *>(a.out.codes) + n0 * wc;
    for (int i = tid; i < KT::TK * wc; i += kThreads) {
        const int r = i / wc, w = i % wc;
        if (n0 + r >= n_total) continue;
        codes[i] = pack_word(s.code8 + r * D, w, a.bits);
    }
    uint32_t *signs = reinterpret_cast<uint32_t *>(a.out.signs) + n0 * ws;
    for (int i = tid; i < KT::TK * ws; i += kThreads) {
        const int r = i / ws, w = i % ws;
        if (n0 + r >= n_total) continue;
        signs[i] = pack_word(s.sign8 + r * D, w, 1);
    }
    if (tid < KT::TK && n0 + tid < n_total) {
        a.out.knorm[n0 + tid] = s.knorm[tid];
        a.out.rnorm[n0 + tid] = s.rnorm[tid];
    }
}

template <int D>
size_t key_smem_bytes()
{
    using KT = KeyTile<D>;
    return sizeof(float) * (KT::TK * KT::LD + kChunk * D + 3 * KT::TK + 512) + 2 * KT::TK * D;
}

template <int D, typename TIn>
hipError_t launch_keys_t(const KeyLaunch &a, hipStream_t stream)
{
    using KT = KeyTile<D>;
    const int64_t n = static_cast<int64_t>(a.B) * a.H * a.T;
    const size_t smem = key_smem_bytes<D>();
    auto kern = k_compress_keys<D, TIn>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    const int64_t blocks = (n + KT::TK - 1) / KT::TK;
    void *tok;
    prof_begin("tq_compress_keys", stream, &tok);
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), smem, stream, a, n);
    prof_end(tok, stream);
    return hipGetLastError();
}

template <typename TIn>
hipError_t launch_keys_d(const KeyLaunch &a, hipStream_t stream)
{
    switch (a.d) {
    case 64: return launch_keys_t<64, TIn>(a, stream);
    case 128: return launch_keys_t<128, TIn>(a, stream);
    case 256: return launch_keys_t<256, TIn>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_compress_keys(const KeyLaunch &a, hipStream_t stream)
{
    switch (a.dtype) {
    case TQ_F32: return launch_keys_d<float>(a, stream);
    case TQ_BF16: return launch_keys_d<bf16_t>(a, stream);
    case TQ_F16: return launch_keys_d<f16_t>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace tq

// Decode-side kernels for gfx950: query preparation, asymmetric scores on the
// packed keys, split-K decode attention with an online softmax, and the
// log-sum-exp merge of the splits.  Method: "turboquant-pytorch" (section
// "What it does": asymmetric scores computed directly on the compressed keys;
// example requests: attention over the compressed cache without full key
// dequantisation) and the discosf.com TurboQuant article (step 4, grouped
// value codes).
//
// Score of key t for query q (rotated query q_rot = Pi q, projected Sq = S q_rot):
//   n_t ( sum_j q_rot[j] c[idx_tj] + sqrt(pi/2)/m rho_t sum_i Sq_i (2 s_ti - 1) ).
#include "tq_internal.h"
#include "tq_device.h"

#include <cmath>

namespace tq {

int query_chunk(int G)
{
    int gc = 16;
    while (gc > 1 && (G % gc) != 0) gc >>= 1;
    return gc;
}

namespace {

constexpr int kThreads = 256;
constexpr int kTile = kDecodeTile;

__device__ __forceinline__ float load1_f32(const float *p) { return *p; }
__device__ __forceinline__ float load1_f32(const bf16_t *p) { return bf16_to_f32(p->bits); }
__device__ __forceinline__ float load1_f32(const f16_t *p) { return f16_bits_to_f32(p->bits); }

// ---------------------------------------------------------------- q-prep
template <typename TIn>
__global__ __launch_bounds__(kThreads) void k_qprep(DecodeLaunch a)
{
    __shared__ float qs[256], qr[256];
    const int row = blockIdx.x;                  // b * Hq + hq
    const int D = a.d, M = a.m, tid = threadIdx.x;
    const TIn *q = static_cast<const TIn *>(a.q) + static_cast<size_t>(row) * D;
    for (int i = tid; i < D; i += kThreads) qs[i] = load1_f32(q + i);
    __syncthreads();
    float *dst = a.qprep + static_cast<size_t>(row) * (D + M);
    if (tid < D) {
        float acc = 0.0f;
        for (int j = 0; j < D; ++j) acc = fmaf(a.piT[j * D + tid], qs[j], acc);
        qr[tid] = acc;
        dst[tid] = acc;
    }
    __syncthreads();
    if (tid < M) {
        float acc = 0.0f;
        for (int j = 0; j < D; ++j) acc = fmaf(a.sT[j * M + tid], qr[j], acc);
        dst[D + tid] = acc;
    }
}

// flip the sign of x unless bit e of w is set: +x for s = 1, -x for s = 0
__device__ __forceinline__ float signed_by_bit(float x, uint32_t w, int e)
{
    return __uint_as_float(__float_as_uint(x) ^ (((~w >> e) & 1u) << 31));
}

// the two inner sums of the score for one key row and GC queries (the sign
// sum only with QJL rows; qjl is uniform over the launch)
template <int BITS, int GC>
__device__ __forceinline__ void key_dots(const uint32_t *__restrict__ crow,
                                         const uint32_t *__restrict__ srow, int D, bool qjl,
                                         const float *qr_s, const float *sq_s, const float *cent_s,
                                         float (&dc)[GC], float (&ds)[GC])
{
#pragma unroll
    for (int g = 0; g < GC; ++g) dc[g] = ds[g] = 0.0f;
    for (int c0 = 0; c0 < D; c0 += 32) {
        uint32_t w[BITS + 1];
#pragma unroll
        for (int i = 0; i < BITS; ++i) w[i] = crow[(c0 / 32) * BITS + i];
        w[BITS] = 0;
        float cv[32];
#pragma unroll
        for (int e = 0; e < 32; ++e) {
            const int bit = BITS * e, wi = bit / 32, sh = bit % 32;
            uint32_t v = w[wi] >> sh;
            if (sh + BITS > 32) v |= w[wi + 1] << (32 - sh);
            cv[e] = cent_s[v & ((1u << BITS) - 1u)];
        }
#pragma unroll
        for (int e4 = 0; e4 < 8; ++e4) {
#pragma unroll
            for (int g = 0; g < GC; ++g) {
                const float4 q4 = *reinterpret_cast<const float4 *>(qr_s + g * D + c0 + 4 * e4);
                dc[g] = fmaf(q4.x, cv[4 * e4], dc[g]);
                dc[g] = fmaf(q4.y, cv[4 * e4 + 1], dc[g]);
                dc[g] = fmaf(q4.z, cv[4 * e4 + 2], dc[g]);
                dc[g] = fmaf(q4.w, cv[4 * e4 + 3], dc[g]);
            }
        }
        if (!qjl) continue;
        const uint32_t sw = srow[c0 / 32];
#pragma unroll
        for (int e4 = 0; e4 < 8; ++e4) {
#pragma unroll
            for (int g = 0; g < GC; ++g) {
                const float4 s4 = *reinterpret_cast<const float4 *>(sq_s + g * D + c0 + 4 * e4);
                ds[g] += signed_by_bit(s4.x, sw, 4 * e4) + signed_by_bit(s4.y, sw, 4 * e4 + 1) +
                         signed_by_bit(s4.z, sw, 4 * e4 + 2) + signed_by_bit(s4.w, sw, 4 * e4 + 3);
            }
        }
    }
}

struct UnitCoords {
    int b, hkv, hq0;
    int64_t bh;   // b * Hkv + hkv: row block of the packed planes
};

__device__ __forceinline__ UnitCoords unit_coords(const DecodeLaunch &a, int unit, int nqc, int gc)
{
    UnitCoords u;
    const int qc = unit % nqc;
    u.bh = unit / nqc;
    u.b = static_cast<int>(u.bh / a.Hkv);
    u.hkv = static_cast<int>(u.bh % a.Hkv);
    u.hq0 = u.hkv * (a.Hq / a.Hkv) + qc * gc;
    return u;
}

// stage GC query rows (q_rot | Sq) and the centroids into LDS
template <int GC>
__device__ __forceinline__ void stage_queries(const DecodeLaunch &a, const UnitCoords &u,
                                              float *qr_s, float *sq_s, float *cent_s)
{
    const int D = a.d, M = a.m, tid = threadIdx.x;
    for (int i = tid; i < GC * D; i += kThreads) {
        const int g = i / D, j = i % D;
        const float *row = a.qprep + (static_cast<size_t>(u.b) * a.Hq + u.hq0 + g) * (D + M);
        qr_s[i] = row[j];
        sq_s[i] = M > 0 ? row[D + j] : 0.0f;
    }
    for (int i = tid; i < (1 << a.bits); i += kThreads) cent_s[i] = a.centroids[i];
}

// ---------------------------------------------------------------- scores
template <int BITS, int GC>
__global__ __launch_bounds__(kThreads) void k_scores(DecodeLaunch a, int nqc, float kappa)
{
    extern __shared__ __align__(16) float sm[];
    float *qr_s = sm, *sq_s = qr_s + GC * a.d, *cent_s = sq_s + GC * a.d;
    const UnitCoords u = unit_coords(a, blockIdx.y, nqc, GC);
    stage_queries<GC>(a, u, qr_s, sq_s, cent_s);
    __syncthreads();
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (t >= a.T) return;
    const int64_t n = u.bh * a.T + t;
    const uint32_t *crow = reinterpret_cast<const uint32_t *>(a.kc.codes) + n * (a.d * BITS / 32);
    const uint32_t *srow = reinterpret_cast<const uint32_t *>(a.kc.signs) + n * (a.m / 32);
    float dc[GC], ds[GC];
    key_dots<BITS, GC>(crow, srow, a.d, a.m > 0, qr_s, sq_s, cent_s, dc, ds);
    const float nrm = a.kc.knorm[n], rho = a.m > 0 ? a.kc.rnorm[n] : 0.0f;
#pragma unroll
    for (int g = 0; g < GC; ++g)
        a.scores[(static_cast<int64_t>(u.b) * a.Hq + u.hq0 + g) * a.T + t] =
            nrm * fmaf(kappa * rho, ds[g], dc[g]);
}

// ---------------------------------------------------------- split-K attend
struct AttendSmem {
    float *qr, *sq, *cent, *p, *m, *l, *alpha, *vsz;
    uint8_t *vcode;
};

template <int GC>
__device__ __forceinline__ AttendSmem attend_smem(float *base, int D, int NG)
{
    AttendSmem s;
    s.qr = base;
    s.sq = s.qr + GC * D;
    s.cent = s.sq + GC * D;
    s.p = s.cent + 256;
    s.m = s.p + GC * kTile;
    s.l = s.m + 16;
    s.alpha = s.l + 16;
    s.vsz = s.alpha + 16;
    s.vcode = reinterpret_cast<uint8_t *>(s.vsz + 2 * kTile * NG);
    return s;
}

template <int BITS, int GC>
__global__ __launch_bounds__(kThreads) void k_attend(DecodeLaunch a, int nqc, float kappa, int64_t chunk)
{
    extern __shared__ __align__(16) float sm[];
    const int D = a.d, NG = D / a.group, VB = D * a.vbits / 8;
    const AttendSmem s = attend_smem<GC>(sm, D, NG);
    const UnitCoords u = unit_coords(a, blockIdx.y, nqc, GC);
    const int split = blockIdx.x, tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
    stage_queries<GC>(a, u, s.qr, s.sq, s.cent);
    if (tid < GC) {
        s.m[tid] = -INFINITY;
        s.l[tid] = 0.0f;
    }
    __shared__ int64_t s_rows[kTile];           // plane row of each token of the tile (-1: none)
    const int64_t t_begin = static_cast<int64_t>(split) * chunk;
    const int64_t len = seq_len_of(a.map, a.T, u.b);
    const int64_t t_end = t_begin + chunk < len ? t_begin + chunk : len;
    const int P = kThreads / D, part = tid / D, c = tid % D;
    const int span = kTile / P, grp = c / a.group;
    const uint32_t vmask = (1u << a.vbits) - 1u;
    const int vshift = (c * a.vbits) % 8, vbyte = c * a.vbits / 8;
    float acc[GC];
#pragma unroll
    for (int g = 0; g < GC; ++g) acc[g] = 0.0f;
    __syncthreads();

    for (int64_t tile0 = t_begin; tile0 < t_end; tile0 += kTile) {
        const int ntile = static_cast<int>(t_end - tile0 < kTile ? t_end - tile0 : kTile);
        // A. scaled scores of this thread's key
        {
            float lam[GC];
            int64_t n = -1;
            if (tid < ntile)
                n = a.map.mode == CacheMap::kPaged ? layout_row(a.map, a.Hkv, u.b, u.hkv, tile0 + tid)
                                                   : u.bh * a.T + tile0 + tid;
            s_rows[tid] = n;
            if (n >= 0) {
                const uint32_t *crow = reinterpret_cast<const uint32_t *>(a.kc.codes) + n * (D * BITS / 32);
                const uint32_t *srow = reinterpret_cast<const uint32_t *>(a.kc.signs) + n * (a.m / 32);
                float dc[GC], ds[GC];
                key_dots<BITS, GC>(crow, srow, D, a.m > 0, s.qr, s.sq, s.cent, dc, ds);
                const float nrm = a.kc.knorm[n], rho = a.m > 0 ? a.kc.rnorm[n] : 0.0f;
#pragma unroll
                for (int g = 0; g < GC; ++g) lam[g] = a.scale * (nrm * fmaf(kappa * rho, ds[g], dc[g]));
            } else {
#pragma unroll
                for (int g = 0; g < GC; ++g) lam[g] = -INFINITY;
            }
#pragma unroll
            for (int g = 0; g < GC; ++g) s.p[g * kTile + tid] = lam[g];
        }
        __syncthreads();        // token rows
        // stage the value tile: raw code rows and (scale, zero) as fp32 (tokens
        // without a row read as zero codes and zero parameters)
        {
            const uint4 *src = reinterpret_cast<const uint4 *>(a.vc.codes);
            uint4 *dst = reinterpret_cast<uint4 *>(s.vcode);
            const int cpr = VB / 16;                // 16-byte chunks per row
            for (int i = tid; i < ntile * cpr; i += kThreads) {
                const int64_t r = s_rows[i / cpr];
                dst[i] = r >= 0 ? src[r * cpr + i % cpr] : make_uint4(0u, 0u, 0u, 0u);
            }
            const uint32_t *par = reinterpret_cast<const uint32_t *>(a.vc.params);
            for (int i = tid; i < kTile * NG; i += kThreads) {
                float sc = 0.0f, ze = 0.0f;
                const int64_t r = i < ntile * NG ? s_rows[i / NG] : -1;
                if (r >= 0) {
                    const uint32_t w = par[r * NG + i % NG];
                    sc = f16_bits_to_f32(w & 0xffffu);
                    ze = f16_bits_to_f32(w >> 16);
                }
                s.vsz[2 * i] = sc;
                s.vsz[2 * i + 1] = ze;
            }
            for (int i = ntile * VB + tid; i < kTile * VB; i += kThreads) s.vcode[i] = 0;
        }
        __syncthreads();
        // B. online softmax update, one wave per query head
        for (int g = wave; g < GC; g += kThreads / 64) {
            float v[4], tmax = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[i] = s.p[g * kTile + lane * 4 + i];
                tmax = fmaxf(tmax, v[i]);
            }
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, off));
            const float m_old = s.m[g], m_new = fmaxf(m_old, tmax);
            float alpha = 1.0f, sum = 0.0f;
            if (m_new != -INFINITY) {
                alpha = expf(m_old - m_new);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[i] = expf(v[i] - m_new);
                    sum += v[i];
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = 0.0f;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) s.p[g * kTile + lane * 4 + i] = v[i];
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
            if (lane == 0) {
                s.m[g] = m_new;
                s.l[g] = s.l[g] * alpha + sum;
                s.alpha[g] = alpha;
            }
        }
        __syncthreads();
        // C. acc[g] = alpha acc[g] + sum_t p[g][t] v_hat[t][c] over this thread's span
#pragma unroll
        for (int g = 0; g < GC; ++g) acc[g] *= s.alpha[g];
        for (int tt = part * span; tt < (part + 1) * span; tt += 4) {
            float vh[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = tt + i;
                const uint32_t code = (s.vcode[t * VB + vbyte] >> vshift) & vmask;
                vh[i] = fmaf(static_cast<float>(code), s.vsz[2 * (t * NG + grp)], s.vsz[2 * (t * NG + grp) + 1]);
            }
#pragma unroll
            for (int g = 0; g < GC; ++g) {
                const float4 p4 = *reinterpret_cast<const float4 *>(s.p + g * kTile + tt);
                acc[g] = fmaf(p4.x, vh[0], acc[g]);
                acc[g] = fmaf(p4.y, vh[1], acc[g]);
                acc[g] = fmaf(p4.z, vh[2], acc[g]);
                acc[g] = fmaf(p4.w, vh[3], acc[g]);
            }
        }
        __syncthreads();
    }
    // merge the P partitions of the token span and write this split's partials
#pragma unroll
    for (int g = 0; g < GC; ++g) s.p[(part * GC + g) * D + c] = acc[g];
    __syncthreads();
    if (part == 0) {
        for (int g = 0; g < GC; ++g) {
            float sum = 0.0f;
            for (int p = 0; p < P; ++p) sum += s.p[(p * GC + g) * D + c];
            const int64_t row = static_cast<int64_t>(u.b) * a.Hq + u.hq0 + g;
            a.part_acc[(row * a.splits + split) * D + c] = sum;
        }
    }
    if (tid < GC) {
        const int64_t row = static_cast<int64_t>(u.b) * a.Hq + u.hq0 + tid;
        a.part_ml[(row * a.splits + split) * 2 + 0] = s.m[tid];
        a.part_ml[(row * a.splits + split) * 2 + 1] = s.l[tid];
    }
}

// ---------------------------------------------------------------- combine
__global__ __launch_bounds__(kThreads) void k_combine(DecodeLaunch a)
{
    const int64_t row = blockIdx.x;     // b * Hq + hq
    const int c = threadIdx.x;
    if (c >= a.d) return;
    const float *ml = a.part_ml + row * a.splits * 2;
    const float *acc = a.part_acc + row * a.splits * a.d;
    float mx = -INFINITY;
    for (int s = 0; s < a.splits; ++s)
        if (ml[2 * s + 1] > 0.0f) mx = fmaxf(mx, ml[2 * s]);
    float den = 0.0f, num = 0.0f;
    for (int s = 0; s < a.splits; ++s) {
        const float l = ml[2 * s + 1];
        if (l > 0.0f) {
            const float w = expf(ml[2 * s] - mx);
            den = fmaf(l, w, den);
            num = fmaf(acc[static_cast<int64_t>(s) * a.d + c], w, num);
        }
    }
    a.out[row * a.d + c] = den > 0.0f ? num / den : 0.0f;
}

__global__ void k_fill_zero(float *p, int64_t n)
{
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

template <int BITS>
hipError_t dispatch_scores(const DecodeLaunch &a, hipStream_t stream, int gc, int nqc, float kappa)
{
    const size_t smem = sizeof(float) * (2 * gc * a.d + 256);
    const dim3 grid(static_cast<unsigned>((a.T + kThreads - 1) / kThreads),
                    static_cast<unsigned>(static_cast<int64_t>(a.B) * a.Hkv * nqc));
    void *tok;
    prof_begin("tq_scores", stream, &tok);
    switch (gc) {
    case 1: hipLaunchKernelGGL((k_scores<BITS, 1>), grid, dim3(kThreads), smem, stream, a, nqc, kappa); break;
    case 2: hipLaunchKernelGGL((k_scores<BITS, 2>), grid, dim3(kThreads), smem, stream, a, nqc, kappa); break;
    case 4: hipLaunchKernelGGL((k_scores<BITS, 4>), grid, dim3(kThreads), smem, stream, a, nqc, kappa); break;
    case 8: hipLaunchKernelGGL((k_scores<BITS, 8>), grid, dim3(kThreads), smem, stream, a, nqc, kappa); break;
    default: hipLaunchKernelGGL((k_scores<BITS, 16>), grid, dim3(kThreads), smem, stream, a, nqc, kappa); break;
    }
    prof_end(tok, stream);
    return hipGetLastError();
}

template <int BITS, int GC>
hipError_t launch_attend_gc(const DecodeLaunch &a, hipStream_t stream, int nqc, float kappa, int64_t chunk)
{
    const int NG = a.d / a.group, VB = a.d * a.vbits / 8;
    const size_t smem = sizeof(float) * (2 * GC * a.d + 256 + GC * kTile + 48 + 2 * kTile * NG) +
                        static_cast<size_t>(kTile) * VB;
    auto kern = k_attend<BITS, GC>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    const dim3 grid(static_cast<unsigned>(a.splits),
                    static_cast<unsigned>(static_cast<int64_t>(a.B) * a.Hkv * nqc));
    void *tok;
    prof_begin("tq_attend_splitk", stream, &tok);
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), smem, stream, a, nqc, kappa, chunk);
    prof_end(tok, stream);
    return hipGetLastError();
}

template <int BITS>
hipError_t dispatch_attend(const DecodeLaunch &a, hipStream_t stream, int gc, int nqc, float kappa,
                           int64_t chunk)
{
    switch (gc) {
    case 1: return launch_attend_gc<BITS, 1>(a, stream, nqc, kappa, chunk);
    case 2: return launch_attend_gc<BITS, 2>(a, stream, nqc, kappa, chunk);
    case 4: return launch_attend_gc<BITS, 4>(a, stream, nqc, kappa, chunk);
    case 8: return launch_attend_gc<BITS, 8>(a, stream, nqc, kappa, chunk);
    default: return launch_attend_gc<BITS, 16>(a, stream, nqc, kappa, chunk);
    }
}

// sqrt(pi/2) / m; 0 for the first-stage format (no QJL rows)
float qjl_kappa(int m) { return m > 0 ? static_cast<float>(std::sqrt(M_PI / 2.0) / m) : 0.0f; }

}  // namespace

hipError_t launch_qprep(const DecodeLaunch &a, hipStream_t stream)
{
    const dim3 grid(static_cast<unsigned>(a.B * a.Hq));
    void *tok;
    prof_begin("tq_qprep", stream, &tok);
    switch (a.dtype) {
    case TQ_F32: hipLaunchKernelGGL(k_qprep<float>, grid, dim3(kThreads), 0, stream, a); break;
    case TQ_BF16: hipLaunchKernelGGL(k_qprep<bf16_t>, grid, dim3(kThreads), 0, stream, a); break;
    case TQ_F16: hipLaunchKernelGGL(k_qprep<f16_t>, grid, dim3(kThreads), 0, stream, a); break;
    }
    prof_end(tok, stream);
    return hipGetLastError();
}

hipError_t launch_scores(const DecodeLaunch &a, hipStream_t stream)
{
    if (a.T == 0) return hipSuccess;
    const int G = a.Hq / a.Hkv, gc = query_chunk(G), nqc = G / gc;
    const float kappa = qjl_kappa(a.m);
    switch (a.bits) {
    case 1: return dispatch_scores<1>(a, stream, gc, nqc, kappa);
    case 2: return dispatch_scores<2>(a, stream, gc, nqc, kappa);
    case 3: return dispatch_scores<3>(a, stream, gc, nqc, kappa);
    case 4: return dispatch_scores<4>(a, stream, gc, nqc, kappa);
    case 5: return dispatch_scores<5>(a, stream, gc, nqc, kappa);
    case 6: return dispatch_scores<6>(a, stream, gc, nqc, kappa);
    case 7: return dispatch_scores<7>(a, stream, gc, nqc, kappa);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_attend(const DecodeLaunch &a, hipStream_t stream)
{
    const int64_t n_out = static_cast<int64_t>(a.B) * a.Hq * a.d;
    if (a.T == 0) {
        hipLaunchKernelGGL(k_fill_zero, dim3(static_cast<unsigned>((n_out + 255) / 256)), dim3(256), 0,
                           stream, a.out, n_out);
        return hipGetLastError();
    }
    const int G = a.Hq / a.Hkv, gc = query_chunk(G), nqc = G / gc;
    const float kappa = qjl_kappa(a.m);
    const int64_t tiles = (a.T + kTile - 1) / kTile;
    const int64_t chunk = ((tiles + a.splits - 1) / a.splits) * kTile;
    hipError_t e = hipErrorInvalidValue;
    switch (a.bits) {
    case 1: e = dispatch_attend<1>(a, stream, gc, nqc, kappa, chunk); break;
    case 2: e = dispatch_attend<2>(a, stream, gc, nqc, kappa, chunk); break;
    case 3: e = dispatch_attend<3>(a, stream, gc, nqc, kappa, chunk); break;
    case 4: e = dispatch_attend<4>(a, stream, gc, nqc, kappa, chunk); break;
    case 5: e = dispatch_attend<5>(a, stream, gc, nqc, kappa, chunk); break;
    case 6: e = dispatch_attend<6>(a, stream, gc, nqc, kappa, chunk); break;
    case 7: e = dispatch_attend<7>(a, stream, gc, nqc, kappa, chunk); break;
    }
    if (e != hipSuccess) return e;
    void *tok;
    prof_begin("tq_combine", stream, &tok);
    hipLaunchKernelGGL(k_combine, dim3(static_cast<unsigned>(a.B * a.Hq)), dim3(kThreads), 0, stream, a);
    prof_end(tok, stream);
    return hipGetLastError();
}

}  // namespace tq

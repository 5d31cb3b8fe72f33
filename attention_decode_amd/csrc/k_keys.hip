// Key compression for gfx950 on the matrix cores: norm, rotation, Lloyd-Max
// codes, residual norm and QJL signs, packed into the four key planes.
// Method: discosf.com TurboQuant article, section "TurboQuant in one sentence",
// steps 1-3 (y = Pi k/||k||, nearest-centroid codes, signs of S r with
// r = y - c[idx]).
//
// One 256-thread workgroup encodes 64 keys (four 16-key tiles).  Both products
// run as v_mfma_f32_16x16x32_bf16 with the keys / residuals as the B operand
// (lane = key column) and the matrix as the A operand, so that every A
// fragment read from L2 serves 64 keys; the four waves split the output rows.
//
// Accuracy: the bf16 operands are made exact or near-fp32 by splitting.
//   * y:  Pi = P0 + P1 + P2 (three bf16 terms, about 24 significant bits); a
//         bf16 key is one exact term, an fp16 key two, an fp32 key three.  The
//         products kept are those whose term ranks sum to at most 2, i.e. every
//         product down to about 2^-24 of the leading one.  The Hadamard sign
//         matrix H D is exact in one term and its 1/sqrt(d) joins 1/||k||.
//   * z:  S = S0 + S1, r = R0 + R1 (16 bits each); S0 R0 + S0 R1 + S1 R0 leaves
//         an error near 2^-16 of |z| per term, far inside the resolution at
//         which a sign can legitimately flip.
// All sums accumulate in fp32 inside the MFMA.  ||k|| is summed in fp64 from
// the exact fp32 squares (each wave takes a quarter of the k-steps); ||r||
// in fp32 per lane and fp64 across lanes.
//
// Codes: idx = #{t_i < y}.  Up to 3 bits the boundaries sit in registers (at
// most seven comparisons, no dependent LDS reads); from 4 bits a uniform grid
// over [t_0, t_{L-2}] gives a lower bound of the count that is at most two
// below it, and two exact comparisons finish it.
#include "tq_internal.h"
#include "tq_device.h"

namespace tq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kKT = 4;              // 16-key tiles per workgroup
constexpr int kKeys = 16 * kKT;     // keys per workgroup

// bf16 terms that represent one input element exactly
template <typename TIn> struct KeyTerms;
template <> struct KeyTerms<bf16_t> { static constexpr int n = 1; };
template <> struct KeyTerms<f16_t> { static constexpr int n = 2; };
template <> struct KeyTerms<float> { static constexpr int n = 3; };

__device__ __forceinline__ uint32_t bf16_rne_bits(float x)
{
    uint32_t u = __float_as_uint(x);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float bf16_bits_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ f32x4 mfma_bf16(const uint4 &a, const uint4 &b, const f32x4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// split eight fp32 values into NT bf16x8 terms (x = t0 + t1 + ...)
template <int NT>
__device__ __forceinline__ void split_terms(const float (&x)[8], uint4 (&t)[NT])
{
    float rem[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) rem[e] = x[e];
#pragma unroll
    for (int p = 0; p < NT; ++p) {
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            h[e] = bf16_rne_bits(rem[e]);
            rem[e] -= bf16_bits_f32(h[e]);
        }
        t[p] = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
    }
}

// eight consecutive channels of one key as B-operand terms; with `norm`, their
// sum of squares is added to ss (each wave sums a quarter of the k-steps)
__device__ __forceinline__ void key_frag(const bf16_t *p, bool valid, uint4 (&t)[1], double &ss, bool norm)
{
    t[0] = valid ? *reinterpret_cast<const uint4 *>(p) : make_uint4(0, 0, 0, 0);
    if (norm) {
        const uint32_t w[4] = {t[0].x, t[0].y, t[0].z, t[0].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float lo = bf16_to_f32(w[i] & 0xffffu), hi = bf16_to_f32(w[i] >> 16);
            ss += static_cast<double>(lo * lo) + static_cast<double>(hi * hi);   // squares exact in fp32
        }
    }
}

template <typename TIn, int NT>
__device__ __forceinline__ void key_frag(const TIn *p, bool valid, uint4 (&t)[NT], double &ss, bool norm)
{
    float x[8];
    if (valid) {
        load8_as_f32(p, x);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.0f;
    }
    if (norm) {
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fma(static_cast<double>(x[e]), static_cast<double>(x[e]), ss);
    }
    split_terms<NT>(x, t);
}

// fp32 pair -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t bf16x2(float x0, float x1)
{
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    const bf2 v = {static_cast<__bf16>(x0), static_cast<__bf16>(x1)};
    return __builtin_bit_cast(uint32_t, v);
}

struct KeySmem {
    uint4 *rfrag;       // [kKT][KS][2][64]  residual B operands (two bf16 terms)
    uint32_t *cw;       // [kKeys][D * bits / 32]  code words
    uint32_t *sw;       // [kKeys][D / 32]         sign words
    double *rho2;       // [4 waves][kKeys]
    double *nrm2;       // [4 waves][kKeys]
    float *cent;        // [256]
    float *bnd;         // [256] (+inf after the last boundary)
    uint8_t *grid;      // [kMaxGrid]
};

template <int D, int BITS>
constexpr size_t key_smem_bytes()
{
    return sizeof(uint4) * kKT * (D / 32) * 2 * 64 + sizeof(uint32_t) * kKeys * (D * BITS / 32 + D / 32)
           + sizeof(double) * 8 * kKeys + sizeof(float) * 512 + (BITS >= 4 ? kMaxGrid : 0);
}

template <int D, typename TIn, int BITS>
__global__ __launch_bounds__(kThreads) void k_compress_keys(KeyLaunch a, int64_t n_total)
{
    constexpr int KS = D / 32;           // k-steps of 32 channels
    constexpr int RTW = D / 64;          // 16-row output tiles per wave
    constexpr int NK = KeyTerms<TIn>::n;
    constexpr int L = 1 << BITS;
    constexpr int CW = D * BITS / 32, SWN = D / 32;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    __shared__ int64_t s_row[kKeys];              // plane row of each key of the workgroup
    KeySmem s;
    {
        unsigned char *p = smem_raw;
        s.rfrag = reinterpret_cast<uint4 *>(p);   p += sizeof(uint4) * kKT * KS * 2 * 64;
        s.rho2 = reinterpret_cast<double *>(p);   p += sizeof(double) * 4 * kKeys;
        s.nrm2 = reinterpret_cast<double *>(p);   p += sizeof(double) * 4 * kKeys;
        s.cw = reinterpret_cast<uint32_t *>(p);   p += sizeof(uint32_t) * kKeys * CW;
        s.sw = reinterpret_cast<uint32_t *>(p);   p += sizeof(uint32_t) * kKeys * SWN;
        s.cent = reinterpret_cast<float *>(p);    p += sizeof(float) * 256;
        s.bnd = reinterpret_cast<float *>(p);     p += sizeof(float) * 256;
        s.grid = p;
    }
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, kb = lane >> 4;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kKeys;

    for (int i = tid; i < kKeys * CW; i += kThreads) s.cw[i] = 0u;
    for (int i = tid; i < kKeys * SWN; i += kThreads) s.sw[i] = 0u;
    for (int i = tid; i < L; i += kThreads) {
        s.cent[i] = a.centroids[i];
        s.bnd[i] = a.boundaries[i];      // entry L - 1 is +inf
    }
    if constexpr (BITS >= 4)
        for (int i = tid; i < a.ngrid; i += kThreads) s.grid[i] = a.grid[i];

    // rows of this lane's four keys: one divide per workgroup (wave-uniform),
    // then each lane steps from (b0, h0, t0) across sequence / head boundaries
    const TIn *kp[kKT];
    bool valid[kKT];
    {
        const int64_t bh0 = n0 / a.T, t0 = n0 - bh0 * a.T;
        const int64_t b0 = bh0 / a.H, h0 = bh0 - b0 * a.H;
#pragma unroll
        for (int kt = 0; kt < kKT; ++kt) {
            const int64_t n = n0 + 16 * kt + col;
            valid[kt] = n < n_total;
            int64_t t = t0 + (valid[kt] ? 16 * kt + col : 0), b = b0, h = h0;
            while (t >= a.T) {          // at most 64 / T + 1 steps
                t -= a.T;
                if (++h == a.H) {
                    h = 0;
                    ++b;
                }
            }
            kp[kt] = static_cast<const TIn *>(a.k) + b * a.sb + h * a.sh + t * a.st + 8 * kb;
        }
    }

    // ---- 1. y = Pi k (unnormalised), this wave's rows 16 (RTW wave + j) + 4 kb + r
    const uint4 *pif = reinterpret_cast<const uint4 *>(a.pifrag);
    const uint4 *sfr = reinterpret_cast<const uint4 *>(a.sfrag);
    f32x4 acc[RTW][kKT];
#pragma unroll
    for (int j = 0; j < RTW; ++j)
#pragma unroll
        for (int kt = 0; kt < kKT; ++kt) acc[j][kt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    double ss[kKT] = {0.0, 0.0, 0.0, 0.0};
    const int npp = a.hadamard ? 1 : 3;
    const int bits = BITS;
#pragma unroll 2
    for (int ks = 0; ks < KS; ++ks) {
        uint4 kf[kKT][NK];
#pragma unroll
        for (int kt = 0; kt < kKT; ++kt) key_frag(kp[kt] + 32 * ks, valid[kt], kf[kt], ss[kt], (ks & 3) == wave);
#pragma unroll
        for (int j = 0; j < RTW; ++j) {
            const int rt = wave * RTW + j;
            for (int pp = 0; pp < npp; ++pp) {
                const uint4 af = pif[((rt * KS + ks) * 3 + pp) * 64 + lane];
#pragma unroll
                for (int kq = 0; kq < NK; ++kq) {
                    if (!a.hadamard && pp + kq > 2) continue;
#pragma unroll
                    for (int kt = 0; kt < kKT; ++kt) acc[j][kt] = mfma_bf16(af, kf[kt][kq], acc[j][kt]);
                }
            }
        }
    }

    // ---- 2. ||k||: fp64 partial sums of this wave's k-steps, over the four lanes
    // that hold one key, then across the waves
#pragma unroll
    for (int kt = 0; kt < kKT; ++kt) {
        double t = ss[kt];
        t += __shfl_xor(t, 16);
        t += __shfl_xor(t, 32);
        if (kb == 0) s.nrm2[wave * kKeys + 16 * kt + col] = t;
    }
    __syncthreads();   // partial norms, cleared words, codebook tables
    float inv_n[kKT];
#pragma unroll
    for (int kt = 0; kt < kKT; ++kt) {
        const int key = 16 * kt + col;
        // 1/||k|| only scales y: fp32 rsqrt (about 1 ulp) moves y by ~1e-7 at most,
        // far inside the 1e-5 boundary band; the stored ||k|| is rounded from fp64
        const float n2 = static_cast<float>(s.nrm2[key] + s.nrm2[kKeys + key] + s.nrm2[2 * kKeys + key] + s.nrm2[3 * kKeys + key]);
        inv_n[kt] = (n2 > 0.0f) ? a.rot_scale * __builtin_amdgcn_rsqf(n2) : 0.0f;
    }
    float tb[BITS <= 3 ? L - 1 : 1];             // boundaries in registers (1-3 bits)
    if constexpr (BITS <= 3) {
#pragma unroll
        for (int i = 0; i < L - 1; ++i) tb[i] = s.bnd[i];
    }

    // ---- 3. codes idx = #{boundaries < y}, residual r = y - c[idx], ||r||
#pragma unroll
    for (int kt = 0; kt < kKT; ++kt) {
        const int key = 16 * kt + col;
        float rr = 0.0f;
#pragma unroll
        for (int j = 0; j < RTW; ++j) {
            const int rt = wave * RTW + j;
            uint32_t chunk = 0;
            float res[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float y = acc[j][kt][r] * inv_n[kt];
                int pos;
                if constexpr (BITS <= 3) {
                    pos = 0;
#pragma unroll
                    for (int i = 0; i < L - 1; ++i) pos += (y > tb[i]) ? 1 : 0;
                } else {
                    int c = static_cast<int>((y - a.grid_lo) * a.grid_scale);
                    c = c < 0 ? 0 : (c >= a.ngrid ? a.ngrid - 1 : c);
                    pos = s.grid[c];
                    pos += (y > s.bnd[pos]) ? 1 : 0;
                    pos += (y > s.bnd[pos]) ? 1 : 0;
                }
                res[r] = y - s.cent[pos];
                rr = fmaf(res[r], res[r], rr);
                chunk |= static_cast<uint32_t>(pos) << (bits * r);
            }
            // residual as two bf16 terms (hardware round to nearest even)
            const uint32_t h01 = bf16x2(res[0], res[1]), h23 = bf16x2(res[2], res[3]);
            const uint32_t l01 = bf16x2(res[0] - __uint_as_float(h01 << 16), res[1] - __uint_as_float(h01 & 0xffff0000u));
            const uint32_t l23 = bf16x2(res[2] - __uint_as_float(h23 << 16), res[3] - __uint_as_float(h23 & 0xffff0000u));
            // 4 codes of `bits` bits at bit offset bits (16 rt + 4 kb) of the key's stream
            const int off = bits * (16 * rt + 4 * kb), w = off >> 5, sh = off & 31;
            atomicOr(&s.cw[key * CW + w], chunk << sh);
            if (sh + 4 * bits > 32) atomicOr(&s.cw[key * CW + w + 1], chunk >> (32 - sh));
            // residual as B operand of k-step rt/2: elements 4 (rt % 2) + r of this lane
            uint32_t *dst = reinterpret_cast<uint32_t *>(&s.rfrag[((kt * KS + rt / 2) * 2 + 0) * 64 + lane]);
            uint32_t *dst1 = reinterpret_cast<uint32_t *>(&s.rfrag[((kt * KS + rt / 2) * 2 + 1) * 64 + lane]);
            const int hw = 2 * (rt & 1);
            *reinterpret_cast<uint2 *>(dst + hw) = make_uint2(h01, h23);
            *reinterpret_cast<uint2 *>(dst1 + hw) = make_uint2(l01, l23);
        }
        double rd = static_cast<double>(rr);
        rd += __shfl_xor(rd, 16);
        rd += __shfl_xor(rd, 32);
        if (kb == 0) s.rho2[wave * kKeys + key] = rd;
    }
    __syncthreads();

    // ---- 4. z = S r on this wave's rows; signs [z >= 0] (skipped for the
    // first-stage format, m = 0; the condition is uniform over the launch)
    const bool qjl = a.m > 0;
    if (qjl) {
    f32x4 zacc[RTW][kKT];
#pragma unroll
    for (int j = 0; j < RTW; ++j)
#pragma unroll
        for (int kt = 0; kt < kKT; ++kt) zacc[j][kt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 2
    for (int ks = 0; ks < KS; ++ks) {
        uint4 rf[kKT][2];
#pragma unroll
        for (int kt = 0; kt < kKT; ++kt) {
            rf[kt][0] = s.rfrag[((kt * KS + ks) * 2 + 0) * 64 + lane];
            rf[kt][1] = s.rfrag[((kt * KS + ks) * 2 + 1) * 64 + lane];
        }
#pragma unroll
        for (int j = 0; j < RTW; ++j) {
            const int rt = wave * RTW + j;
            const uint4 s0 = sfr[((rt * KS + ks) * 2 + 0) * 64 + lane];
            const uint4 s1 = sfr[((rt * KS + ks) * 2 + 1) * 64 + lane];
#pragma unroll
            for (int kt = 0; kt < kKT; ++kt) {
                zacc[j][kt] = mfma_bf16(s0, rf[kt][0], zacc[j][kt]);
                zacc[j][kt] = mfma_bf16(s0, rf[kt][1], zacc[j][kt]);
                zacc[j][kt] = mfma_bf16(s1, rf[kt][0], zacc[j][kt]);
            }
        }
    }
#pragma unroll
    for (int j = 0; j < RTW; ++j) {
        const int rt = wave * RTW + j;
        const int off = 16 * rt + 4 * kb;
#pragma unroll
        for (int kt = 0; kt < kKT; ++kt) {
            uint32_t nib = 0;
#pragma unroll
            for (int r = 0; r < 4; ++r) nib |= (zacc[j][kt][r] >= 0.0f ? 1u : 0u) << r;
            atomicOr(&s.sw[(16 * kt + col) * SWN + (off >> 5)], nib << (off & 31));
        }
    }
    __syncthreads();
    }

    // ---- 5. store the WG's keys: contiguous rows of every plane, or (when
    // appending to a layout cache) each key at its own row
    const int nk = static_cast<int>(n_total - n0 < kKeys ? n_total - n0 : kKeys);
    if (a.map.mode == CacheMap::kFlat) {
        uint32_t *codes = reinterpret_cast<uint32_t *>(a.out.codes) + n0 * CW;
        for (int i = tid; i < nk * CW; i += kThreads) codes[i] = s.cw[i];
        if (qjl) {
            uint32_t *signs = reinterpret_cast<uint32_t *>(a.out.signs) + n0 * SWN;
            for (int i = tid; i < nk * SWN; i += kThreads) signs[i] = s.sw[i];
        }
        if (tid < nk) s_row[tid] = n0 + tid;
    } else {
        if (tid < nk) s_row[tid] = out_row(a.map, a.H, a.T, n0 + tid);
        __syncthreads();
        uint32_t *codes = reinterpret_cast<uint32_t *>(a.out.codes);
        for (int i = tid; i < nk * CW; i += kThreads) {
            const int64_t r = s_row[i / CW];
            if (r >= 0) codes[r * CW + i % CW] = s.cw[i];
        }
        if (qjl) {
            uint32_t *signs = reinterpret_cast<uint32_t *>(a.out.signs);
            for (int i = tid; i < nk * SWN; i += kThreads) {
                const int64_t r = s_row[i / SWN];
                if (r >= 0) signs[r * SWN + i % SWN] = s.sw[i];
            }
        }
    }
    if (tid < nk && s_row[tid] >= 0) {
        const int64_t r = s_row[tid];
        const double n2 = s.nrm2[tid] + s.nrm2[kKeys + tid] + s.nrm2[2 * kKeys + tid] + s.nrm2[3 * kKeys + tid];
        a.out.knorm[r] = static_cast<float>(sqrt(n2));
        if (qjl) {
            const double r2 = s.rho2[tid] + s.rho2[kKeys + tid] + s.rho2[2 * kKeys + tid] + s.rho2[3 * kKeys + tid];
            a.out.rnorm[r] = static_cast<float>(sqrt(r2));
        }
    }
}

template <int D, typename TIn, int BITS>
hipError_t launch_keys_t(const KeyLaunch &a, hipStream_t stream)
{
    const int64_t n = static_cast<int64_t>(a.B) * a.H * a.T;
    constexpr size_t smem = key_smem_bytes<D, BITS>();
    auto kern = k_compress_keys<D, TIn, BITS>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    const int64_t blocks = (n + kKeys - 1) / kKeys;
    void *tok;
    prof_begin("tq_compress_keys", stream, &tok);
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), smem, stream, a, n);
    prof_end(tok, stream);
    return hipGetLastError();
}

template <int D, typename TIn>
hipError_t launch_keys_b(const KeyLaunch &a, hipStream_t stream)
{
    switch (a.bits) {
    case 1: return launch_keys_t<D, TIn, 1>(a, stream);
    case 2: return launch_keys_t<D, TIn, 2>(a, stream);
    case 3: return launch_keys_t<D, TIn, 3>(a, stream);
    case 4: return launch_keys_t<D, TIn, 4>(a, stream);
    case 5: return launch_keys_t<D, TIn, 5>(a, stream);
    case 6: return launch_keys_t<D, TIn, 6>(a, stream);
    case 7: return launch_keys_t<D, TIn, 7>(a, stream);
    }
    return hipErrorInvalidValue;
}

template <typename TIn>
hipError_t launch_keys_d(const KeyLaunch &a, hipStream_t stream)
{
    switch (a.d) {
    case 64: return launch_keys_b<64, TIn>(a, stream);
    case 128: return launch_keys_b<128, TIn>(a, stream);
    case 256: return launch_keys_b<256, TIn>(a, stream);
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

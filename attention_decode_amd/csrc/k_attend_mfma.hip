// Matrix-core decode attention for gfx950 (keys with 1 or 2 Lloyd-Max bits,
// d in {128, 256}, up to 8 query heads per KV head).
//
// Scores ("turboquant-pytorch", section "What it does": asymmetric scores on
// the compressed keys).  With an exactly symmetric codebook, the centroid of
// a 2-bit index is affine in its two bits:
//   c[b0 + 2 b1] = c[0] + (c[1] - c[0]) b0 + (c[2] - c[0]) b1,
// so sum_j q_rot[j] c[idx_j] is a weighted sum of the raw bits of the code
// row, and sum_i Sq_i s_i a weighted sum of the raw sign bits.  Each bit is an
// exact int8 operand ((dword >> k) & 0x01010101 yields four of them), and the
// weights are fixed point with four balanced 7-bit digits, so a
// v_mfma_i32_16x16x64_i8 accumulates every limb exactly in int32.  Matrix rows
// are (query, digit), columns are keys.
//
// Values (discosf.com TurboQuant article, step 4).  out[g][c] =
//   sum_t p[g][t] scale[t][grp(c)] code[t][c] + sum_t p[g][t] zero[t][grp(c)].
// The first sum is an fp16 matrix product (v_mfma_f32_16x16x32_f16): rows
// are (query, hi/lo) with p * scale split into two fp16 parts (22 bits),
// columns are channels.  The code operand is the code itself as the bits of an
// fp16 subnormal (value code * 2^-24, exact; the product is scaled back by
// 2^24), taken straight from the packed bytes: the LDS transpose read
// (ds_read_b64_tr_b8) gives each lane one byte column over eight tokens and a
// shift and mask leave one field per half.  The zero-point sum is a per-lane
// running sum reduced once per split.
//
// One 256-thread workgroup owns one (sequence, KV head, query chunk) and one
// token range; tiles of 64 keys.  The last workgroup of a unit to finish
// merges the splits (log-sum-exp), so one launch does the whole decode step.
#include "tq_internal.h"
#include "tq_device.h"

#include <cmath>

namespace tq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v2i lds_v2i;

constexpr int kThreads = 256;
constexpr int kKeys = 64;          // keys per tile
constexpr int kMaxG = 8;           // query heads per unit
constexpr int kMaxNG = 8;          // value groups per vector (d / group)

// dwords of one key row that one lane of a 4-lane k-block group handles
__host__ __device__ constexpr int code_dwords(int d, int bits) { return d * bits / 128; }
__host__ __device__ constexpr int sign_dwords(int d) { return d / 128; }

// balanced base-128 digit k of x (|x| < 2^27): x = sum_k digit_k 128^k, digits in [-64, 64]
__device__ __forceinline__ int digit7(int x, int k)
{
    int d = 0;
#pragma unroll
    for (int i = 0; i <= 3; ++i) {
        d = ((x + 64) & 127) - 64;
        if (i == k) break;
        x = (x - d) >> 7;
    }
    return (k == 3) ? x : d;
}

// value of a limb-row quadruple: c0 + 128 c1 + 128^2 c2 + 128^3 c3 (each |c| < 2^24)
__device__ __forceinline__ float limbs_to_float(v4i c)
{
    return static_cast<float>(c[0]) +
           128.0f * (static_cast<float>(c[1]) +
                     128.0f * (static_cast<float>(c[2]) + 128.0f * static_cast<float>(c[3])));
}

__device__ __forceinline__ float wave_max(float x)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

__device__ __forceinline__ float load1(const float *p) { return *p; }
__device__ __forceinline__ float load1(const bf16_t *p) { return bf16_to_f32(p->bits); }
__device__ __forceinline__ float load1(const f16_t *p) { return f16_bits_to_f32(p->bits); }

// ---------------------------------------------------------------- q-prep
// One workgroup per query row (b, hq): q_rot = Pi q and Sq = (S Pi) q as two
// coalesced float4 matrix-vector products with every load of a pass in
// flight, then this query's fixed-point digit operands (its four rows of the
// score products), its scalars, and (first query of a unit) the zeroed split
// counter and the zero rows of absent queries.
template <typename TIn>
__global__ __launch_bounds__(kThreads) void k_qprep_mfma(DecodeLaunch a)
{
    __shared__ float qs[256];
    __shared__ float part[2][8][256];
    __shared__ float qr[256], sq[256];
    __shared__ float red[4];
    __shared__ float s_acoef[2];
    const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
    const int D = a.d, M = a.m;
    const int64_t row = blockIdx.x;                 // b * Hq + hq
    const int b = static_cast<int>(row / a.Hq), hq = static_cast<int>(row % a.Hq);
    const int G = a.Hq / a.Hkv, hkv = hq / G, gi = hq % G;
    const int GC = a.mf.gc, qc = gi / GC, g = gi % GC;
    const int MT = a.mf.mt;
    const int unit = (b * a.Hkv + hkv) * a.mf.nqc + qc;

    for (int i = tid; i < D; i += kThreads) qs[i] = load1(static_cast<const TIn *>(a.q) + row * D + i);
    if (tid == 0) {
        // bit-affine form of the codebook (exact for symmetric codebooks)
        s_acoef[0] = a.centroids[1] - a.centroids[0];
        s_acoef[1] = (a.bits == 2) ? a.centroids[2] - a.centroids[0] : 0.0f;
    }
    __syncthreads();
    {
        const int NQ = D / 4, RG = kThreads / NQ;
        const int c4 = tid % NQ, rg = tid / NQ;
        const float4 *p1 = reinterpret_cast<const float4 *>(a.piT);
        const float4 *p2 = reinterpret_cast<const float4 *>(a.spiT);
        float4 y1 = make_float4(0.f, 0.f, 0.f, 0.f), y2 = y1;
#pragma unroll 16
        for (int jj = rg; jj < D; jj += RG) {
            const float4 u = p1[jj * NQ + c4], v = p2[jj * NQ + c4];
            const float qj = qs[jj];
            y1.x = fmaf(u.x, qj, y1.x); y1.y = fmaf(u.y, qj, y1.y);
            y1.z = fmaf(u.z, qj, y1.z); y1.w = fmaf(u.w, qj, y1.w);
            y2.x = fmaf(v.x, qj, y2.x); y2.y = fmaf(v.y, qj, y2.y);
            y2.z = fmaf(v.z, qj, y2.z); y2.w = fmaf(v.w, qj, y2.w);
        }
        *reinterpret_cast<float4 *>(&part[0][rg][4 * c4]) = y1;
        *reinterpret_cast<float4 *>(&part[1][rg][4 * c4]) = y2;
        __syncthreads();
        if (tid < D) {
            float s1 = 0.0f, s2 = 0.0f;
            for (int r = 0; r < RG; ++r) {
                s1 += part[0][r][tid];
                s2 += part[1][r][tid];
            }
            qr[tid] = s1;
            sq[tid] = s2;
        }
    }
    __syncthreads();
    if (wave < 2) {
        const float *v = wave == 0 ? qr : sq;
        const int n = wave == 0 ? D : M;
        float mx = 0.0f, sum = 0.0f;
        for (int j = lane; j < n; j += 64) {
            mx = fmaxf(mx, fabsf(v[j]));
            sum += v[j];
        }
        mx = wave_max(mx);
        sum = wave_sum(sum);
        if (lane == 0) {
            red[2 * wave] = mx;
            red[2 * wave + 1] = sum;
        }
    }
    __syncthreads();
    const float mw = red[0] * fmaxf(fabsf(s_acoef[0]), fabsf(s_acoef[1]));
    int ec = 0, es = 0;
    frexpf(mw, &ec);          // mw < 2^ec
    frexpf(red[2], &es);
    const int fc = (mw > 0.0f) ? 26 - ec : 0;
    const int fs = (red[2] > 0.0f) ? 26 - es : 0;
    if (tid == 0) {
        float *sc = a.mf.qscal + row * 4;
        sc[0] = ldexpf(1.0f, -fc);
        sc[1] = a.centroids[0] * red[1];
        sc[2] = ldexpf(1.0f, -fs);
        sc[3] = red[3];
    }
    // this query's digit rows: lanes 16 kb + 4 (g % 4) + digit of row tile g / 4;
    // dword r of a lane holds elements 4r..4r+3 of its 16-element k-block
    const int nc = code_dwords(D, a.bits), ns = sign_dwords(D);
    const int S = 2 * nc + 2 * ns;
    uint32_t *out = a.mf.aops + static_cast<int64_t>(unit) * MT * S * 256;
    for (int w = tid; w < S * 64; w += kThreads) {
        const int r = w % 4, limb = (w / 4) % 4, kb = (w / 16) % 4, s = w / 64;
        const int l = 16 * kb + 4 * (g % 4) + limb;
        uint32_t dw = 0;
#pragma unroll
        for (int K = 0; K < 4; ++K) {
            float wv;
            int f;
            if (s < 2 * nc) {
                const int u = s / 2, h = s % 2;
                const int bit = 32 * (kb * nc + u) + 8 * K + 4 * h + r;
                wv = qr[bit / a.bits] * s_acoef[bit % a.bits];
                f = fc;
            } else {
                const int s2 = s - 2 * nc, u = s2 / 2, h = s2 % 2;
                const int bit = 32 * (kb * ns + u) + 8 * K + 4 * h + r;
                wv = sq[bit];
                f = fs;
            }
            const int x = static_cast<int>(rintf(ldexpf(wv, f)));
            dw |= (static_cast<uint32_t>(digit7(x, limb)) & 0xffu) << (8 * K);
        }
        out[((g / 4) * S + s) * 256 + l * 4 + r] = dw;
    }
    if (g == 0) {
        // rows of absent queries (unit with fewer than four query heads) stay zero
        for (int w = tid; w < S * 64 * 4; w += kThreads) {
            const int l = (w / 4) % 64;
            if ((l % 16) / 4 >= GC) out[(w / 256) * 256 + (w % 256)] = 0u;
        }
        if (tid == 0) a.mf.counters[unit] = 0;
    }
}

// ------------------------------------------------------------ attention
template <int BITS, int D, int MT, int VBITS>
__global__ __launch_bounds__(kThreads, 2) void k_attend_mfma(DecodeLaunch a, float kappa, int64_t chunk)
{
    constexpr int NC = code_dwords(D, BITS), NS = sign_dwords(D);
    constexpr int SC = 2 * NC, SS = 2 * NS, S = SC + SS;
    constexpr int GCMAX = 4 * MT;
    constexpr int VB = D * VBITS / 8;            // value code bytes per token
    constexpr int VSTR = VB + 16;                // LDS row stride (odd multiple of 16 B)
    constexpr int NCB = VB / 16;                 // 16-column blocks of value bytes
    constexpr int NF = 8 / VBITS;                // code fields per byte
    constexpr int NTILE = NCB * NF;              // 16-channel tiles of the value product
    constexpr int NTW = (NTILE + 3) / 4;         // tiles per wave
    constexpr uint32_t VMASK = VBITS == 4 ? 0x0F0F0F0Fu : 0x03030303u;

    __shared__ float lam[GCMAX][kKeys];
    __shared__ float s_alpha[GCMAX], s_m[GCMAX], s_l[GCMAX];
    __shared__ float pmax[4][GCMAX], psum[4][GCMAX];
    __shared__ float zsum[GCMAX][kMaxNG];
    __shared__ __align__(16) unsigned char vtile[kKeys * VSTR];
    __shared__ float2 vsz[kKeys * kMaxNG];       // (scale, zero) per (key, group)
    // value-product A fragments: [group][k-step][lane][4 dwords of fp16 pairs]
    __shared__ __align__(16) uint32_t afr[kMaxNG][2][64][4];
    __shared__ int s_last;

    const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
    const int GC = a.mf.gc, nqc = a.mf.nqc, G = a.Hq / a.Hkv;
    const int NG = D / a.group;
    const int unit = blockIdx.y, split = blockIdx.x;
    const int qc = unit % nqc;
    const int64_t bh = unit / nqc;
    const int b = static_cast<int>(bh / a.Hkv), hkv = static_cast<int>(bh % a.Hkv);
    const int hq0 = hkv * G + qc * GC;
    const int64_t row0 = static_cast<int64_t>(b) * a.Hq + hq0;
    const int64_t t_begin = static_cast<int64_t>(split) * chunk;
    const int64_t t_end = t_begin + chunk < a.T ? t_begin + chunk : a.T;

    // score operands of this unit (loop invariant)
    v4i aop[MT][S];
    {
        const v4i *src = reinterpret_cast<const v4i *>(a.mf.aops) + static_cast<int64_t>(unit) * MT * S * 64;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int s = 0; s < S; ++s) aop[mt][s] = src[(mt * S + s) * 64 + lane];
    }
    const int j = lane % 16, kb = lane / 16, rb = lane / 16;
    float fc[MT], cc[MT], fs[MT], ssq[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int g = 4 * mt + rb;
        if (g < GC) {
            const float *sc = a.mf.qscal + (row0 + g) * 4;
            fc[mt] = sc[0];
            cc[mt] = sc[1];
            fs[mt] = sc[2];
            ssq[mt] = sc[3];
        } else {
            fc[mt] = cc[mt] = fs[mt] = ssq[mt] = 0.0f;
        }
    }
    // rows of absent queries stay zero in the value operands
    for (int i = tid; i < kMaxNG * 2 * 64 * 4; i += kThreads) (&afr[0][0][0][0])[i] = 0u;
    if (tid < GCMAX) {
        s_m[tid] = -INFINITY;
        s_l[tid] = 0.0f;
    }
    // softmax state of this lane's (query 4 mt + rb, key column j): running max
    // (identical in all lanes of a query), this lane's share of the running sum
    // and of the zero-point sums
    float m_run[MT], l_run[MT];
    float zacc[MT][kMaxNG];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        m_run[mt] = -INFINITY;
        l_run[mt] = 0.0f;
#pragma unroll
        for (int gg = 0; gg < kMaxNG; ++gg) zacc[mt][gg] = 0.0f;
    }
    // lane (channel column, rb) accumulates queries 2 rb and 2 rb + 1
    float oacc[NTW][2];
#pragma unroll
    for (int x = 0; x < NTW; ++x) oacc[x][0] = oacc[x][1] = 0.0f;
    __syncthreads();

    // Register prefetch of one tile: value code chunk, value params, the key
    // row slices of this lane's key.  The next tile's loads are issued before
    // the current tile is computed, so their latency hides behind the work.
    constexpr int VCH = kKeys * VB / 16;          // 16-byte value chunks per tile
    constexpr int VCPT = (VCH + kThreads - 1) / kThreads;   // chunks per thread
    struct Prefetch {
        uint4 vcode[VCPT];
        uint32_t vpar[2];
        uint32_t cw[NC], sw[NS];
        float nrm, rho;
    };
    auto fetch = [&](int64_t tile0, Prefetch &pf) {
        const int ntile = static_cast<int>(t_end - tile0 < kKeys ? t_end - tile0 : kKeys);
        const int64_t n0 = bh * a.T + tile0;
#pragma unroll
        for (int k = 0; k < VCPT; ++k) {
            const int i = tid + k * kThreads;
            pf.vcode[k] = make_uint4(0u, 0u, 0u, 0u);
            if (i < VCH && i / (VB / 16) < ntile) pf.vcode[k] = reinterpret_cast<const uint4 *>(a.vc.codes + n0 * VB)[i];
        }
        const uint32_t *par = reinterpret_cast<const uint32_t *>(a.vc.params) + n0 * NG;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int i = tid + k * kThreads;
            pf.vpar[k] = (i < ntile * NG) ? par[i] : 0u;
        }
        const int t = 16 * wave + j;
        const bool valid = t < ntile;
        const int64_t n = n0 + (valid ? t : 0);
        const uint32_t *crow = reinterpret_cast<const uint32_t *>(a.kc.codes) + n * (D * BITS / 32) + kb * NC;
        const uint32_t *srow = reinterpret_cast<const uint32_t *>(a.kc.signs) + n * (D / 32) + kb * NS;
#pragma unroll
        for (int u = 0; u < NC; ++u) pf.cw[u] = valid ? crow[u] : 0u;
#pragma unroll
        for (int u = 0; u < NS; ++u) pf.sw[u] = valid ? srow[u] : 0u;
        pf.nrm = valid ? a.kc.knorm[n] : 0.0f;
        pf.rho = valid ? a.kc.rnorm[n] : 0.0f;
    };
    Prefetch pre;
    if (t_begin < t_end) fetch(t_begin, pre);

    for (int64_t tile0 = t_begin; tile0 < t_end; tile0 += kKeys) {
        const int ntile = static_cast<int>(t_end - tile0 < kKeys ? t_end - tile0 : kKeys);
        const Prefetch cur = pre;
        if (tile0 + kKeys < t_end) fetch(tile0 + kKeys, pre);
        // ---- stage the value tile (code rows, fp32 scale / zero)
#pragma unroll
        for (int k = 0; k < VCPT; ++k) {
            const int i = tid + k * kThreads;
            if (i < VCH) *reinterpret_cast<uint4 *>(vtile + (i / (VB / 16)) * VSTR + (i % (VB / 16)) * 16) = cur.vcode[k];
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int i = tid + k * kThreads;
            if (i < kKeys * NG)
                vsz[i] = make_float2(f16_bits_to_f32(cur.vpar[k] & 0xffffu), f16_bits_to_f32(cur.vpar[k] >> 16));
        }
        // ---- scores of keys 16 wave + j: 4 lanes (kb) split each key row
        float lamr[MT];
        {
            const int t = 16 * wave + j;
            const bool valid = t < ntile;
            v4i accc[MT], accs[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) accc[mt] = accs[mt] = v4i{0, 0, 0, 0};
#pragma unroll
            for (int s = 0; s < SC; ++s) {
                const uint32_t dw = cur.cw[s / 2];
                const int h = 4 * (s % 2);
                const v4i bop = {static_cast<int>((dw >> h) & 0x01010101u), static_cast<int>((dw >> (h + 1)) & 0x01010101u),
                                 static_cast<int>((dw >> (h + 2)) & 0x01010101u), static_cast<int>((dw >> (h + 3)) & 0x01010101u)};
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    accc[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop[mt][s], bop, accc[mt], 0, 0, 0);
            }
#pragma unroll
            for (int s = 0; s < SS; ++s) {
                const uint32_t dw = cur.sw[s / 2];
                const int h = 4 * (s % 2);
                const v4i bop = {static_cast<int>((dw >> h) & 0x01010101u), static_cast<int>((dw >> (h + 1)) & 0x01010101u),
                                 static_cast<int>((dw >> (h + 2)) & 0x01010101u), static_cast<int>((dw >> (h + 3)) & 0x01010101u)};
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    accs[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop[mt][SC + s], bop, accs[mt], 0, 0, 0);
            }
            // lane (key j, row block rb) holds the four digits of query 4 mt + rb;
            // per-wave partial maxima over the 16 key columns
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const float dcode = fmaf(limbs_to_float(accc[mt]), fc[mt], cc[mt]);
                const float dsign = fmaf(2.0f * limbs_to_float(accs[mt]), fs[mt], -ssq[mt]);
                const float score = cur.nrm * fmaf(kappa * cur.rho, dsign, dcode);
                lamr[mt] = (valid && 4 * mt + rb < GC) ? a.scale * score : -INFINITY;
                float pm = lamr[mt];
#pragma unroll
                for (int off = 1; off < 16; off <<= 1) pm = fmaxf(pm, __shfl_xor(pm, off));
                if (j == 0) pmax[wave][4 * mt + rb] = pm;
            }
        }
        __syncthreads();
        // ---- online softmax and value-product operands, per (query, key) lane:
        // p = e^(lambda - m), w = p * scale as fp16 hi + lo into row 2 g + part of
        // the A fragment at the token's k position (tr-read order {0,2|1,3|4,6|5,7})
        {
            const int t = 16 * wave + j;
            const int ks = t / 32, kbq = (t % 32) / 8, tau = t % 8;
            const int u = 2 * (tau / 4) + (tau % 2), half = (tau % 4) / 2;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int g = 4 * mt + rb;
                if (g < GC) {
                    const float tmax = fmaxf(fmaxf(pmax[0][g], pmax[1][g]), fmaxf(pmax[2][g], pmax[3][g]));
                    const float m_new = fmaxf(m_run[mt], tmax);
                    float alpha = 1.0f, p = 0.0f;
                    if (m_new != -INFINITY) {
                        alpha = __expf(m_run[mt] - m_new);
                        p = __expf(lamr[mt] - m_new);
                    }
                    m_run[mt] = m_new;
                    l_run[mt] = fmaf(l_run[mt], alpha, p);
                    if (wave == 0 && j == 0) s_alpha[g] = alpha;
                    uint16_t *arow = reinterpret_cast<uint16_t *>(&afr[0][ks][16 * kbq + 2 * g][u]) + half;
#pragma unroll
                    for (int gg = 0; gg < kMaxNG; ++gg) {
                        if (gg < NG) {
                            const float2 sz = vsz[t * NG + gg];
                            zacc[mt][gg] = fmaf(p, sz.y, zacc[mt][gg] * alpha);
                            const float w = p * sz.x;
                            const auto hi = __builtin_amdgcn_cvt_pkrtz(w, 0.0f);
                            const auto lo = __builtin_amdgcn_cvt_pkrtz(w - static_cast<float>(hi[0]), 0.0f);
                            // afr[gg][ks][row][u]: rows 2 g (hi) and 2 g + 1 (lo)
                            arow[gg * (2 * 64 * 4 * 2)] = __builtin_bit_cast(uint32_t, hi) & 0xffffu;
                            arow[gg * (2 * 64 * 4 * 2) + 4 * 2] = __builtin_bit_cast(uint32_t, lo) & 0xffffu;
                        }
                    }
                }
            }
        }
        __syncthreads();
        // ---- value product: wave w handles channel tiles w, w + 4, ...
#pragma unroll
        for (int x = 0; x < NTW; ++x) {
            const int nt = wave + 4 * x;
            if (nt < NTILE) {
                const int cb = nt / NF, f = nt % NF;
                const int pl = lane % 16;
                const int sh = VBITS * f;
                const uint32_t fm = (VBITS == 4 ? 0x000F000Fu : 0x00030003u);
                // column i = byte column 16 cb + i -> channel NF (16 cb + i) + f
                const int ch = NF * (16 * cb + j) + f;
                const int g_lo = (NF * 16 * cb) / a.group;
                const bool two = NF * 16 > a.group;          // the tile spans two value groups
                v4f acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const unsigned char *base = vtile + (32 * ks + 8 * kb + pl / 2) * VSTR + 16 * cb + 8 * (pl % 2);
                    const v2i raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i *)(base));
                    const uint32_t x0 = static_cast<uint32_t>(raw.x), x1 = static_cast<uint32_t>(raw.y);
                    const v4i bop = {static_cast<int>((x0 >> sh) & fm), static_cast<int>((x0 >> (8 + sh)) & fm),
                                     static_cast<int>((x1 >> sh) & fm), static_cast<int>((x1 >> (8 + sh)) & fm)};
                    const v8h bh = __builtin_bit_cast(v8h, bop);
                    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        __builtin_bit_cast(v8h, *reinterpret_cast<const v4i *>(&afr[g_lo][ks][lane][0])), bh, acc0, 0, 0, 0);
                    if (two)
                        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            __builtin_bit_cast(v8h, *reinterpret_cast<const v4i *>(&afr[g_lo + 1][ks][lane][0])), bh, acc1, 0, 0, 0);
                }
                const v4f acc = (two && ch / a.group != g_lo) ? acc1 : acc0;
                // rows 4 rb .. 4 rb + 3 = (query 2 rb, hi), (2 rb, lo), (2 rb + 1, hi), (2 rb + 1, lo)
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int g = 2 * rb + q;
                    const float alpha = (g < GC) ? s_alpha[g] : 1.0f;
                    oacc[x][q] = fmaf(oacc[x][q], alpha, 16777216.0f * (acc[2 * q] + acc[2 * q + 1]));
                }
            }
        }
        __syncthreads();
    }

    // ---- this split's partials: m, l per query; acc[c] = value sum + zero-point sum.
    // l and the zero-point sums are spread over the 16 key columns of each wave
    // and over the 4 waves: reduce across j, then across waves.
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int g = 4 * mt + rb;
        float l = l_run[mt];
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) l += __shfl_xor(l, off);
        if (j == 0 && g < GC) psum[wave][g] = l;
        if (wave == 0 && j == 0 && g < GC) s_m[g] = m_run[mt];
#pragma unroll
        for (int gg = 0; gg < kMaxNG; ++gg) {
            if (gg < NG) {
                float z = zacc[mt][gg];
#pragma unroll
                for (int off = 1; off < 16; off <<= 1) z += __shfl_xor(z, off);
                if (j == 0 && g < GC) vsz[(wave * GCMAX + g) * kMaxNG + gg].x = z;
            }
        }
    }
    __syncthreads();
    if (tid < GC) {
        s_l[tid] = psum[0][tid] + psum[1][tid] + psum[2][tid] + psum[3][tid];
        for (int gg = 0; gg < NG; ++gg) {
            float z = 0.0f;
            for (int w = 0; w < 4; ++w) z += vsz[(w * GCMAX + tid) * kMaxNG + gg].x;
            zsum[tid][gg] = z;
        }
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < NTW; ++x) {
        const int nt = wave + 4 * x;
        if (nt < NTILE) {
            const int cb = nt / NF, f = nt % NF;
            const int ch = NF * (16 * cb + j) + f;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int g = 2 * rb + q;
                if (g < GC)
                    a.part_acc[((row0 + g) * a.splits + split) * D + ch] = oacc[x][q] + zsum[g][ch / a.group];
            }
        }
    }
    if (tid < GC) {
        a.part_ml[((row0 + tid) * a.splits + split) * 2 + 0] = s_m[tid];
        a.part_ml[((row0 + tid) * a.splits + split) * 2 + 1] = s_l[tid];
    }
    // ---- the last workgroup of this unit merges the splits
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = (atomicAdd(a.mf.counters + unit, 1) == a.splits - 1) ? 1 : 0;
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    // pass 1: one wave per query turns the split maxima and sums into weights
    // w_s = e^(m_s - M) / sum_s' l_s' e^(m_s' - M)   (splits <= 64, lane = split)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int g = wave + 4 * q;
        if (g < GC) {
            const float *ml = a.part_ml + (row0 + g) * a.splits * 2;
            float m = -INFINITY, l = 0.0f;
            if (lane < a.splits) {
                m = ml[2 * lane];
                l = ml[2 * lane + 1];
            }
            const float mx = wave_max(l > 0.0f ? m : -INFINITY);
            const float w = (l > 0.0f) ? expf(m - mx) : 0.0f;
            const float den = wave_sum(l * w);
            lam[g][lane] = den > 0.0f ? w / den : 0.0f;
        }
    }
    __syncthreads();
    // pass 2: out[g][c..c+3] = sum_s w_s acc_s[c..c+3], sixteen splits' loads in flight
    for (int i = tid; i < GC * (D / 4); i += kThreads) {
        const int g = i / (D / 4), c4 = i % (D / 4);
        const float4 *pa = reinterpret_cast<const float4 *>(a.part_acc + (row0 + g) * a.splits * D) + c4;
        float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        for (int s0 = 0; s0 < a.splits; s0 += 16) {
            float4 v[16];
#pragma unroll
            for (int k = 0; k < 16; ++k)
                v[k] = (s0 + k < a.splits) ? pa[static_cast<int64_t>(s0 + k) * (D / 4)] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const float w = (s0 + k < a.splits) ? lam[g][s0 + k] : 0.0f;
                o.x = fmaf(w, v[k].x, o.x);
                o.y = fmaf(w, v[k].y, o.y);
                o.z = fmaf(w, v[k].z, o.z);
                o.w = fmaf(w, v[k].w, o.w);
            }
        }
        reinterpret_cast<float4 *>(a.out + (row0 + g) * D)[c4] = o;
    }
    if (tid == 0) a.mf.counters[unit] = 0;
}

template <int BITS, int D, int MT, int VBITS>
hipError_t launch_mfma_t(const DecodeLaunch &a, hipStream_t stream, float kappa, int64_t chunk)
{
    const dim3 grid(static_cast<unsigned>(a.splits), static_cast<unsigned>(a.mf.units));
    void *tok;
    prof_begin("tq_attend_splitk", stream, &tok);
    hipLaunchKernelGGL((k_attend_mfma<BITS, D, MT, VBITS>), grid, dim3(kThreads), 0, stream, a, kappa, chunk);
    prof_end(tok, stream);
    return hipGetLastError();
}

template <int BITS, int D, int MT>
hipError_t launch_mfma_v(const DecodeLaunch &a, hipStream_t s, float kappa, int64_t chunk)
{
    return a.vbits == 2 ? launch_mfma_t<BITS, D, MT, 2>(a, s, kappa, chunk)
                        : launch_mfma_t<BITS, D, MT, 4>(a, s, kappa, chunk);
}

template <int BITS, int D>
hipError_t launch_mfma_m(const DecodeLaunch &a, hipStream_t s, float kappa, int64_t chunk)
{
    return a.mf.mt == 1 ? launch_mfma_v<BITS, D, 1>(a, s, kappa, chunk) : launch_mfma_v<BITS, D, 2>(a, s, kappa, chunk);
}

template <int BITS>
hipError_t launch_mfma_d(const DecodeLaunch &a, hipStream_t s, float kappa, int64_t chunk)
{
    return a.d == 128 ? launch_mfma_m<BITS, 128>(a, s, kappa, chunk) : launch_mfma_m<BITS, 256>(a, s, kappa, chunk);
}

}  // namespace

bool mfma_decode_supported(int d, int bits, int G, int vbits, int group)
{
    (void)group;
    const int gc = mfma_query_chunk(G);
    return (d == 128 || d == 256) && (bits == 1 || bits == 2) && gc >= 1 && (vbits == 2 || vbits == 4);
}

int mfma_query_chunk(int G)
{
    int gc = kMaxG;
    while (gc > 1 && (G % gc) != 0) gc >>= 1;
    return gc;
}

int mfma_score_steps(int d, int bits) { return 2 * code_dwords(d, bits) + 2 * sign_dwords(d); }

hipError_t launch_decode_mfma(const DecodeLaunch &a, hipStream_t stream)
{
    const dim3 qgrid(static_cast<unsigned>(static_cast<int64_t>(a.B) * a.Hq));
    void *tok;
    prof_begin("tq_qprep", stream, &tok);
    switch (a.dtype) {
    case TQ_F32: hipLaunchKernelGGL(k_qprep_mfma<float>, qgrid, dim3(kThreads), 0, stream, a); break;
    case TQ_BF16: hipLaunchKernelGGL(k_qprep_mfma<bf16_t>, qgrid, dim3(kThreads), 0, stream, a); break;
    case TQ_F16: hipLaunchKernelGGL(k_qprep_mfma<f16_t>, qgrid, dim3(kThreads), 0, stream, a); break;
    }
    prof_end(tok, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const float kappa = static_cast<float>(std::sqrt(M_PI / 2.0) / a.m);
    const int64_t tiles = (a.T + kKeys - 1) / kKeys;
    const int64_t chunk = ((tiles + a.splits - 1) / a.splits) * kKeys;
    return a.bits == 1 ? launch_mfma_d<1>(a, stream, kappa, chunk) : launch_mfma_d<2>(a, stream, kappa, chunk);
}

}  // namespace tq

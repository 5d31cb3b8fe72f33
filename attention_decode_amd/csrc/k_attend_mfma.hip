// Matrix-core decode attention for gfx950 (keys with 1 or 2 Lloyd-Max bits,
// d in {128, 256}, up to 8 query heads per KV head).
//
// Scores ("turboquant-pytorch", section "What it does": asymmetric scores on
// the compressed keys).  With an exactly symmetric codebook, the centroid of
// a 2-bit index is affine in its two bits:
//   c[b0 + 2 b1] = c[0] + (c[1] - c[0]) b0 + (c[2] - c[0]) b1,
// so sum_j q_rot[j] c[idx_j] is a weighted sum of the raw bits of the code
// row, and sum_i Sq_i s_i a weighted sum of the raw sign bits.  Each bit is an
// exact int8 operand: dword & (0x01010101 << k) yields four of them as bytes
// of value 2^k (-128 for k = 7), and the weight of that position carries
// 2^-k (negated for k = 7).  The weights are fixed point with four balanced
// 7-bit digits, so a v_mfma_i32_16x16x64_i8 accumulates every limb exactly in
// int32.  Matrix rows are (query, digit), columns are keys.
//
// Values (discosf.com TurboQuant article, step 4).  out[g][c] =
//   sum_t p[g][t] scale[t][grp(c)] code[t][c] + sum_t p[g][t] zero[t][grp(c)].
// The first sum is an fp16 matrix product (v_mfma_f32_16x16x32_f16): rows
// are (query, hi/lo) with p * scale split into two fp16 parts (22 bits),
// columns are channels.  The code operand is the code itself as the bits of an
// fp16 subnormal (value code * 2^-24, exact; the product is scaled back by
// 2^24), taken straight from the packed bytes: the LDS transpose read
// (ds_read_b64_tr_b8) gives each lane one byte column over eight tokens, and a
// mask leaves one field per half in place (field f of a byte reads as
// code * 2^(bits f), undone when the accumulator is read out).  The
// zero-point sum is a per-lane running sum reduced once per split.
//
// One 256-thread workgroup owns one (sequence, KV head, query chunk) and one
// token range; every wave runs its own 32-key tiles without workgroup
// barriers.  Split partials (max, sum, weighted values) are merged by
// log-sum-exp in a second, small kernel (none with a single split).
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

// value of a limb-row quadruple: c0 + 128 c1 + 128^2 c2 + 128^3 c3 (each |c| < 2^23,
// so the two pair sums are exact in int32)
__device__ __forceinline__ float limbs_to_float(v4i c)
{
    const int lo = c[0] + (c[1] << 7), hi = c[2] + (c[3] << 7);
    return fmaf(static_cast<float>(hi), 16384.0f, static_cast<float>(lo));
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
            // the key bit arrives as byte 2^sh (masked in place, not shifted):
            // weight w 2^-sh, negated for sh = 7 where the byte reads as -128
            const int sh = 4 * (s % 2) + r;
            int x = static_cast<int>(rintf(ldexpf(wv, f - sh)));
            if (sh == 7) x = -x;
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
    }
}

// ------------------------------------------------------------ attention
// 16-lane (one DPP row) reductions: xor 1, xor 2, half-row mirror, row mirror

template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float row16_max(float x)
{
    x = fmaxf(x, dpp<0xB1>(x));
    x = fmaxf(x, dpp<0x4E>(x));
    x = fmaxf(x, dpp<0x141>(x));
    return fmaxf(x, dpp<0x140>(x));
}

__device__ __forceinline__ float row16_sum(float x)
{
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x141>(x);
    return x + dpp<0x140>(x);
}

// k-slot order of a 32-token wave tile in the value product: slot 2j holds
// token j, slot 2j + 1 token 16 + j, so that the lane owning key column j of
// both score tiles writes its two tokens as one packed fp16 pair.
__device__ __forceinline__ int slot_token(int slot) { return (slot & 1) ? 16 + (slot >> 1) : (slot >> 1); }

// One 256-thread workgroup owns one (sequence, KV head, query chunk) and one
// token range; each wave walks its own 32-key tiles (wave w takes tiles w,
// w + 4, ...) with its own online-softmax state and value accumulators, so
// the tile loop has no workgroup barrier.  Loads of the next tile are issued
// before the current one is computed (two register buffers in turn).  The
// four waves are merged in LDS at the end; with one split the workgroup
// writes the normalised output, else its partial (max, sum, weighted values).
template <int BITS, int D, int MT, int VBITS>
__global__ __launch_bounds__(kThreads, D == 256 ? 1 : 2) void k_attend_mfma(DecodeLaunch a, float kappa, int64_t chunk)
{
    constexpr int NC = code_dwords(D, BITS), NS = sign_dwords(D);
    constexpr int SC = 2 * NC, SS = 2 * NS, S = SC + SS;
    constexpr int TK = 32;                       // keys per wave tile
    constexpr int VB = D * VBITS / 8;            // value code bytes per token
    constexpr int VSTR = VB + 16;                // LDS row stride (odd multiple of 16 B)
    constexpr int NCB = VB / 16;                 // 16-byte column blocks of a value row
    constexpr int NF = 8 / VBITS;                // code fields per byte
    constexpr int NTILE = NCB * NF;              // 16-channel tiles of the value product
    constexpr bool kTwoGroups = NF * 16 > 32;    // a tile can span two value groups (group >= 32)
    constexpr int VCL = TK * VB / 16 / 64;       // 16-byte value chunks per lane per tile
    constexpr int NGM = D / 32;                  // most value groups per row (group >= 32)
    constexpr int PD = TK * NGM / 64;            // (scale, zero) dwords per lane per tile
    constexpr int VT_BYTES = TK * VSTR;
    constexpr int AF_BYTES = NGM * 64 * 16;
    constexpr int PS_BYTES = TK * NGM * 4;
    constexpr int WAVE_BYTES = VT_BYTES + AF_BYTES + PS_BYTES;
    constexpr int MERGE_BYTES = 4 * kMaxG * D * 4;
    constexpr int SMEM = (4 * WAVE_BYTES > MERGE_BYTES) ? 4 * WAVE_BYTES : MERGE_BYTES;

    __shared__ __align__(16) unsigned char smem[SMEM];
    __shared__ float s_alpha[4][kMaxG];
    __shared__ float s_wm[4][kMaxG], s_wl[4][kMaxG];
    __shared__ float s_wz[4][kMaxG][kMaxNG];

    const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
    const int GC = a.mf.gc, nqc = a.mf.nqc;
    const int NG = D / a.group;                  // 1, 2, 4 or 8
    const int lg_ng = __builtin_ctz(NG);
    const int unit = blockIdx.y, split = blockIdx.x;
    const int qc = unit % nqc;
    const int64_t bh = unit / nqc;
    const int b = static_cast<int>(bh / a.Hkv), hkv = static_cast<int>(bh % a.Hkv);
    const int G = a.Hq / a.Hkv;
    const int hq0 = hkv * G + qc * GC;
    const int64_t row0 = static_cast<int64_t>(b) * a.Hq + hq0;
    const int64_t t_begin = static_cast<int64_t>(split) * chunk;
    const int64_t t_end = t_begin + chunk < a.T ? t_begin + chunk : a.T;
    const int j = lane % 16, kb = lane / 16;

    unsigned char *vt = smem + wave * WAVE_BYTES;
    uint32_t *afr = reinterpret_cast<uint32_t *>(vt + VT_BYTES);              // [NGM][64 lanes][4]
    uint32_t *pst = reinterpret_cast<uint32_t *>(vt + VT_BYTES + AF_BYTES);   // [TK][NGM]

    // score operands of this unit (loop invariant)
    v4i aop[MT][S];
    {
        const v4i *src = reinterpret_cast<const v4i *>(a.mf.aops) + static_cast<int64_t>(unit) * MT * S * 64;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int s = 0; s < S; ++s) aop[mt][s] = src[(mt * S + s) * 64 + lane];
    }
    float fc[MT], cc[MT], fs[MT], ssq[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int g = 4 * mt + kb;
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
    // value-product A rows of absent queries stay zero; alphas of absent queries are 1
    for (int i = lane; i < NGM * 64 * 4; i += 64) afr[i] = 0u;
    if (lane < kMaxG) s_alpha[wave][lane] = 1.0f;

    float m_run[MT], l_run[MT];
    float zacc[MT][NGM];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        m_run[mt] = -INFINITY;
        l_run[mt] = 0.0f;
#pragma unroll
        for (int gg = 0; gg < NGM; ++gg) zacc[mt][gg] = 0.0f;
    }
    // value-product accumulators, rows (query 2 kb + r / 2, fp16 part r % 2),
    // column j = byte column 16 cb + j, field f; acc1 for tiles whose second
    // half of columns lies in the next value group
    v4f acc0[NTILE], acc1[kTwoGroups ? NTILE : 1];
#pragma unroll
    for (int nt = 0; nt < NTILE; ++nt) acc0[nt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int nt = 0; nt < (kTwoGroups ? NTILE : 1); ++nt) acc1[nt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // tr-read row of this lane in every value block: k-slot 8 kb + e holds the
    // token of slot order; lanes 2r, 2r + 1 address read row r, and row r lands
    // in half e(r) of the operand with e = {0, 2, 1, 3, 4, 6, 5, 7}
    const int rr = j / 2;
    const int e_of_r = (rr & 4) | ((rr & 1) << 1) | ((rr >> 1) & 1);
    const unsigned char *tr_base = vt + slot_token(8 * kb + e_of_r) * VSTR + 8 * (j % 2);

    struct Prefetch {
        uint32_t cw[2][NC], sw[2][NS];
        float nrm[2], rho[2];
        v4i vcode[VCL];
        uint32_t par[PD];
    };
    const int64_t first = t_begin + TK * wave;
    // Loads of one tile, all unconditional: rows past the valid range are
    // clamped to the last valid row and masked where they are used; a tile
    // past the end reloads the wave's first tile.
    auto fetch = [&](int64_t tile0, Prefetch &pf) {
        const int64_t tc = tile0 < t_end ? tile0 : first;
        const int nv = static_cast<int>(t_end - tc < TK ? t_end - tc : TK);
        const int64_t n0 = bh * a.T + tc;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int t = 16 * c + j;
            const int64_t n = n0 + (t < nv ? t : nv - 1);
            const uint32_t *crow = reinterpret_cast<const uint32_t *>(a.kc.codes) + n * (D * BITS / 32) + kb * NC;
            const uint32_t *srow = reinterpret_cast<const uint32_t *>(a.kc.signs) + n * (D / 32) + kb * NS;
#pragma unroll
            for (int u = 0; u < NC; ++u) pf.cw[c][u] = crow[u];
#pragma unroll
            for (int u = 0; u < NS; ++u) pf.sw[c][u] = srow[u];
            pf.nrm[c] = a.kc.knorm[n];
            pf.rho[c] = a.kc.rnorm[n];
        }
        const v4i *vsrc = reinterpret_cast<const v4i *>(a.vc.codes + n0 * VB);
#pragma unroll
        for (int v = 0; v < VCL; ++v) {
            const int i = lane + 64 * v;
            const int tok = i / (VB / 16);
            pf.vcode[v] = vsrc[(tok < nv ? tok : nv - 1) * (VB / 16) + i % (VB / 16)];
        }
        const uint32_t *psrc = reinterpret_cast<const uint32_t *>(a.vc.params) + n0 * NG;
        const int plim = nv * NG - 1;
#pragma unroll
        for (int k = 0; k < PD; ++k) {
            const int idx = lane + 64 * k;
            pf.par[k] = psrc[idx < plim ? idx : plim];
        }
    };

    auto compute = [&](int64_t tile0, const Prefetch &cur) {
        const int nv = static_cast<int>(t_end - tile0 < TK ? t_end - tile0 : TK);
        // ---- value codes and (scale, zero) words of the tile into this wave's LDS
#pragma unroll
        for (int v = 0; v < VCL; ++v) {
            const int i = lane + 64 * v;
            *reinterpret_cast<v4i *>(vt + (i / (VB / 16)) * VSTR + (i % (VB / 16)) * 16) = cur.vcode[v];
        }
#pragma unroll
        for (int k = 0; k < PD; ++k) {
            const int idx = lane + 64 * k;
            if (idx < TK * NG) pst[(idx >> lg_ng) * NGM + (idx & (NG - 1))] = idx < nv * NG ? cur.par[k] : 0u;
        }

        // ---- scores of keys j and 16 + j: B bytes are raw key bits at weight
        // 2^k (mask without shift; the digit rows carry the 2^-k)
        float lamv[MT][2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            v4i accc[MT], accs[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) accc[mt] = accs[mt] = v4i{0, 0, 0, 0};
#pragma unroll
            for (int s = 0; s < SC; ++s) {
                const uint32_t dw = cur.cw[c][s / 2];
                const int h = 4 * (s % 2);
                const v4i bop = {static_cast<int>(dw & (0x01010101u << h)), static_cast<int>(dw & (0x01010101u << (h + 1))),
                                 static_cast<int>(dw & (0x01010101u << (h + 2))), static_cast<int>(dw & (0x01010101u << (h + 3)))};
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    accc[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop[mt][s], bop, accc[mt], 0, 0, 0);
            }
#pragma unroll
            for (int s = 0; s < SS; ++s) {
                const uint32_t dw = cur.sw[c][s / 2];
                const int h = 4 * (s % 2);
                const v4i bop = {static_cast<int>(dw & (0x01010101u << h)), static_cast<int>(dw & (0x01010101u << (h + 1))),
                                 static_cast<int>(dw & (0x01010101u << (h + 2))), static_cast<int>(dw & (0x01010101u << (h + 3)))};
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    accs[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop[mt][SC + s], bop, accs[mt], 0, 0, 0);
            }
            // lane (key column j, row block kb) holds the four digits of query 4 mt + kb
            const bool valid = 16 * c + j < nv;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const float dcode = fmaf(limbs_to_float(accc[mt]), fc[mt], cc[mt]);
                const float dsign = fmaf(2.0f * limbs_to_float(accs[mt]), fs[mt], -ssq[mt]);
                const float score = cur.nrm[c] * fmaf(kappa * cur.rho[c], dsign, dcode);
                lamv[mt][c] = (valid && 4 * mt + kb < GC) ? a.scale * score : -INFINITY;
            }
        }

        // ---- online softmax (per query, over the 16 lanes of its row block)
        bool grow = false;
        float m_new[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            m_new[mt] = fmaxf(m_run[mt], row16_max(fmaxf(lamv[mt][0], lamv[mt][1])));
            grow |= m_new[mt] > m_run[mt];
        }
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
            // the running maximum moved: rescale this wave's sums and accumulators
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const float alpha = (m_new[mt] > m_run[mt]) ? __expf(m_run[mt] - m_new[mt]) : 1.0f;
                l_run[mt] *= alpha;
#pragma unroll
                for (int gg = 0; gg < NGM; ++gg) zacc[mt][gg] *= alpha;
                if (j == 0) s_alpha[wave][4 * mt + kb] = alpha;
                m_run[mt] = m_new[mt];
            }
            const float a0 = s_alpha[wave][2 * kb], a1 = s_alpha[wave][2 * kb + 1];
#pragma unroll
            for (int nt = 0; nt < NTILE; ++nt) {
                acc0[nt][0] *= a0; acc0[nt][1] *= a0; acc0[nt][2] *= a1; acc0[nt][3] *= a1;
            }
#pragma unroll
            for (int nt = 0; nt < (kTwoGroups ? NTILE : 1); ++nt) {
                acc1[nt][0] *= a0; acc1[nt][1] *= a0; acc1[nt][2] *= a1; acc1[nt][3] *= a1;
            }
        }
        float p[MT][2];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const float mref = m_run[mt] == -INFINITY ? 0.0f : m_run[mt];
            p[mt][0] = __expf(lamv[mt][0] - mref);
            p[mt][1] = __expf(lamv[mt][1] - mref);
            l_run[mt] += p[mt][0] + p[mt][1];
        }

        // ---- value-product A operand: p * scale as fp16 hi + lo in rows 2 q and
        // 2 q + 1, tokens j and 16 + j packed in dword j % 4 of k-block j / 4
        uint32_t pr[2][NGM];
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int k = 0; k < NGM / 4; ++k) {
                const v4i w4 = *reinterpret_cast<const v4i *>(pst + (16 * c + j) * NGM + 4 * k);
#pragma unroll
                for (int e = 0; e < 4; ++e) pr[c][4 * k + e] = static_cast<uint32_t>(w4[e]);
            }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int q = 4 * mt + kb;
            uint32_t *dst = afr + ((2 * q + 16 * (j / 4)) * 4 + (j % 4));
#pragma unroll
            for (int gg = 0; gg < NGM; ++gg) {
                if (gg < NG) {
                    const float w0 = p[mt][0] * f16_bits_to_f32(pr[0][gg] & 0xffffu);
                    const float w1 = p[mt][1] * f16_bits_to_f32(pr[1][gg] & 0xffffu);
                    zacc[mt][gg] = fmaf(p[mt][0], f16_bits_to_f32(pr[0][gg] >> 16),
                                        fmaf(p[mt][1], f16_bits_to_f32(pr[1][gg] >> 16), zacc[mt][gg]));
                    const auto hi = __builtin_amdgcn_cvt_pkrtz(w0, w1);
                    const auto lo = __builtin_amdgcn_cvt_pkrtz(w0 - static_cast<float>(hi[0]), w1 - static_cast<float>(hi[1]));
                    dst[gg * 256] = __builtin_bit_cast(uint32_t, hi);
                    dst[gg * 256 + 4] = __builtin_bit_cast(uint32_t, lo);
                }
            }
        }

        // ---- value product over the 32 tokens, all channel tiles
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const int g_lo = (NF * 16 * cb) >> (__builtin_ctz(a.group));
            const v8h af0 = __builtin_bit_cast(v8h, *reinterpret_cast<const v4i *>(afr + g_lo * 256 + lane * 4));
            v8h af1 = af0;
            if (kTwoGroups && NF * 16 > a.group)
                af1 = __builtin_bit_cast(v8h, *reinterpret_cast<const v4i *>(afr + (g_lo + 1) * 256 + lane * 4));
            const v2i raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i *)(tr_base + 16 * cb));
            const uint32_t x0 = static_cast<uint32_t>(raw.x), x1 = static_cast<uint32_t>(raw.y);
            const uint32_t y0 = x0 >> 8, y1 = x1 >> 8;
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                // field f of every byte, in place: the fp16 subnormal code * 2^(VBITS f - 24)
                const uint32_t fm = (VBITS == 4 ? 0x000F000Fu : 0x00030003u) << (VBITS * f);
                const v4i bop = {static_cast<int>(x0 & fm), static_cast<int>(y0 & fm),
                                 static_cast<int>(x1 & fm), static_cast<int>(y1 & fm)};
                const v8h bv = __builtin_bit_cast(v8h, bop);
                const int nt = cb * NF + f;
                acc0[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af0, bv, acc0[nt], 0, 0, 0);
                if (kTwoGroups && NF * 16 > a.group)
                    acc1[kTwoGroups ? nt : 0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af1, bv, acc1[kTwoGroups ? nt : 0], 0, 0, 0);
            }
        }
    };

    // two tiles per trip, the loads of each issued one tile ahead; an odd
    // last tile is computed after the loop
    if (first < t_end) {
        Prefetch pa, pb;
        fetch(first, pa);
        int64_t t = first;
        for (; t + 4 * TK < t_end; t += 8 * TK) {
            fetch(t + 4 * TK, pb);
            compute(t, pa);
            fetch(t + 8 * TK, pa);
            compute(t + 4 * TK, pb);
        }
        if (t < t_end) compute(t, pa);
    }

    // ---- merge the four waves: m, l, zero-point sums and value sums per query
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int g = 4 * mt + kb;
        const float l = row16_sum(l_run[mt]);
        if (j == 0) {
            s_wm[wave][g] = m_run[mt];
            s_wl[wave][g] = l;
        }
#pragma unroll
        for (int gg = 0; gg < NGM; ++gg) {
            const float z = row16_sum(zacc[mt][gg]);
            if (j == 0) s_wz[wave][g][gg] = z;
        }
    }
    __syncthreads();        // every wave is done with its tile buffers
    float *wo = reinterpret_cast<float *>(smem);      // [4 waves][kMaxG][D]
#pragma unroll
    for (int nt = 0; nt < NTILE; ++nt) {
        const int cb = nt / NF, f = nt % NF;
        const int ch = NF * (16 * cb + j) + f;
        const int g_lo = (NF * 16 * cb) / a.group;
        const v4f acc = (kTwoGroups && NF * 16 > a.group && ch / a.group != g_lo) ? acc1[kTwoGroups ? nt : 0] : acc0[nt];
        const float sc = 16777216.0f / static_cast<float>(1 << (VBITS * f));
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
            const int g = 2 * kb + qq;
            wo[(wave * kMaxG + g) * D + ch] = sc * (acc[2 * qq] + acc[2 * qq + 1]);
        }
    }
    __syncthreads();
    for (int i = tid; i < GC * D; i += kThreads) {
        const int g = i / D, ch = i % D, grp = ch / a.group;
        float mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) mx = fmaxf(mx, s_wm[w][g]);
        float l = 0.0f, o = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float e = (s_wm[w][g] == -INFINITY) ? 0.0f : __expf(s_wm[w][g] - mx);
            l = fmaf(e, s_wl[w][g], l);
            o = fmaf(e, wo[(w * kMaxG + g) * D + ch] + s_wz[w][g][grp], o);
        }
        if (a.splits == 1) {
            a.out[(row0 + g) * D + ch] = l > 0.0f ? o / l : 0.0f;
        } else {
            a.part_acc[((row0 + g) * a.splits + split) * D + ch] = o;
            if (ch == 0) {
                a.part_ml[((row0 + g) * a.splits + split) * 2 + 0] = mx;
                a.part_ml[((row0 + g) * a.splits + split) * 2 + 1] = l;
            }
        }
    }
}

// ------------------------------------------------------------ split merge
// One workgroup per query row: out = sum_s e^(m_s - M) acc_s / sum_s e^(m_s - M) l_s
// (M the largest split maximum), split weights staged through LDS 256 at a time.
__global__ __launch_bounds__(kThreads) void k_merge_splits(DecodeLaunch a)
{
    __shared__ float red[kThreads / 64];
    __shared__ float wts[kThreads];
    const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
    const int64_t row = blockIdx.x;
    const int S = a.splits, D = a.d;
    const float *ml = a.part_ml + row * S * 2;
    float mx = -INFINITY;
    for (int s = tid; s < S; s += kThreads)
        if (ml[2 * s + 1] > 0.0f) mx = fmaxf(mx, ml[2 * s]);
    mx = wave_max(mx);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    float l = 0.0f;
    for (int s = tid; s < S; s += kThreads)
        if (ml[2 * s + 1] > 0.0f) l = fmaf(ml[2 * s + 1], __expf(ml[2 * s] - mx), l);
    l = wave_sum(l);
    if (lane == 0) red[wave] = l;
    __syncthreads();
    l = red[0] + red[1] + red[2] + red[3];
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    const float *pa = a.part_acc + row * S * D;
    float o = 0.0f;
    for (int s0 = 0; s0 < S; s0 += kThreads) {
        __syncthreads();
        const int s = s0 + tid;
        wts[tid] = (s < S && ml[2 * s + 1] > 0.0f) ? __expf(ml[2 * s] - mx) * inv : 0.0f;
        __syncthreads();
        const int n = S - s0 < kThreads ? S - s0 : kThreads;
        if (tid < D) {
            int k = 0;
            for (; k + 8 <= n; k += 8) {
                float v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) v[u] = pa[static_cast<int64_t>(s0 + k + u) * D + tid];
#pragma unroll
                for (int u = 0; u < 8; ++u) o = fmaf(wts[k + u], v[u], o);
            }
            for (; k < n; ++k) o = fmaf(wts[k], pa[static_cast<int64_t>(s0 + k) * D + tid], o);
        }
    }
    if (tid < D) a.out[row * D + tid] = o;
}

template <int BITS, int D, int MT, int VBITS>
hipError_t launch_mfma_t(const DecodeLaunch &a, hipStream_t stream, float kappa, int64_t chunk)
{
    const dim3 grid(static_cast<unsigned>(a.splits), static_cast<unsigned>(a.mf.units));
    void *tok;
    prof_begin("tq_attend_splitk", stream, &tok);
    hipLaunchKernelGGL((k_attend_mfma<BITS, D, MT, VBITS>), grid, dim3(kThreads), 0, stream, a, kappa, chunk);
    prof_end(tok, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1) return e;
    prof_begin("tq_merge_splits", stream, &tok);
    hipLaunchKernelGGL(k_merge_splits, dim3(static_cast<unsigned>(static_cast<int64_t>(a.B) * a.Hq)), dim3(kThreads), 0,
                       stream, a);
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
    const int64_t tiles = (a.T + kMfmaTile - 1) / kMfmaTile;
    const int64_t chunk = ((tiles + a.splits - 1) / a.splits) * kMfmaTile;
    return a.bits == 1 ? launch_mfma_d<1>(a, stream, kappa, chunk) : launch_mfma_d<2>(a, stream, kappa, chunk);
}

}  // namespace tq

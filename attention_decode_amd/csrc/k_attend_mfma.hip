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

// value of a limb-row quadruple: c0 + 128 c1 + 128^2 c2 + 128^3 c3 (each |c| < 2^23,
// so the two pair sums are exact in int32)
__device__ __forceinline__ float limbs_to_float(v4i c)
{
    const int lo = c[0] + (c[1] << 7), hi = c[2] + (c[3] << 7);
    return fmaf(static_cast<float>(hi), 16384.0f, static_cast<float>(lo));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// wavefront sum: DPP within each 16-lane row (quad swaps, half-row and row
// mirrors), then the four row sums read from lanes 0, 16, 32, 48; the result
// is wave-uniform
__device__ __forceinline__ float wave_sum(float x)
{
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x141>(x);
    x += dpp<0x140>(x);
    const int xi = __builtin_bit_cast(int, x);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 48));
    return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ float load1(const float *p) { return *p; }
__device__ __forceinline__ float load1(const bf16_t *p) { return bf16_to_f32(p->bits); }
__device__ __forceinline__ float load1(const f16_t *p) { return f16_bits_to_f32(p->bits); }

// unit index -> first query row
__device__ __forceinline__ int64_t unit_row0(const DecodeLaunch &a, int unit)
{
    const int qc = unit % a.mf.nqc, bh = unit / a.mf.nqc;
    const int b = bh / a.Hkv, hkv = bh % a.Hkv;
    return static_cast<int64_t>(b) * a.Hq + hkv * (a.Hq / a.Hkv) + qc * a.mf.gc;
}

// ---------------------------------------------------------------- q-prep
// Score operands of the unit's queries (unit = sequence, KV head, query
// chunk): q_rot = Pi q and Sq = (S Pi) q ("turboquant-pytorch", section "What
// it does": the query is rotated once and projected once per decode step),
// converted to the A-operand layouts of the score products.  k-block kb of
// every score step reads coordinates [kb D/4, (kb + 1) D/4) of one of the two
// vectors, so workgroup (unit, part, kb) computes just that quarter of q_rot
// (part 0) or Sq (part 1): eight workgroups per unit, each with a short
// dependency chain.  The fixed-point exponents come from bounds that every
// workgroup evaluates alike, with no exchange between them: |q_rot_j| <= |q|
// (Pi is orthogonal) and |Sq_i| <= |q| max_i |(S Pi)_i|.  The constant terms
// use column sums of Pi and S Pi fixed at rotation set-up:
// sum_j q_rot_j = (1^T Pi) q and sum_i Sq_i = (1^T S Pi) q.
constexpr int kCodeExp = 10;       // centroid tables hold c * 2^kCodeExp

__device__ __forceinline__ uint32_t f16_rn_bits(float x) { return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x)); }

template <typename TIn, int D, int GQ>
__global__ __launch_bounds__(kThreads) void k_qprep(DecodeLaunch a)
{
    constexpr int CB = D / 4;                  // coordinates of the quarter
    constexpr int R = kThreads / CB;           // row parts of each product
    constexpr int NR = D / R;                  // matrix rows per thread
    __shared__ float qs[GQ][D];
    __shared__ float red[R][GQ][CB];
    __shared__ float xv[GQ][CB];
    __shared__ int s_f[GQ][2];
    __shared__ float s_acoef[2];
    const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
    const int unit = blockIdx.x, part = blockIdx.y / 4, kb = blockIdx.y % 4;
    const bool bitplane = a.bits <= 2 && !a.kfmt_block;
    const int64_t row0 = unit_row0(a, unit);
    // this thread's rows of the matrix column: issued before the query load,
    // which they do not depend on
    const float *mtx = part ? a.spiT : a.piT;     // [D][D], row j = input coordinate
    const int cl = tid % CB, jp = tid / CB;
    float mv[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) mv[i] = mtx[(jp * NR + i) * D + kb * CB + cl];
    // table scores at d = 256 take int8 sign products (ScoreLut::I8S)
    constexpr bool kI8S = D == 256;
    // column sums for the constant terms (bit-plane codes, and the int8 QJL
    // sign sums, written by the (part 0, quarter 0) workgroup): coordinates
    // lane + 64 i of this lane
    const bool head = blockIdx.y == 0;
    const bool sums = head && (bitplane || (kI8S && !a.kfmt_block));
    float psum[D / 64], pssum[D / 64];
    if (sums) {
#pragma unroll
        for (int i = 0; i < D / 64; ++i) {
            psum[i] = a.pisum[lane + 64 * i];
            pssum[i] = a.spisum[lane + 64 * i];
        }
    }
    {
        const int i = 8 * tid, g = i / D, c = i % D;
        if (g < GQ) {
            float v[8];
            load8_as_f32(static_cast<const TIn *>(a.q) + (row0 + g) * D + c, v);
#pragma unroll
            for (int e = 0; e < 8; ++e) qs[g][c + e] = v[e];
        }
    }
    if (tid == 0) {
        // bit-affine form of a symmetric 1- or 2-bit codebook
        s_acoef[0] = bitplane ? a.centroids[1] - a.centroids[0] : 0.0f;
        s_acoef[1] = (a.bits == 2) ? a.centroids[2] - a.centroids[0] : 0.0f;
    }
    __syncthreads();
    {
        float acc[GQ];
#pragma unroll
        for (int g = 0; g < GQ; ++g) acc[g] = 0.0f;
#pragma unroll
        for (int i = 0; i < NR; ++i)
#pragma unroll
            for (int g = 0; g < GQ; ++g) acc[g] = fmaf(mv[i], qs[g][jp * NR + i], acc[g]);
#pragma unroll
        for (int g = 0; g < GQ; ++g) red[jp][g][cl] = acc[g];
    }
    // per query: |q| bound, exponents; the (part 0, quarter 0) workgroup also
    // writes the scales and constant terms
    for (int g = wave; g < GQ; g += 4) {
        float s2 = 0.0f, sc = 0.0f, ss = 0.0f;
#pragma unroll
        for (int i = 0; i < D / 64; ++i) {
            const float x = qs[g][lane + 64 * i];
            s2 = fmaf(x, x, s2);
            if (sums) {
                sc = fmaf(psum[i], x, sc);
                ss = fmaf(pssum[i], x, ss);
            }
        }
        s2 = wave_sum(s2);
        if (sums) {
            sc = wave_sum(sc);
            ss = wave_sum(ss);
        }
        if (lane == 0) {
            const float qn = sqrtf(s2) * (1.0f + 0x1p-16f);      // >= max_j |q_rot_j|, rounding included
            const float mc = bitplane ? qn * fmaxf(fabsf(s_acoef[0]), fabsf(s_acoef[1])) : qn;
            const float ms = qn * a.sq_bound;
            // |scaled value| < 2^top: 2^26 for int8 digit rows (bit-plane and
            // block codes, bit-plane and d = 256 table signs), 2^10 for fp16
            // rows (table codes, d = 128 table signs)
            const int topc = (bitplane || a.kfmt_block) ? 26 : 10;
            const int tops = (bitplane || kI8S) ? 26 : 10;
            int ec = 0, es = 0;
            frexpf(mc, &ec);
            frexpf(ms, &es);
            const int fc = (mc > 0.0f) ? topc - ec : 0;
            const int fs = (ms > 0.0f) ? tops - es : 0;
            s_f[g][0] = fc;
            s_f[g][1] = fs;
            if (head) {
                float *sc4 = a.mf.qscal + (row0 + g) * 4;
                if (a.kfmt_block) {
                    sc4[0] = ldexpf(1.0f, -fc);
                    sc4[1] = sc4[2] = sc4[3] = 0.0f;
                } else if (bitplane) {
                    sc4[0] = ldexpf(1.0f, -fc);
                    sc4[1] = a.centroids[0] * sc;
                    sc4[2] = ldexpf(1.0f, -fs);
                    sc4[3] = ss;
                } else if (kI8S) {
                    sc4[0] = ldexpf(1.0f, -(fc + kCodeExp));
                    sc4[1] = 0.0f;
                    sc4[2] = ldexpf(1.0f, -fs);
                    sc4[3] = ss;
                } else {
                    sc4[0] = ldexpf(1.0f, -(fc + kCodeExp));
                    sc4[1] = ldexpf(1.0f, -fs);
                    sc4[2] = 0.0f;
                    sc4[3] = 0.0f;
                }
            }
        }
    }
    __syncthreads();
    for (int o = tid; o < GQ * CB; o += kThreads) {
        const int g = o / CB, c = o % CB;
        float x = 0.0f;
#pragma unroll
        for (int r = 0; r < R; ++r) x += red[r][g][c];
        xv[g][c] = x;
    }
    __syncthreads();
    if (a.kfmt_block) {
        // Block key formats: int8 digit rows of the 16x16x32 int8 product, one
        // 8-byte A slot per (row tile, block, lane) in aops[unit][MT][D/32][64];
        // lane (row 4 q + digit, k-block kk) holds coordinates 32 b + 8 kk + o(e)
        // of query 4 mt + q, with o(e) = e for 8-bit codes and the nibble order
        // {0, 2, 4, 6, 1, 3, 5, 7} (low nibbles, then high ones) for 4-bit codes.
        // With 4-bit codes stored as q + 8, qaux[row][b] = 8 sum_b x (in the
        // units of the integer block sums) removes the offset.
        constexpr int NB = D / 32, NBQ = CB / 32;
        const int MT = a.mf.mt;
        uint64_t *out = reinterpret_cast<uint64_t *>(a.mf.aops) + static_cast<int64_t>(unit) * MT * NB * 64;
        for (int w = tid; w < MT * NBQ * 64; w += kThreads) {
            const int ln = w % 64, bq = (w / 64) % NBQ, mt = w / (64 * NBQ);
            const int row = ln % 16, kk = ln / 16, g = 4 * mt + row / 4, digit = row % 4;
            uint64_t v = 0;
            if (g < GQ) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int o = a.bits == 8 ? e : (e < 4 ? 2 * e : 2 * (e - 4) + 1);
                    int x = static_cast<int>(rintf(ldexpf(xv[g][32 * bq + 8 * kk + o], s_f[g][0])));
                    for (int r = 0; r < digit; ++r) x = (x - (((x + 64) & 127) - 64)) >> 7;
                    const int dg = digit < 3 ? ((x + 64) & 127) - 64 : x;
                    v |= static_cast<uint64_t>(static_cast<uint32_t>(dg) & 0xffu) << (8 * e);
                }
            }
            out[(mt * NB + kb * NBQ + bq) * 64 + ln] = v;
        }
        for (int w = tid; w < GQ * NBQ; w += kThreads) {
            const int g = w / NBQ, bq = w % NBQ;
            double sum = 0.0;
            for (int e = 0; e < 32; ++e) sum += rintf(ldexpf(xv[g][32 * bq + e], s_f[g][0]));
            a.qaux[(row0 + g) * NB + kb * NBQ + bq] = a.bits == 4 ? static_cast<float>(8.0 * sum) : 0.0f;
        }
    } else if (bitplane) {
        // int8 digit rows: query g uses lanes 16 kb + 4 (g % 4) + digit of row
        // tile g / 4; dword r of a lane holds elements 4r..4r+3 of its k-block.
        // Code step s = 2u + h reads word u of the quarter (bit 32 u + 8 K + 4 h + r,
        // coordinate bit / bits); sign step 2 nc + 2u + h reads coordinate
        // 32 u + 8 K + 4 h + r of Sq.
        const int nc = code_dwords(D, a.bits), ns = a.m > 0 ? sign_dwords(D) : 0;
        const int S = 2 * nc + 2 * ns, MT = a.mf.mt;
        const int s_lo = part ? 2 * nc : 0, s_n = part ? 2 * ns : 2 * nc;
        uint32_t *out = a.mf.aops + static_cast<int64_t>(unit) * MT * S * 256;
        for (int w = tid; w < MT * 4 * s_n * 4; w += kThreads) {
            const int r = w % 4, sl = (w / 4) % s_n, g = w / (4 * s_n);
            const int u = sl / 2, h = sl % 2;
            uint32_t dw[4] = {0u, 0u, 0u, 0u};
            if (g < GQ) {
                const int f = s_f[g][part];
#pragma unroll
                for (int K = 0; K < 4; ++K) {
                    const int bit = 32 * u + 8 * K + 4 * h + r;
                    const float wv = part ? xv[g][bit] : xv[g][bit >> (a.bits - 1)] * s_acoef[bit & (a.bits - 1)];
                    // the key bit arrives as byte 2^sh (masked in place, not shifted):
                    // weight w 2^-sh, negated for sh = 7 where the byte reads as -128
                    const int sh = 4 * h + r;
                    int x = static_cast<int>(rintf(ldexpf(wv, f - sh)));
                    if (sh == 7) x = -x;
#pragma unroll
                    for (int limb = 0; limb < 3; ++limb) {
                        const int d = ((x + 64) & 127) - 64;
                        dw[limb] |= (static_cast<uint32_t>(d) & 0xffu) << (8 * K);
                        x = (x - d) >> 7;
                    }
                    dw[3] |= (static_cast<uint32_t>(x) & 0xffu) << (8 * K);
                }
            }
#pragma unroll
            for (int limb = 0; limb < 4; ++limb) {
                const int l = 16 * kb + 4 * (g % 4) + limb;
                out[((g / 4) * S + s_lo + sl) * 256 + l * 4 + r] = dw[limb];
            }
        }
    } else {
        // Table scores, aops[unit][step][lane][4 dwords] with the code steps
        // first, then the sign steps.
        // Code steps: fp16 hi + lo rows of the A operands of
        // v_mfma_f32_16x16x32_f16, row 4 kk + r holding query kk + 4 (r / 2)
        // at d = 256, 2 kk + r / 2 at d = 128, part r % 2 (kk the row block).
        // Two steps per ks, m = 0, 1, over
        // coordinates kb D/4 + 8 ks + 4 m + i, each coordinate repeated for the
        // hi and lo halves of its centroid in the B operand: slots (x0, x1, x0,
        // x1, x2, x3, x2, x3) against pair entries (up to 5 bits), (x0, x0, x1,
        // x1, x2, x2, x3, x3) against single entries.
        // Sign steps, d = 256: int8 digit rows of v_mfma_i32_16x16x64_i8 as
        // in the bit-plane scores, two row tiles of four queries (query g in
        // lanes 16 kb + 4 (g % 4) + digit of tile g / 4), tile-major; step sl
        // of a tile reads sign dword u = sl / 2 of the quarter, dword r of a
        // lane holding coordinates 32 u + 8 K + 4 (sl % 2) + r, K = 0..3.
        // Sign steps, d = 128: fp16 hi + lo rows in the code rows' order, step
        // ks holding coordinates kb D/4 + 8 ks + e of Sq.
        constexpr int KS = D / 32;
        const bool pair = a.bits <= 5;
        const int code_steps = 2 * KS;
        uint32_t *out = a.mf.aops + static_cast<int64_t>(unit) * (code_steps + KS) * 256;
        if (part == 0) {
            for (int w = tid; w < code_steps * 64; w += kThreads) {
                const int r = w % 4, row = (w / 4) % 16, st = w / 64;
                const int g = kI8S ? (row >> 2) + 4 * ((row >> 1) & 1) : row >> 1, lo = row & 1;
                // coordinates of this dword's two slots: c0 + h * dc
                const int base = 8 * (st / 2) + 4 * (st % 2);
                const int c0 = pair ? base + 2 * (r / 2) : base + r;
                const int dc = pair ? 1 : 0;
                uint32_t dw = 0u;
                if (g < GQ) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const float x = ldexpf(xv[g][c0 + h * dc], s_f[g][0]);
                        const _Float16 xh = static_cast<_Float16>(x);
                        const uint32_t bits = lo ? f16_rn_bits(x - static_cast<float>(xh)) : __builtin_bit_cast(uint16_t, xh);
                        dw |= bits << (16 * h);
                    }
                }
                out[(st * 64 + 16 * kb + row) * 4 + r] = dw;
            }
        } else if (!kI8S) {
            for (int w = tid; w < KS * 64; w += kThreads) {
                const int r = w % 4, row = (w / 4) % 16, st = w / 64;
                const int g = row >> 1, lo = row & 1;
                uint32_t dw = 0u;
                if (g < GQ) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const float x = ldexpf(xv[g][8 * st + 2 * r + h], s_f[g][1]);
                        const _Float16 xh = static_cast<_Float16>(x);
                        const uint32_t bits = lo ? f16_rn_bits(x - static_cast<float>(xh)) : __builtin_bit_cast(uint16_t, xh);
                        dw |= bits << (16 * h);
                    }
                }
                out[((code_steps + st) * 64 + 16 * kb + row) * 4 + r] = dw;
            }
        } else {
            constexpr int SS = D / 64;           // two steps per sign dword of a quarter
            uint32_t *sout = out + code_steps * 256;
            for (int w = tid; w < 2 * 4 * SS * 4; w += kThreads) {
                const int r = w % 4, sl = (w / 4) % SS, g = w / (4 * SS);
                const int u = sl / 2, h = sl % 2;
                uint32_t dw[4] = {0u, 0u, 0u, 0u};
                if (g < GQ) {
                    const int f = s_f[g][1];
#pragma unroll
                    for (int K = 0; K < 4; ++K) {
                        // the sign bit arrives as byte 2^sh (masked in place):
                        // weight Sq 2^-sh, negated for sh = 7 (the byte reads -128)
                        const int sh = 4 * h + r;
                        int x = static_cast<int>(rintf(ldexpf(xv[g][32 * u + 8 * K + sh], f - sh)));
                        if (sh == 7) x = -x;
#pragma unroll
                        for (int limb = 0; limb < 3; ++limb) {
                            const int d = ((x + 64) & 127) - 64;
                            dw[limb] |= (static_cast<uint32_t>(d) & 0xffu) << (8 * K);
                            x = (x - d) >> 7;
                        }
                        dw[3] |= (static_cast<uint32_t>(x) & 0xffu) << (8 * K);
                    }
                }
#pragma unroll
                for (int limb = 0; limb < 4; ++limb) {
                    const int l = 16 * kb + 4 * (g % 4) + limb;
                    sout[((g / 4) * SS + sl) * 256 + l * 4 + r] = dw[limb];
                }
            }
        }
    }
}


// ------------------------------------------------------------ attention
// Softmax runs in base 2: scores leave the score stage multiplied by
// scale log2(e) (the host's factor a.mf.lscale), so every weight is one
// v_exp_f32 (2^x; -inf gives 0).  The split maxima handed to the merge are in
// the same units.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-lane (one DPP row) reductions: xor 1, xor 2, half-row mirror, row mirror
// The maximum runs as four v_max_f32 with a DPP operand, each in place (every
// lane of a row reads its source before any lane writes); the s_nop covers the
// wait states between a VALU write and a DPP read of the same register.  The
// operands are finite scores or -inf, never NaN, so the IEEE quieting that
// fmaxf would add around a DPP move is not needed.
__device__ __forceinline__ float row16_max(float x)
{
    asm("s_nop 1\n\tv_max_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\tv_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\tv_max_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\tv_max_f32_dpp %0, %0, %0 row_mirror row_mask:0xf bank_mask:0xf"
        : "+v"(x));
    return x;
}

__device__ __forceinline__ float row16_sum(float x)
{
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x141>(x);
    return x + dpp<0x140>(x);
}

// Orders this wave's LDS writes before its later LDS reads by other lanes (and
// the reverse): a compiler-level fence at wavefront scope, free at run time,
// since one wave's LDS operations execute in order.
__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// k-slot order of a 32-token wave tile in the value product: slot 2j holds
// token j, slot 2j + 1 token 16 + j, so that the lane owning key column j of
// both score tiles writes its two tokens as one packed fp16 pair.
__device__ __forceinline__ int slot_token(int slot) { return (slot & 1) ? 16 + (slot >> 1) : (slot >> 1); }

// base + a 32-bit byte offset: with a wave-uniform base the load takes the
// base from scalar registers and the offset from one VGPR
template <class T>
__device__ __forceinline__ const T *at_bytes(const T *base, uint32_t off)
{
    return reinterpret_cast<const T *>(reinterpret_cast<const unsigned char *>(base) + off);
}

// The packed rows are read once per call.  Loads of a wave that cover whole
// cache lines carry the nontemporal hint (the "nt" bit), under which the
// memory system streams the lines instead of keeping them like reused data:
// the value rows, and the code and sign rows of keys whose quarter row a lane
// takes in one load (up to 16 bytes: 16 keys' whole rows per load).  A
// streaming read of 2 GiB in contiguous per-workgroup chunks runs at about
// 7.0 TB/s with the hint and 6.2 TB/s without.  Wider code rows (a line spread
// over several loads of a wave) and the per-key norms (half a line per load)
// keep plain loads: the hint made those slower.
template <class T>
__device__ __forceinline__ T ld_stream(const T *p)
{
    return __builtin_nontemporal_load(p);
}

// Key words of the two keys (columns j and 16 + j of a wave tile) that lane
// (j, kb) reads: the kb-th quarter of the code row and of the sign row.  The
// first-stage format (QJL false) has no sign row and no residual norm.
// Loads go through wave-uniform plane bases of the tile (scalar registers)
// plus 32-bit lane offsets.
template <int BITS, int D, bool QJL>
struct KeyWords {
    static constexpr int NC = D * BITS / 128, NS = QJL ? D / 128 : 0;
    uint32_t cw[2][NC], sw[2][NS > 0 ? NS : 1];
    float nrm[2], rho[2];
    struct Bases {
        const uint32_t *c, *s;
        const float *n, *r;
    };
    __device__ static Bases bases(const DecodeLaunch &a, int64_t n0)
    {
        return {reinterpret_cast<const uint32_t *>(a.kc.codes) + n0 * (D * BITS / 32),
                reinterpret_cast<const uint32_t *>(a.kc.signs) + n0 * (D / 32), a.kc.knorm + n0, a.kc.rnorm + n0};
    }
    // key t of the tile (column c of this lane: key j or 16 + j), k-block kb
    static constexpr bool STREAM = NC <= 4;     // a lane's quarter row in one load
    __device__ void load(const Bases &b, uint32_t t, int kb, int c)
    {
        const uint32_t *crow = at_bytes(b.c, 4u * (t * (D * BITS / 32) + kb * NC));
#pragma unroll
        for (int u = 0; u < NC; ++u) cw[c][u] = STREAM ? ld_stream(crow + u) : crow[u];
        nrm[c] = *at_bytes(b.n, 4u * t);
        if constexpr (QJL) {
            const uint32_t *srow = at_bytes(b.s, 4u * (t * (D / 32) + kb * NS));
#pragma unroll
            for (int u = 0; u < NS; ++u) sw[c][u] = ld_stream(srow + u);
            rho[c] = *at_bytes(b.r, 4u * t);
        } else {
            rho[c] = 0.0f;
        }
    }
};

// Bit-plane scores (1-2 bit keys).  Rows of the int8 products are (query,
// digit), four queries per 16-row tile: lane (j, kb) scores query 4 slot + kb.
template <int BITS, int D, int MT, bool QJL>
struct ScoreBits {
    using KW = KeyWords<BITS, D, QJL>;
    static constexpr int NQ = MT;
    static constexpr int TAB_BYTES = 0;
    static constexpr bool OCC3 = false;     // three workgroups measured no faster
    static constexpr int NC = D * BITS / 128, NS = QJL ? D / 128 : 0;
    static constexpr int SC = 2 * NC, SS = 2 * NS, S = SC + SS;
    v4i aop[MT][S];
    float fc[MT], cc[MT], fs[MT], ssq[MT];

    __device__ static int query(int slot, int kb) { return 4 * slot + kb; }

    // value of a per-slot quantity for query q, fetched from a lane of the
    // row block that scores q (block q % 4, slot q / 4)
    __device__ static float for_query(const float (&v)[MT], int q, int j)
    {
        float r = 1.0f;
#pragma unroll
        for (int s = 0; s < MT; ++s) {
            const float t = __shfl(v[s], 16 * (q % 4) + j);
            if (q / 4 == s) r = t;
        }
        return r;
    }

    __device__ void init(const DecodeLaunch &a, int unit, int64_t row0, int lane, int kb, int GC, float kappa, unsigned char *)
    {
        const v4i *src = reinterpret_cast<const v4i *>(a.mf.aops) + static_cast<int64_t>(unit) * MT * S * 64;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int s = 0; s < S; ++s) aop[mt][s] = src[(mt * S + s) * 64 + lane];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int g = 4 * mt + kb;
            const bool ok = g < GC;
            // loaded unconditionally (row clamped): no wait on the operand
            // loads in flight until the scores need them
            const float4 sc = *reinterpret_cast<const float4 *>(a.mf.qscal + (row0 + (ok ? g : 0)) * 4);
            // scores leave in log2 units of the softmax: scale log2(e) and the
            // QJL factor kappa are folded into the per-query terms
            const float f = a.mf.lscale, fk = f * kappa;
            fc[mt] = ok ? sc.x * f : 0.0f;
            cc[mt] = ok ? sc.y * f : 0.0f;
            fs[mt] = ok ? 2.0f * sc.z * fk : 0.0f;
            ssq[mt] = ok ? sc.w * fk : 0.0f;
        }
    }

    __device__ void scores(const KW &kw, float (&sc)[2][MT]) const
    {
        score_tile(kw, 0, sc[0]);
        score_tile(kw, 1, sc[1]);
    }

    // B bytes are raw key bits at weight 2^k (mask without shift; the digit
    // rows carry the 2^-k); returns n (sum q_rot c + kappa rho sum Sq (2s - 1))
    // per slot, times scale log2(e)
    __device__ void score_tile(const KW &kw, int c, float (&sc)[MT]) const
    {
        v4i accc[MT], accs[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) accc[mt] = accs[mt] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < SC; ++s) {
            const uint32_t dw = kw.cw[c][s / 2];
            const int h = 4 * (s % 2);
            const v4i bop = {static_cast<int>(dw & (0x01010101u << h)), static_cast<int>(dw & (0x01010101u << (h + 1))),
                             static_cast<int>(dw & (0x01010101u << (h + 2))), static_cast<int>(dw & (0x01010101u << (h + 3)))};
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) accc[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop[mt][s], bop, accc[mt], 0, 0, 0);
        }
#pragma unroll
        for (int s = 0; s < SS; ++s) {
            const uint32_t dw = kw.sw[c][s / 2];
            const int h = 4 * (s % 2);
            const v4i bop = {static_cast<int>(dw & (0x01010101u << h)), static_cast<int>(dw & (0x01010101u << (h + 1))),
                             static_cast<int>(dw & (0x01010101u << (h + 2))), static_cast<int>(dw & (0x01010101u << (h + 3)))};
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                accs[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop[mt][SC + s], bop, accs[mt], 0, 0, 0);
        }
        // lane (key column j, row block kb) holds the four digits of query 4 mt + kb
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const float dcode = fmaf(limbs_to_float(accc[mt]), fc[mt], cc[mt]);
            if constexpr (QJL) {
                const float dsign = fmaf(limbs_to_float(accs[mt]), fs[mt], -ssq[mt]);
                sc[mt] = kw.nrm[c] * fmaf(kw.rho[c], dsign, dcode);
            } else {
                sc[mt] = kw.nrm[c] * dcode;
            }
        }
    }
};

// Table scores (3-7 bit keys).  The key's centroids are looked up in LDS as
// fp16 hi + lo (c * 2^kCodeExp); the code products run on
// v_mfma_f32_16x16x32_f16 with rows (query, hi/lo part of the query).
// The QJL sign bits:
//   d = 128: each sign byte indexes a 256-entry LDS table of eight fp16 +-1,
//     in a product with the same rows; row 4 kb + r holds query 2 kb + r / 2,
//     part r % 2, so lane (j, kb) scores queries 2 kb and 2 kb + 1.
//   d = 256 (I8S): as in the bit-plane scores, masked in place into int8
//     operands against int8 digit rows of Sq (v_mfma_i32_16x16x64_i8, row
//     tile t holding queries 4 t .. 4 t + 3, lane block kb the digits of query
//     4 t + kb), with no table; the code rows follow, row 4 kb + r holding
//     query kb + 4 (r / 2), so lane (j, kb) scores queries kb and kb + 4.  With
//     at most four query heads one int8 tile takes the 32 x 8 sign bits of a
//     key in half the products of the fp16 form.
// The hi and lo
// halves of the centroids share one product over 16 coordinates: up to 5 bits
// an 8-byte entry (hi pair, lo pair) per two coordinates, read with one
// ds_read_b64, two entries making the lane's B quad (hi01, lo01, hi23, lo23)
// against A slots (x0, x1, x0, x1, x2, x3, x2, x3); from 6 bits a 4-byte
// entry (hi | lo << 16) per coordinate, four making the quad against A slots
// (x0, x0, x1, x1, x2, x2, x3, x3).
template <int BITS, int D, bool QJL, int TB = 8192>
struct ScoreLut {
    using KW = KeyWords<BITS, D, QJL>;
    static constexpr int NQ = 2;
    static constexpr bool OCC3 = true;
    static constexpr int KS = D / 32;
    static constexpr bool PAIR = BITS <= 5;
    static constexpr int NENT = PAIR ? (1 << (2 * BITS)) : (1 << BITS);
    static constexpr int EBYTES = PAIR ? 8 : 4;                       // bytes per table entry
    // copies of the code table within TB bytes, interleaved entry-major so
    // that lane l reads copy l % COPIES (fewer lanes per bank).  The budget is
    // 8 KB, and 4 KB at d = 128 with 4-bit values, whose larger value staging
    // would otherwise leave room for two workgroups per CU instead of three.
    static constexpr int COPIES_RAW = TB / (NENT * EBYTES);
    static constexpr int COPIES = COPIES_RAW >= 64 ? 64 : (COPIES_RAW >= 32 ? 32 : (COPIES_RAW >= 16 ? 16 : (COPIES_RAW >= 8 ? 8 : (COPIES_RAW >= 4 ? 4 : 1))));
    static constexpr int CODE_TAB = NENT * EBYTES * COPIES;
    static constexpr bool I8S = QJL && D == 256;                      // int8 sign products
    static constexpr int SIGN_TAB = (QJL && !I8S) ? 256 * 16 : 0;
    // int8 sign K-steps: two per sign dword of a lane (the bits at positions
    // 0-3 and 4-7 of each byte), for each of the two row tiles
    static constexpr int SS = I8S ? 2 * (D / 128) : 0;
    // the unit's A operands, [step][64 lanes] with CODE_STEPS code steps then
    // KS sign steps (fp16; or int8, 2 SS = KS, tile-major): in registers for
    // the first-stage format at d = 128 (no sign steps), else in LDS, shared
    // by the four waves and read per k-step (registers for both parts cost a
    // workgroup per CU, which measured slower)
    static constexpr int CODE_STEPS = 2 * KS;
    static constexpr int NSTEP = CODE_STEPS + KS;                     // per unit in the workspace
    static_assert(!I8S || 2 * SS == KS, "two int8 sign tiles fill the workspace's KS sign steps");
    static constexpr bool AREG = D == 128 && !QJL;
    static constexpr int LSTEP = CODE_STEPS + (QJL ? KS : 0);         // steps kept in LDS
    static constexpr int AOP_BYTES = AREG ? 0 : LSTEP * 64 * 16;
    static constexpr int TAB_BYTES = CODE_TAB + SIGN_TAB + AOP_BYTES;
    template <int TB2>
    using WithTable = ScoreLut<BITS, D, QJL, TB2>;
    float scc[2], scs[2], ssq[2];
    v4i areg[AREG ? CODE_STEPS : 1];
    const unsigned char *tab;
    uint32_t copyb;            // byte offset of this lane's table copy within an entry
    int lane_;
    bool two_;                 // I8S: the second sign tile (queries 4-7) holds a query of the unit

    __device__ static int query(int slot, int kb) { return I8S ? kb + 4 * slot : 2 * kb + slot; }

    // the lane (of column j) and the slot that score query q
    __device__ static constexpr int lane_of(int q, int j) { return I8S ? 16 * (q % 4) + j : 16 * (q / 2) + j; }
    __device__ static constexpr int slot_of(int q) { return I8S ? q / 4 : q % 2; }

    // value of a per-slot quantity for query q, fetched from a lane that
    // scores q (d = 128: the callers ask for queries 2 kb and 2 kb + 1, this
    // lane's own slots)
    __device__ static float for_query(const float (&v)[2], int q, int j)
    {
        if constexpr (!I8S) {
            return v[q % 2];
        } else {
            const float t0 = __shfl(v[0], lane_of(q, j)), t1 = __shfl(v[1], lane_of(q, j));
            return slot_of(q) ? t1 : t0;
        }
    }

    // builds the tables (all threads; the caller synchronises) and loads the operands
    __device__ void init(const DecodeLaunch &a, int unit, int64_t row0, int lane, int kb, int GC, float kappa, unsigned char *lds)
    {
        tab = lds;
        copyb = static_cast<uint32_t>(EBYTES * (lane % COPIES));
        const int tid = threadIdx.x;
        constexpr int L = 1 << BITS;
        if (PAIR) {
            uint2 *t2 = reinterpret_cast<uint2 *>(lds);
            for (int x = tid; x < L * L * COPIES; x += kThreads) {
                const int i = x / COPIES;
                const float c0 = ldexpf(a.centroids[i & (L - 1)], kCodeExp), c1 = ldexpf(a.centroids[i >> BITS], kCodeExp);
                const _Float16 h0 = static_cast<_Float16>(c0), h1 = static_cast<_Float16>(c1);
                t2[x] = make_uint2(__builtin_bit_cast(uint16_t, h0) | (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h1)) << 16),
                                   f16_rn_bits(c0 - static_cast<float>(h0)) | (f16_rn_bits(c1 - static_cast<float>(h1)) << 16));
            }
        } else {
            uint32_t *t1 = reinterpret_cast<uint32_t *>(lds);
            for (int x = tid; x < L * COPIES; x += kThreads) {
                const float c0 = ldexpf(a.centroids[x / COPIES], kCodeExp);
                const _Float16 h0 = static_cast<_Float16>(c0);
                t1[x] = __builtin_bit_cast(uint16_t, h0) | (f16_rn_bits(c0 - static_cast<float>(h0)) << 16);
            }
        }
        uint32_t *ts = reinterpret_cast<uint32_t *>(lds + CODE_TAB);
        for (int i = tid; i < (SIGN_TAB ? 256 * 4 : 0); i += kThreads) {
            const int e = i / 4, r = i % 4;
            const uint32_t lo = ((e >> (2 * r)) & 1) ? 0x3C00u : 0xBC00u;
            const uint32_t hi = ((e >> (2 * r + 1)) & 1) ? 0x3C00u : 0xBC00u;
            ts[i] = lo | (hi << 16);
        }
        const v4i *src = reinterpret_cast<const v4i *>(a.mf.aops) + static_cast<int64_t>(unit) * NSTEP * 64;
        if constexpr (AREG) {
#pragma unroll
            for (int st = 0; st < CODE_STEPS; ++st) areg[st] = src[st * 64 + lane];
        } else {
            v4i *adst = reinterpret_cast<v4i *>(lds + CODE_TAB + SIGN_TAB);
            for (int i = tid; i < LSTEP * 64; i += kThreads) adst[i] = src[i];
        }
        lane_ = lane;
        two_ = GC > 4;
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
            const int g = query(qq, kb);
            const bool ok = g < GC;
            const float4 sc = *reinterpret_cast<const float4 *>(a.mf.qscal + (row0 + (ok ? g : 0)) * 4);
            // scores leave in log2 units of the softmax (scale log2(e) folded
            // in); the int8 sign sum is 2 sum Sq s - sum Sq for bits s in {0, 1}
            const float f = a.mf.lscale, fk = f * kappa;
            scc[qq] = ok ? sc.x * f : 0.0f;
            scs[qq] = ok ? (I8S ? 2.0f * sc.z : sc.y) * fk : 0.0f;
            ssq[qq] = ok && I8S ? sc.w * fk : 0.0f;
        }
    }

    // byte offset of the table entry for the W-bit field at bit offset o of a
    // lane's word array (o constant after unrolling): the field lands at bit
    // ESH = log2(entry stride) by one shift, so with the copy bits or-ed in the
    // offset costs a shift and an and-or
    static constexpr int ESH = __builtin_ctz(EBYTES * COPIES);
    template <int W, int NW>
    __device__ uint32_t entry(const uint32_t (&w)[NW], int o) const
    {
        const int i = o / 32, s = o % 32;
        constexpr uint32_t mask = ((1u << W) - 1u) << ESH;
        uint32_t x;
        if (s + W <= 32 || i + 1 >= NW) x = s >= ESH ? (w[i] >> (s - ESH)) : (w[i] << (ESH - s));
        else x = __builtin_amdgcn_alignbit(w[i + 1], w[i], s) << ESH;
        uint32_t off = (x & mask) | copyb;
        // keeps the offset one v_and_or (the table base then folds into the
        // LDS instruction's offset field instead of a separate add)
        asm("" : "+v"(off));
        return off;
    }

    __device__ void scores(const KW &kw, float (&sc)[2][2]) const
    {
        const v4i *ts = reinterpret_cast<const v4i *>(tab + CODE_TAB);
        const v4i *aop = reinterpret_cast<const v4i *>(tab + CODE_TAB + SIGN_TAB);
        v4f accc[2], accf[2];     // code products; fp16 sign products (d = 128)
        v4i accs[2][I8S ? 2 : 1]; // int8 sign products [key column][sign tile]
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            accc[c] = accf[c] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int t = 0; t < (I8S ? 2 : 1); ++t) accs[c][t] = v4i{0, 0, 0, 0};
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if constexpr (PAIR) {
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const int st = 2 * ks + m;
                    v8h acode;
                    if constexpr (AREG) acode = __builtin_bit_cast(v8h, areg[st]);
                    else acode = __builtin_bit_cast(v8h, aop[st * 64 + lane_]);
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        const uint2 t0 = *reinterpret_cast<const uint2 *>(
                            tab + entry<2 * BITS>(kw.cw[c], 8 * BITS * ks + 2 * BITS * (2 * m)));
                        const uint2 t1 = *reinterpret_cast<const uint2 *>(
                            tab + entry<2 * BITS>(kw.cw[c], 8 * BITS * ks + 2 * BITS * (2 * m + 1)));
                        const v4i b = {static_cast<int>(t0.x), static_cast<int>(t0.y), static_cast<int>(t1.x),
                                       static_cast<int>(t1.y)};
                        accc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(acode, __builtin_bit_cast(v8h, b), accc[c], 0, 0, 0);
                    }
                }
            } else {
                const uint32_t *t1 = reinterpret_cast<const uint32_t *>(tab);
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const int st = 2 * ks + m;
                    v8h acode;
                    if constexpr (AREG) acode = __builtin_bit_cast(v8h, areg[st]);
                    else acode = __builtin_bit_cast(v8h, aop[st * 64 + lane_]);
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        v4i b;
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            b[i] = static_cast<int>(*at_bytes(t1, entry<BITS>(kw.cw[c], 8 * BITS * ks + BITS * (4 * m + i))));
                        accc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(acode, __builtin_bit_cast(v8h, b), accc[c], 0, 0, 0);
                    }
                }
            }
            if constexpr (QJL && !I8S) {
                const v8h asign = __builtin_bit_cast(v8h, aop[(CODE_STEPS + ks) * 64 + lane_]);
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const uint32_t sb = (kw.sw[c][ks / 4] >> (8 * (ks % 4))) & 0xffu;
                    accf[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(asign, __builtin_bit_cast(v8h, ts[sb]), accf[c], 0, 0, 0);
                }
            }
        }
        if constexpr (I8S) {
            // sign step s: the bits at 4 (s % 2) .. 4 (s % 2) + 3 of each byte of
            // sign dword s / 2, masked in place (byte value 2^k; the digit rows
            // carry 2^-k, negated for k = 7)
            const v4i *asg = aop + CODE_STEPS * 64 + lane_;
#pragma unroll
            for (int st = 0; st < SS; ++st) {
                const int h = 4 * (st % 2);
                const v4i a0 = asg[st * 64];
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const uint32_t dw = kw.sw[c][st / 2];
                    const v4i bop = {static_cast<int>(dw & (0x01010101u << h)), static_cast<int>(dw & (0x01010101u << (h + 1))),
                                     static_cast<int>(dw & (0x01010101u << (h + 2))), static_cast<int>(dw & (0x01010101u << (h + 3)))};
                    accs[c][0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, bop, accs[c][0], 0, 0, 0);
                }
                if (two_) {
                    const v4i a1 = asg[(SS + st) * 64];
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        const uint32_t dw = kw.sw[c][st / 2];
                        const v4i bop = {static_cast<int>(dw & (0x01010101u << h)), static_cast<int>(dw & (0x01010101u << (h + 1))),
                                         static_cast<int>(dw & (0x01010101u << (h + 2))), static_cast<int>(dw & (0x01010101u << (h + 3)))};
                        accs[c][1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, bop, accs[c][1], 0, 0, 0);
                    }
                }
            }
        }
        // code and fp16 sign rows 4 kb + r: (query(r / 2, kb), part r % 2);
        // int8 sign tile qq: lane block kb holds the four digits of query kb + 4 qq
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) {
                const float dcode = (accc[c][2 * qq] + accc[c][2 * qq + 1]) * scc[qq];
                if constexpr (QJL) {
                    float dsign;
                    if constexpr (I8S) dsign = fmaf(limbs_to_float(accs[c][qq]), scs[qq], -ssq[qq]);
                    else dsign = (accf[c][2 * qq] + accf[c][2 * qq + 1]) * scs[qq];
                    sc[c][qq] = kw.nrm[c] * fmaf(kw.rho[c], dsign, dcode);
                } else {
                    sc[c][qq] = kw.nrm[c] * dcode;
                }
            }
    }
};

// One 256-thread workgroup owns one (sequence, KV head, query chunk) and one
// token range; each wave walks its own 32-key tiles (wave w takes tiles w,
// w + 4, ...) with its own online-softmax state and value accumulators, so
// the tile loop has no workgroup barrier.  Loads of the next tile are issued
// before the current one is computed (two register buffers in turn).  The
// four waves are merged in LDS at the end; with one split the workgroup
// writes the normalised output, else its partial (max, sum, weighted values).
// Rotated block key formats (8-bit or 4-bit codes, one fp16 scale per 32
// rotated coordinates).  Lane (j, kb) holds, for each block, the 8 codes at
// coordinates 32 b + 8 kb .. + 7 of keys j and 16 + j (two dwords of bytes,
// or one dword of nibbles) and the keys' block scales.
template <int QB, int D>
struct KeyWordsQ {
    static constexpr int NB = D / 32;
    static constexpr int WB = QB == 8 ? 2 : 1;     // code dwords per block and lane
    static constexpr int PB = QB;                  // code dwords per block (32 codes)
    static constexpr int ROWW = D * QB / 32;       // code dwords per key
    static constexpr int SW = D / 64;              // scale dwords per key (fp16 pairs)
    static constexpr int NC = 0, NS = 0;
    uint32_t cw[2][NB * WB];
    uint32_t sc[2][SW];
    struct Bases {
        const uint32_t *c, *s;
    };
    __device__ static Bases bases(const DecodeLaunch &a, int64_t n0)
    {
        return {reinterpret_cast<const uint32_t *>(a.kq.codes) + n0 * ROWW,
                reinterpret_cast<const uint32_t *>(a.kq.scales) + n0 * SW};
    }
    __device__ void load(const Bases &b, uint32_t t, int kb, int c)
    {
#pragma unroll
        for (int blk = 0; blk < NB; ++blk)
#pragma unroll
            for (int w = 0; w < WB; ++w) cw[c][blk * WB + w] = *at_bytes(b.c, 4u * (t * ROWW + blk * PB + kb * WB + w));
#pragma unroll
        for (int w = 0; w < SW; ++w) sc[c][w] = *at_bytes(b.s, 4u * (t * SW + w));
    }
};

// Block-format scores: per block one v_mfma_i32_16x16x32_i8 with rows
// (query, digit) as in the bit-plane scores (the query as four balanced 7-bit
// digits of a fixed-point value) and the raw codes as B: 8-bit codes as they
// are, 4-bit codes as their low and high nibbles (q + 8, the offset removed
// with a per-query block constant).  Each block's exact integer sum is scaled
// by the key's block scale.
template <int QB, int D, int MT>
struct ScoreQ {
    using KW = KeyWordsQ<QB, D>;
    static constexpr int NQ = MT;
    static constexpr int TAB_BYTES = 0;
    static constexpr bool OCC3 = false;     // three workgroups measured no faster
    static constexpr int NB = D / 32;
    int64_t aop[MT][NB];
    float fq[MT];              // 2^-f * softmax scale * log2(e)
    float kq[MT][NB];          // 4-bit codes: 8 sum_block x (integer units of the block sums)

    __device__ static int query(int slot, int kb) { return 4 * slot + kb; }

    __device__ static float for_query(const float (&v)[MT], int q, int j)
    {
        float r = 1.0f;
#pragma unroll
        for (int s = 0; s < MT; ++s) {
            const float t = __shfl(v[s], 16 * (q % 4) + j);
            if (q / 4 == s) r = t;
        }
        return r;
    }

    __device__ void init(const DecodeLaunch &a, int unit, int64_t row0, int lane, int kb, int GC, float, unsigned char *)
    {
        const int64_t *src = reinterpret_cast<const int64_t *>(a.mf.aops) + static_cast<int64_t>(unit) * MT * NB * 64;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int b = 0; b < NB; ++b) aop[mt][b] = src[(mt * NB + b) * 64 + lane];
        const float f = a.mf.lscale;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int g = 4 * mt + kb;
            const bool ok = g < GC;
            const int64_t r = row0 + (ok ? g : 0);
            const float4 sc = *reinterpret_cast<const float4 *>(a.mf.qscal + r * 4);
            fq[mt] = ok ? sc.x * f : 0.0f;
            if constexpr (QB == 4) {
                float kv[NB];
#pragma unroll
                for (int b = 0; b < NB; ++b) kv[b] = a.qaux[r * NB + b];
#pragma unroll
                for (int b = 0; b < NB; ++b) kq[mt][b] = ok ? kv[b] : 0.0f;
            } else {
#pragma unroll
                for (int b = 0; b < NB; ++b) kq[mt][b] = 0.0f;
            }
        }
    }

    __device__ void scores(const KW &kw, float (&sc)[2][MT]) const
    {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            float s[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) s[mt] = 0.0f;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                int64_t bop;
                if constexpr (QB == 8) {
                    bop = static_cast<int64_t>(kw.cw[c][2 * b]) | (static_cast<int64_t>(kw.cw[c][2 * b + 1]) << 32);
                } else {
                    const uint32_t x = kw.cw[c][b];
                    bop = static_cast<int64_t>(x & 0x0F0F0F0Fu) | (static_cast<int64_t>((x >> 4) & 0x0F0F0F0Fu) << 32);
                }
                const float scl = f16_bits_to_f32((kw.sc[c][b / 2] >> (16 * (b % 2))) & 0xffffu);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const v4i acc = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop[mt][b], bop, v4i{0, 0, 0, 0}, 0, 0, 0);
                    float val = limbs_to_float(acc);
                    if constexpr (QB == 4) val -= kq[mt][b];
                    s[mt] = fmaf(scl, val, s[mt]);
                }
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) sc[c][mt] = s[mt] * fq[mt];
        }
    }
};

// Workgroups per CU the register budget is fitted to: one at d = 256, two for
// the spread-operand table scores there (SP: keys prefetched one tile ahead,
// values loaded with their own tile); three for the table scores (OCC3) at
// d = 128, with a two-deep prefetch ring; otherwise two, with a three-deep
// ring.
template <class SCORE, int D, bool TWO, bool SP = false>
constexpr int attend_occupancy()
{
    return D == 256 ? (SP ? 2 : 1) : SCORE::OCC3 ? 3 : 2;
}

// SP (table scores, at most two query heads per unit, at least four value
// groups): the value-product A operand of the unit's queries is built with its
// (query, group) pairs spread over the four lanes that share a token pair
// (lane kb takes groups kb, kb + 4, ...), instead of each lane building all
// groups for its own two query slots, three of whose four lanes would hold
// only absent queries.
// SO: scores only (tq_scores): the same tiles and score products, the raw
// scores written to a.scores [B, Hq, T]; no value loads, softmax or merge.
template <class SCORE, int BITS, int D, int VBITS, bool TWO, bool SP = false, bool SO = false>
__global__ __launch_bounds__(kThreads, (attend_occupancy<SCORE, D, TWO, SP>())) void k_attend(DecodeLaunch a, float kappa, int64_t chunk)
{
    constexpr int NQ = SCORE::NQ;
    constexpr int TK = 32;                       // keys per wave tile
    constexpr int VB = D * VBITS / 8;            // value code bytes per token
    constexpr int VSTR = VB + 16;                // LDS row stride (odd multiple of 16 B)
    constexpr int NCB = VB / 16;                 // 16-byte column blocks of a value row
    constexpr int NF = 8 / VBITS;                // code fields per byte
    constexpr int NTILE = NCB * NF;              // 16-channel tiles of the value product
    constexpr bool kTwoGroups = TWO;             // a 16-channel tile spans two value groups (2-bit values, group 32)
    constexpr int VCL = TK * VB / 16 / 64;       // 16-byte value chunks per lane per tile
    constexpr int NGM = D / 32;                  // most value groups per row (group >= 32)
    constexpr int PD = TK * NGM / 64;            // (scale, zero) dwords per lane per tile
    constexpr int VT_BYTES = TK * VSTR;
    // value-product A operand per group: 64 lanes x 16 B; in SP mode only the
    // 16 lanes of rows 0-3 (queries 0 and 1, hi and lo) are stored, at a
    // stride of 68 dwords (a bank skew between the groups the four row blocks
    // write together), followed by 16 zero bytes the other lanes read
    constexpr int AF_GSTRIDE = SP ? 68 : 256;     // dwords per group
    constexpr int AF_BYTES = NGM * AF_GSTRIDE * 4 + (SP ? 16 : 0);
    constexpr int PS_BYTES = TK * NGM * 4;
    constexpr int WAVE_BYTES = VT_BYTES + AF_BYTES + PS_BYTES;
    constexpr int MG = SP ? 2 : kMaxG;            // query rows of the merge area (SP: at most two)
    constexpr int MERGE_BYTES = 4 * MG * D * 4;
    constexpr int SMEM = (4 * WAVE_BYTES > MERGE_BYTES) ? 4 * WAVE_BYTES : MERGE_BYTES;

    __shared__ __align__(16) unsigned char smem[SMEM];
    __shared__ __align__(16) unsigned char stab[SCORE::TAB_BYTES > 0 ? SCORE::TAB_BYTES : 16];
    __shared__ float s_wm[4][kMaxG], s_wl[4][kMaxG];
    __shared__ float s_wz[4][kMaxG][kMaxNG];
    __shared__ int32_t s_blk[kStageBlocks];       // block ids of this split (paged caches)

    const int tid = threadIdx.x, lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);   // wave-uniform: tile bases stay scalar
    const int GC = a.mf.gc, nqc = a.mf.nqc;
    const int NG = D / a.group;                  // 1, 2, 4 or 8
    const int lg_ng = __builtin_ctz(NG);
    const int unit = blockIdx.y, split = blockIdx.x;
    const int64_t bh = unit / nqc;
    const int64_t seq = bh / a.Hkv, kvh = bh - seq * a.Hkv;
    const int64_t row0 = unit_row0(a, unit);
    const int64_t t_begin = static_cast<int64_t>(split) * chunk;
    const int64_t len = seq_len_of(a.map, a.T, seq);        // T, or the sequence's length
    const int64_t t_end = t_begin + chunk < len ? t_begin + chunk : len;
    const int j = lane % 16, kb = lane / 16;

    unsigned char *vt = smem + wave * WAVE_BYTES;
    uint32_t *afr = reinterpret_cast<uint32_t *>(vt + VT_BYTES);              // [NGM][64 lanes][4]
    uint32_t *pst = reinterpret_cast<uint32_t *>(vt + VT_BYTES + AF_BYTES);   // [TK][NGM]

    SCORE score;
    score.init(a, unit, row0, lane, kb, GC, kappa, stab);
    // value-product A rows of absent queries stay zero
    for (int i = lane; i < AF_BYTES / 4; i += 64) afr[i] = 0u;
    // Rows of the split's tiles, one formula for every cache: token t of the
    // unit lives at row (blk * Hkv + kvh) * rstride + (t & rmask) with blk =
    // s_blk[(t >> rshift) - blk0].  Flat and contiguous caches: one "block" per
    // sequence (blk = seq, rstride = T).  Paged: the split's block ids, staged
    // in LDS once (the host keeps a split within kStageBlocks blocks), ids
    // outside the pool as -1.  A tile's row costs an LDS read, no branch.
    const bool paged = a.map.mode == CacheMap::kPaged;
    const int rshift = paged ? __builtin_ctz(a.map.bs) : 31;       // t < 2^31
    const uint32_t rmask = paged ? static_cast<uint32_t>(a.map.bs - 1) : 0x7fffffffu;
    const int64_t rstride = paged ? a.map.bs : a.T;
    const int blk0 = static_cast<int>(t_begin >> rshift);
    if (paged) {
        const int nblk = t_end > t_begin ? static_cast<int>((t_end - 1) >> rshift) - blk0 + 1 : 0;
        for (int i = tid; i < nblk && i < kStageBlocks; i += kThreads) {
            const int32_t id = a.map.bt[seq * a.map.maxb + blk0 + i];
            s_blk[i] = (id >= 0 && id < a.map.nblocks) ? id : -1;
        }
    } else if (tid == 0) {
        s_blk[0] = static_cast<int32_t>(seq);
    }
    __syncthreads();        // block ids (and score tables), written by all threads

    static_assert(!SP || (SCORE::TAB_BYTES > 0 && NGM >= 4), "spread A operand: table scores, >= 4 value groups");
    constexpr int NSP = SP ? NGM / 4 : 1;         // groups per lane in the spread A operand
    float m_run[NQ], l_run[NQ];
    float zacc[NQ][NGM];
    float zsp[2][NSP];                            // spread mode: zero-point sums of queries 0, 1
#pragma unroll
    for (int i = 0; i < NSP; ++i) zsp[0][i] = zsp[1][i] = 0.0f;
#pragma unroll
    for (int sl = 0; sl < NQ; ++sl) {
        m_run[sl] = -INFINITY;
        l_run[sl] = 0.0f;
#pragma unroll
        for (int gg = 0; gg < NGM; ++gg) zacc[sl][gg] = 0.0f;
    }
    // value-product accumulators, rows (query 2 kb + r / 2, fp16 part r % 2),
    // column j = byte column 16 cb + j, field f; acc1 for tiles whose second
    // half of columns lies in the next value group
    v4f acc0[NTILE], acc1[kTwoGroups ? NTILE : 1];
#pragma unroll
    for (int nt = 0; nt < NTILE; ++nt) acc0[nt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int nt = 0; nt < (kTwoGroups ? NTILE : 1); ++nt) acc1[nt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // A-operand slots of the value product are swizzled (slot of lane L is
    // L ^ ((L >> 4) & 3)) so that the writes of one row block spread over all
    // banks; this lane's write offsets (rows 2 q, 2 q + 1 of its query slots)
    // and read offset are fixed.
    auto aslot = [](int L) { return L ^ ((L >> 4) & 3); };
    int awr[NQ][2];
#pragma unroll
    for (int sl = 0; sl < NQ; ++sl)
#pragma unroll
        for (int part = 0; part < 2; ++part)
            awr[sl][part] = aslot(2 * SCORE::query(sl, kb) + part + 16 * (j / 4)) * 4 + (j % 4);
    // A-operand read of this lane: its row's slot, or (SP, rows 4-15) the zero block
    const bool a_live = !SP || (lane % 16) < 4;
    const uint32_t *abase = SP ? (a_live ? afr + (4 * (lane / 16) + lane % 16) * 4 : afr + NGM * AF_GSTRIDE)
                               : afr + aslot(lane) * 4;
    const int agstep = a_live ? AF_GSTRIDE : 0;
    int awq[2][2];                                // spread mode: slots of queries 0 and 1
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int part = 0; part < 2; ++part)
            awq[q][part] = SP ? (4 * (j / 4) + 2 * q + part) * 4 + (j % 4)
                              : aslot(2 * q + part + 16 * (j / 4)) * 4 + (j % 4);
    // tr-read row of this lane in every value block: k-slot 8 kb + e holds the
    // token of slot order; lanes 2r, 2r + 1 address read row r, and row r lands
    // in half e(r) of the operand with e = {0, 2, 1, 3, 4, 6, 5, 7}
    const int rr = j / 2;
    const int e_of_r = (rr & 4) | ((rr & 1) << 1) | ((rr >> 1) & 1);
    const unsigned char *tr_base = vt + slot_token(8 * kb + e_of_r) * VSTR + 8 * (j % 2);

    struct Prefetch {
        int nvalid;             // keys of the tile (0: a block id outside the pool)
        typename SCORE::KW kw;
        v4i vcode[VCL];
        uint32_t par[PD];
    };
    const int64_t first = t_begin + TK * wave;
    // Loads of one tile, all unconditional: rows past the valid range are
    // clamped to the last valid row and masked where they are used; a tile
    // past the end reloads the wave's first tile.
    // wave-uniform first row and valid keys of the tile starting at tile0: a
    // tile never straddles a block (tiles start at multiples of 32 tokens,
    // blocks hold a multiple of 32); nv = 0 for a block id outside the pool
    // (the clamp only guards LDS: the host keeps every split within kStageBlocks blocks)
    // (flat and contiguous caches skip the LDS read: their one block is the sequence)
    auto tile_rows = [&](int64_t tile0, int64_t &n0, int &nv) {
        const int64_t tc = tile0 < t_end ? tile0 : first;
        nv = static_cast<int>(t_end - tc < TK ? t_end - tc : TK);
        const int bi = min(static_cast<int>(tc >> rshift) - blk0, kStageBlocks - 1);
        const int blk = paged ? __builtin_amdgcn_readfirstlane(s_blk[bi]) : static_cast<int>(seq);
        n0 = blk >= 0 ? (static_cast<int64_t>(blk) * a.Hkv + kvh) * rstride + (static_cast<uint32_t>(tc) & rmask) : 0;
        if (blk < 0) nv = 0;
    };
    auto fetch_keys = [&](int64_t tile0, Prefetch &pf) {
        int64_t n0;
        int nvv;
        tile_rows(tile0, n0, nvv);
        const int nv = nvv > 0 ? nvv : 1;      // loads stay in the tile's first row
        pf.nvalid = nvv;
        const auto kbase = SCORE::KW::bases(a, n0);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const uint32_t t = static_cast<uint32_t>(16 * c + j < nv ? 16 * c + j : nv - 1);
            pf.kw.load(kbase, t, kb, c);
        }
    };
    auto fetch_vals = [&](int64_t tile0, Prefetch &pf) {
        int64_t n0;
        int nvv;
        tile_rows(tile0, n0, nvv);
        const int nv = nvv > 0 ? nvv : 1;
        if constexpr (!SO) {
            const v4i *vsrc = reinterpret_cast<const v4i *>(a.vc.codes + n0 * VB);
#pragma unroll
            for (int v = 0; v < VCL; ++v) {
                const uint32_t i = static_cast<uint32_t>(lane + 64 * v);
                const uint32_t tok = i / (VB / 16);
                pf.vcode[v] = ld_stream(at_bytes(vsrc, 16u * ((tok < static_cast<uint32_t>(nv) ? tok : nv - 1) * (VB / 16) + i % (VB / 16))));
            }
            const uint32_t *psrc = reinterpret_cast<const uint32_t *>(a.vc.params) + n0 * NG;
            const uint32_t plim = static_cast<uint32_t>(nv * NG - 1);
#pragma unroll
            for (int k = 0; k < PD; ++k) {
                const uint32_t idx = static_cast<uint32_t>(lane + 64 * k);
                pf.par[k] = ld_stream(at_bytes(psrc, 4u * (idx < plim ? idx : plim)));
            }
        }
    };
    auto fetch = [&](int64_t tile0, Prefetch &pf) {
        fetch_keys(tile0, pf);
        fetch_vals(tile0, pf);
    };

    // staging of the tile's value codes and (scale, zero) words in this wave's LDS
    auto stage_values = [&](const Prefetch &vals, int nv) {
        wave_sync();        // the previous tile's LDS reads come before these writes
#pragma unroll
        for (int v = 0; v < VCL; ++v) {
            const int i = lane + 64 * v;
            *reinterpret_cast<v4i *>(vt + (i / (VB / 16)) * VSTR + (i % (VB / 16)) * 16) = vals.vcode[v];
        }
#pragma unroll
        for (int k = 0; k < PD; ++k) {
            const int idx = lane + 64 * k;
            if (idx < TK * NG) pst[(idx >> lg_ng) * NGM + (idx & (NG - 1))] = idx < nv * NG ? vals.par[k] : 0u;
        }
        wave_sync();        // staged rows are read by other lanes below
    };

    // cur: the tile's key words; vals: its value words (the same buffer,
    // except in SP mode, where the value words are staged after the scores and
    // the buffer then takes the loads of the tile at next_vals)
    auto compute = [&](int64_t tile0, const Prefetch &cur, Prefetch &vals, int64_t next_vals = -1) {
        (void)tile0;
        const int nv = cur.nvalid;
        if constexpr (SO) {
            // raw scores (the host sets the folded score factor to 1)
            float sc[2][NQ];
            score.scores(cur.kw, sc);
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int sl = 0; sl < NQ; ++sl) {
                    const int q = SCORE::query(sl, kb);
                    if (16 * c + j < nv && q < GC) a.scores[(row0 + q) * a.T + tile0 + 16 * c + j] = sc[c][sl];
                }
            return;
        }
        // ---- value codes and (scale, zero) words of the tile into this wave's LDS
        if constexpr (!SP) stage_values(vals, nv);

        // ---- scores of keys j and 16 + j for this lane's queries
        float lamv[NQ][2];
        {
            float sc[2][NQ];
            score.scores(cur.kw, sc);
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const bool valid = 16 * c + j < nv;
#pragma unroll
                for (int sl = 0; sl < NQ; ++sl)
                    lamv[sl][c] = (valid && SCORE::query(sl, kb) < GC) ? sc[c][sl] : -INFINITY;
            }
        }

        // ---- online softmax (per query, over the 16 lanes of its row block)
        bool grow = false;
        float m_new[NQ];
#pragma unroll
        for (int sl = 0; sl < NQ; ++sl) {
            m_new[sl] = fmaxf(m_run[sl], row16_max(fmaxf(lamv[sl][0], lamv[sl][1])));
            grow |= m_new[sl] > m_run[sl];
        }
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
            // the running maximum moved: rescale this wave's sums and accumulators
            float alpha[NQ];
#pragma unroll
            for (int sl = 0; sl < NQ; ++sl) {
                alpha[sl] = (m_new[sl] > m_run[sl]) ? exp2_fast(m_run[sl] - m_new[sl]) : 1.0f;
                l_run[sl] *= alpha[sl];
#pragma unroll
                for (int gg = 0; gg < NGM; ++gg) zacc[sl][gg] *= alpha[sl];
                m_run[sl] = m_new[sl];
            }
            if constexpr (SP) {
                // queries 0 and 1, from the lanes that score them
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const float aq = __shfl(alpha[SCORE::slot_of(q)], SCORE::lane_of(q, j));
#pragma unroll
                    for (int i = 0; i < NSP; ++i) zsp[q][i] *= aq;
                }
            }
            // value rows of this lane: queries 2 kb and 2 kb + 1
            const float a0 = SCORE::for_query(alpha, 2 * kb, j), a1 = SCORE::for_query(alpha, 2 * kb + 1, j);
            const v4f av = {a0, a0, a1, a1};
#pragma unroll
            for (int nt = 0; nt < NTILE; ++nt) acc0[nt] = acc0[nt] * av;
            if constexpr (kTwoGroups) {
#pragma unroll
                for (int nt = 0; nt < NTILE; ++nt) acc1[nt] = acc1[nt] * av;
            }
        }
        float p[NQ][2];
#pragma unroll
        for (int sl = 0; sl < NQ; ++sl) {
            const float mref = m_run[sl] == -INFINITY ? 0.0f : m_run[sl];
            p[sl][0] = exp2_fast(lamv[sl][0] - mref);
            p[sl][1] = exp2_fast(lamv[sl][1] - mref);
            l_run[sl] += p[sl][0] + p[sl][1];
        }

        // (SP: the tile's value words are staged now, after the scores, and
        // the next tile's value loads go out at once)
        if constexpr (SP) {
            stage_values(vals, nv);
            if (next_vals >= 0) fetch_vals(next_vals, vals);
        }

        // ---- value-product A operand: p * scale as fp16 hi + lo in rows 2 q and
        // 2 q + 1, tokens j and 16 + j packed in dword j % 4 of k-block j / 4
        if constexpr (SP) {
            float pq[2][2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                pq[q][0] = __shfl(p[SCORE::slot_of(q)][0], SCORE::lane_of(q, j));
                pq[q][1] = __shfl(p[SCORE::slot_of(q)][1], SCORE::lane_of(q, j));
            }
#pragma unroll
            for (int i = 0; i < NSP; ++i) {
                const int gg = 4 * i + kb;
                if (gg < NG) {
                    const uint32_t r0 = pst[j * NGM + gg], r1 = pst[(16 + j) * NGM + gg];
                    const float s0 = f16_bits_to_f32(r0 & 0xffffu), s1 = f16_bits_to_f32(r1 & 0xffffu);
                    const float z0 = f16_bits_to_f32(r0 >> 16), z1 = f16_bits_to_f32(r1 >> 16);
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        const float w0 = pq[q][0] * s0, w1 = pq[q][1] * s1;
                        zsp[q][i] = fmaf(pq[q][0], z0, fmaf(pq[q][1], z1, zsp[q][i]));
                        const auto hi = __builtin_amdgcn_cvt_pkrtz(w0, w1);
                        const auto lo = __builtin_amdgcn_cvt_pkrtz(w0 - static_cast<float>(hi[0]), w1 - static_cast<float>(hi[1]));
                        afr[gg * AF_GSTRIDE + awq[q][0]] = __builtin_bit_cast(uint32_t, hi);
                        afr[gg * AF_GSTRIDE + awq[q][1]] = __builtin_bit_cast(uint32_t, lo);
                    }
                }
            }
        } else {
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
        for (int sl = 0; sl < NQ; ++sl) {
#pragma unroll
            for (int gg = 0; gg < NGM; ++gg) {
                if (gg < NG) {
                    const float w0 = p[sl][0] * f16_bits_to_f32(pr[0][gg] & 0xffffu);
                    const float w1 = p[sl][1] * f16_bits_to_f32(pr[1][gg] & 0xffffu);
                    zacc[sl][gg] = fmaf(p[sl][0], f16_bits_to_f32(pr[0][gg] >> 16),
                                        fmaf(p[sl][1], f16_bits_to_f32(pr[1][gg] >> 16), zacc[sl][gg]));
                    const auto hi = __builtin_amdgcn_cvt_pkrtz(w0, w1);
                    const auto lo = __builtin_amdgcn_cvt_pkrtz(w0 - static_cast<float>(hi[0]), w1 - static_cast<float>(hi[1]));
                    afr[gg * 256 + awr[sl][0]] = __builtin_bit_cast(uint32_t, hi);
                    afr[gg * 256 + awr[sl][1]] = __builtin_bit_cast(uint32_t, lo);
                }
            }
        }
        }

        wave_sync();        // the A operand is read by other lanes below
        // ---- value product over the 32 tokens, all channel tiles
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const int g_lo = (NF * 16 * cb) >> (__builtin_ctz(a.group));
            const v8h af0 = __builtin_bit_cast(v8h, *reinterpret_cast<const v4i *>(abase + g_lo * agstep));
            v8h af1 = af0;
            if constexpr (kTwoGroups)
                af1 = __builtin_bit_cast(v8h, *reinterpret_cast<const v4i *>(abase + (g_lo + 1) * agstep));
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
                if constexpr (kTwoGroups) acc1[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af1, bv, acc1[nt], 0, 0, 0);
            }
        }
    };

    // Register ring of prefetched tiles: the loads of each tile are issued
    // DEPTH - 1 tiles ahead of its use, so that a wave keeps that many tiles
    // of HBM reads in flight behind its compute (two buffers at one or three
    // workgroups per CU, three at two).  Tiles left after the unrolled trips
    // are computed from the buffers that already hold them.
    constexpr int STEP = 4 * TK;
    constexpr bool kRing2 = attend_occupancy<SCORE, D, TWO, SP>() != 2;
    if (first < t_end) {
        if constexpr (SP) {
            // two workgroups per CU: the key words one tile ahead; the value
            // words of the next tile go out once the current tile's are staged
            // (half a tile ahead: they are needed only after the scores)
            Prefetch ka, kc, va;
            fetch_keys(first, ka);
            fetch_vals(first, va);
            int64_t t = first;
            for (; t + STEP < t_end; t += 2 * STEP) {
                fetch_keys(t + STEP, kc);
                compute(t, ka, va, t + STEP);
                fetch_keys(t + 2 * STEP, ka);
                compute(t + STEP, kc, va, t + 2 * STEP < t_end ? t + 2 * STEP : -1);
            }
            if (t < t_end) compute(t, ka, va);
        } else if constexpr (kRing2) {
            Prefetch pa, pb;
            fetch(first, pa);
            int64_t t = first;
            for (; t + STEP < t_end; t += 2 * STEP) {
                fetch(t + STEP, pb);
                compute(t, pa, pa);
                fetch(t + 2 * STEP, pa);
                compute(t + STEP, pb, pb);
            }
            if (t < t_end) compute(t, pa, pa);
        } else {
            Prefetch p0, p1, p2;
            fetch(first, p0);
            fetch(first + STEP, p1);
            int64_t t = first;
            for (; t + 2 * STEP < t_end; t += 3 * STEP) {
                fetch(t + 2 * STEP, p2);
                compute(t, p0, p0);
                fetch(t + 3 * STEP, p0);
                compute(t + STEP, p1, p1);
                fetch(t + 4 * STEP, p1);
                compute(t + 2 * STEP, p2, p2);
            }
            if (t < t_end) compute(t, p0, p0);
            if (t + STEP < t_end) compute(t + STEP, p1, p1);
        }
    }

    if constexpr (SO) return;
    // ---- merge the four waves: m, l, zero-point sums and value sums per query
#pragma unroll
    for (int sl = 0; sl < NQ; ++sl) {
        const int g = SCORE::query(sl, kb);
        const float l = row16_sum(l_run[sl]);
        if (j == 0) {
            s_wm[wave][g] = m_run[sl];
            s_wl[wave][g] = l;
        }
        if constexpr (!SP) {
#pragma unroll
            for (int gg = 0; gg < NGM; ++gg) {
                const float z = row16_sum(zacc[sl][gg]);
                if (j == 0) s_wz[wave][g][gg] = z;
            }
        }
    }
    if constexpr (SP) {
        // group 4 i + kb of queries 0 and 1 is summed over the 16 lanes of row kb
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int i = 0; i < NSP; ++i) {
                const float z = row16_sum(zsp[q][i]);
                if (j == 0) s_wz[wave][q][4 * i + kb] = z;
            }
    }
    __syncthreads();        // every wave is done with its tile buffers
    float *wo = reinterpret_cast<float *>(smem);      // [4 waves][MG][D]
#pragma unroll
    for (int nt = 0; nt < NTILE; ++nt) {
        const int cb = nt / NF, f = nt % NF;
        const int ch = NF * (16 * cb + j) + f;
        const int g_lo = (NF * 16 * cb) / a.group;
        v4f acc = acc0[nt];
        if constexpr (kTwoGroups) {
            const v4f alt = acc1[nt];
            if (ch / a.group != g_lo) acc = alt;
        }
        const float sc = 16777216.0f / static_cast<float>(1 << (VBITS * f));
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
            const int g = 2 * kb + qq;
            if (MG == kMaxG || g < MG) wo[(wave * MG + g) * D + ch] = sc * (acc[2 * qq] + acc[2 * qq + 1]);
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
            const float e = (s_wm[w][g] == -INFINITY) ? 0.0f : exp2_fast(s_wm[w][g] - mx);
            l = fmaf(e, s_wl[w][g], l);
            o = fmaf(e, wo[(w * MG + g) * D + ch] + s_wz[w][g][grp], o);
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
// out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s with M the largest
// split maximum (maxima in log2 units).  Beyond 16 splits: one workgroup per
// (query row, block of CH channels); thread (channel c, phase ph) takes splits
// ph, ph + P, ... (P = 256 / CH) in batches of NB, every load of a batch
// unconditional (indices clamped, weights zeroed), and the first batch is
// issued before the maxima are reduced.

__device__ __forceinline__ void ml_combine(float &m, float &l, float m2, float l2)
{
    const float mn = fmaxf(m, m2);
    if (mn == -INFINITY) return;                 // both empty
    l = l * exp2_fast(m - mn) + l2 * exp2_fast(m2 - mn);
    m = mn;
}

// Up to NS <= 16 splits: one workgroup of D threads per query row, thread c
// loads channel c of every split's partial and every (m, l) pair at once
// (indices clamped, weights zeroed past S) and combines them with no
// barrier: out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s.
template <int D, int NS>
__global__ __launch_bounds__(D) void k_merge_rows(DecodeLaunch a)
{
    const int64_t row = blockIdx.x;
    const int S = a.splits, c = threadIdx.x;
    const float2 *ml = reinterpret_cast<const float2 *>(a.part_ml + row * S * 2);
    const float *pa = a.part_acc + row * S * D + c;
    float2 m2[NS];
    float v[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int sc = s < S ? s : S - 1;
        m2[s] = ml[sc];
        v[s] = pa[static_cast<int64_t>(sc) * D];
    }
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < NS; ++s)
        if (s < S && m2[s].y > 0.0f) M = fmaxf(M, m2[s].x);
    float L = 0.0f, o = 0.0f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const float e = (s < S && m2[s].y > 0.0f) ? exp2_fast(m2[s].x - M) : 0.0f;
        L = fmaf(e, m2[s].y, L);
        o = fmaf(e, v[s], o);
    }
    a.out[row * D + c] = L > 0.0f ? o / L : 0.0f;
}

// Up to P * NB splits (P = kThreads / CH phases, NB splits each): one
// workgroup per (query row, CH channels) holds every partial after one round
// of loads.  The maximum needs no exchange of (m, l) pairs: each thread takes
// the maximum of its own splits, the two phases of a wave meet in one lane
// swap and the four waves in LDS; then each thread weights its own splits,
// and the phases' sums of weighted values and of weights meet in LDS.
template <int CH, int NB>
__global__ __launch_bounds__(kThreads) void k_merge_batch(DecodeLaunch a)
{
    constexpr int P = kThreads / CH;
    static_assert(P == 8 && CH == 32, "two phases per wave, four waves");
    __shared__ float s_m[kThreads / 64];
    __shared__ float s_o[P][CH];
    __shared__ float s_l[P];
    const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
    const int64_t row = blockIdx.x;
    const int S = a.splits, D = a.d;
    const int ch = tid % CH, c = blockIdx.y * CH + ch, ph = tid / CH;
    const float2 *ml = reinterpret_cast<const float2 *>(a.part_ml + row * S * 2);
    const float *pa = a.part_acc + row * S * D;
    float v[NB];
    float2 mv[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
        const int s = min(ph + P * u, S - 1);
        v[u] = pa[static_cast<int64_t>(s) * D + c];
        mv[u] = ml[s];
    }
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < NB; ++u)
        if (ph + P * u < S && mv[u].y > 0.0f) m = fmaxf(m, mv[u].x);
    m = fmaxf(m, __shfl_xor(m, 32));
    if (lane == 0) s_m[wave] = m;
    __syncthreads();
    m = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
    float o = 0.0f, l = 0.0f;
#pragma unroll
    for (int u = 0; u < NB; ++u) {
        const float e = (ph + P * u < S && mv[u].y > 0.0f) ? exp2_fast(mv[u].x - m) : 0.0f;
        o = fmaf(e, v[u], o);
        l = fmaf(e, mv[u].y, l);
    }
    s_o[ph][ch] = o;
    if (ch == 0) s_l[ph] = l;
    __syncthreads();
    if (tid < CH) {
        float O = 0.0f, L = 0.0f;
#pragma unroll
        for (int q = 0; q < P; ++q) {
            O += s_o[q][tid];
            L += s_l[q];
        }
        a.out[row * D + c] = L > 0.0f ? O / L : 0.0f;
    }
}

template <int CH, int NB>
__global__ __launch_bounds__(kThreads) void k_merge_splits(DecodeLaunch a)
{
    constexpr int P = kThreads / CH;
    __shared__ float red[2][kThreads / 64];
    __shared__ float part[kThreads];
    const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
    const int64_t row = blockIdx.x;
    const int S = a.splits, D = a.d;
    const int c = blockIdx.y * CH + tid % CH, ph = tid / CH;
    const float2 *ml = reinterpret_cast<const float2 *>(a.part_ml + row * S * 2);
    const float *pa = a.part_acc + row * S * D;
    float v[NB];
    float2 mv[NB];
    auto load_batch = [&](int s0) {
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int s = min(s0 + ph + P * u, S - 1);
            v[u] = pa[static_cast<int64_t>(s) * D + c];
            mv[u] = ml[s];
        }
    };
    load_batch(0);
    // (M, L) over all splits: per-thread online pairs, then wave and block
    float m = -INFINITY, l = 0.0f;
    for (int s = tid; s < S; s += kThreads) {
        const float2 x = ml[s];
        if (x.y > 0.0f) ml_combine(m, l, x.x, x.y);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float m2 = __shfl_xor(m, off), l2 = __shfl_xor(l, off);
        ml_combine(m, l, m2, l2);
    }
    if (lane == 0) {
        red[0][wave] = m;
        red[1][wave] = l;
    }
    __syncthreads();
    m = red[0][0];
    l = red[1][0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) ml_combine(m, l, red[0][w], red[1][w]);
    float o = 0.0f;
    for (int s0 = 0;;) {
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const bool ok = s0 + ph + P * u < S && mv[u].y > 0.0f;
            o = fmaf(ok ? exp2_fast(mv[u].x - m) : 0.0f, v[u], o);
        }
        s0 += P * NB;
        if (s0 >= S) break;
        load_batch(s0);
    }
    part[tid] = o;
    __syncthreads();
    if (tid < CH) {
#pragma unroll
        for (int p = 1; p < P; ++p) o += part[p * CH + tid];
        a.out[row * D + c] = l > 0.0f ? o / l : 0.0f;
    }
}

template <class SCORE, int BITS, int D, int VBITS, bool SP = false>
hipError_t launch_attend_t(const DecodeLaunch &a, hipStream_t stream, float kappa, int64_t chunk)
{
    const dim3 grid(static_cast<unsigned>(a.splits), static_cast<unsigned>(a.mf.units));
    void *tok;
    prof_begin("tq_attend_splitk", stream, &tok);
    // 2-bit values in groups of 32: a 16-byte column block spans two groups
    hipError_t bad = hipSuccess;
    if (VBITS == 2 && a.group == 32) {
        if constexpr (SP)
            bad = hipErrorInvalidValue;         // not dispatched: the spread mode excludes two-group value tiles
        else
            hipLaunchKernelGGL((k_attend<SCORE, BITS, D, VBITS, VBITS == 2>), grid, dim3(kThreads), 0, stream, a, kappa, chunk);
    } else {
        hipLaunchKernelGGL((k_attend<SCORE, BITS, D, VBITS, false, SP>), grid, dim3(kThreads), 0, stream, a, kappa, chunk);
    }
    prof_end(tok, stream);
    if (bad != hipSuccess) return bad;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1) return e;
    prof_begin("tq_merge_splits", stream, &tok);
    const unsigned rows = static_cast<unsigned>(static_cast<int64_t>(a.B) * a.Hq);
    const int S = a.splits;
    if (S <= 2) hipLaunchKernelGGL((k_merge_rows<D, 2>), dim3(rows), dim3(D), 0, stream, a);
    else if (S <= 4) hipLaunchKernelGGL((k_merge_rows<D, 4>), dim3(rows), dim3(D), 0, stream, a);
    else if (S <= 8) hipLaunchKernelGGL((k_merge_rows<D, 8>), dim3(rows), dim3(D), 0, stream, a);
    else if (S <= 16) hipLaunchKernelGGL((k_merge_rows<D, 16>), dim3(rows), dim3(D), 0, stream, a);
    else if (S <= 32) hipLaunchKernelGGL((k_merge_batch<32, 4>), dim3(rows, a.d / 32), dim3(kThreads), 0, stream, a);
    else if (S <= 64) hipLaunchKernelGGL((k_merge_batch<32, 8>), dim3(rows, a.d / 32), dim3(kThreads), 0, stream, a);
    else if (S <= 128) hipLaunchKernelGGL((k_merge_batch<32, 16>), dim3(rows, a.d / 32), dim3(kThreads), 0, stream, a);
    else if (S <= 256) hipLaunchKernelGGL((k_merge_batch<32, 32>), dim3(rows, a.d / 32), dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((k_merge_splits<32, 16>), dim3(rows, a.d / 32), dim3(kThreads), 0, stream, a);
    prof_end(tok, stream);
    return hipGetLastError();
}

template <class SCORE, int BITS, int D>
hipError_t launch_attend_v(const DecodeLaunch &a, hipStream_t s, float kappa, int64_t chunk)
{
    if constexpr (SCORE::TAB_BYTES > 0 && D == 256) {
        // spread operand, two workgroups per CU: 16 KB of centroid tables (32
        // copies) fit beside the smaller merge area
        using SPS = typename SCORE::template WithTable<16384>;
        if (a.mf.gc <= 2 && a.d / a.group >= 4 && !(a.vbits == 2 && a.group == 32))
            return a.vbits == 2 ? launch_attend_t<SPS, BITS, D, 2, true>(a, s, kappa, chunk)
                                : launch_attend_t<SPS, BITS, D, 4, true>(a, s, kappa, chunk);
    }
    return a.vbits == 2 ? launch_attend_t<SCORE, BITS, D, 2>(a, s, kappa, chunk)
                        : launch_attend_t<SCORE, BITS, D, 4>(a, s, kappa, chunk);
}

template <int BITS, int D, bool QJL>
hipError_t launch_attend_b(const DecodeLaunch &a, hipStream_t s, float kappa, int64_t chunk)
{
    if constexpr (BITS <= 2) {
        return a.mf.mt == 1 ? launch_attend_v<ScoreBits<BITS, D, 1, QJL>, BITS, D>(a, s, kappa, chunk)
                            : launch_attend_v<ScoreBits<BITS, D, 2, QJL>, BITS, D>(a, s, kappa, chunk);
    } else {
        if constexpr (D == 128)
            if (a.vbits == 4) return launch_attend_t<ScoreLut<BITS, D, QJL, 4096>, BITS, D, 4>(a, s, kappa, chunk);
        return launch_attend_v<ScoreLut<BITS, D, QJL>, BITS, D>(a, s, kappa, chunk);
    }
}

template <int D, bool QJL>
hipError_t launch_attend_d(const DecodeLaunch &a, hipStream_t s, float kappa, int64_t chunk)
{
    switch (a.bits) {
    case 1: return launch_attend_b<1, D, QJL>(a, s, kappa, chunk);
    case 2: return launch_attend_b<2, D, QJL>(a, s, kappa, chunk);
    case 3: return launch_attend_b<3, D, QJL>(a, s, kappa, chunk);
    case 4: return launch_attend_b<4, D, QJL>(a, s, kappa, chunk);
    case 5: return launch_attend_b<5, D, QJL>(a, s, kappa, chunk);
    case 6: return launch_attend_b<6, D, QJL>(a, s, kappa, chunk);
    case 7: return launch_attend_b<7, D, QJL>(a, s, kappa, chunk);
    }
    return hipErrorInvalidValue;
}

template <typename TIn, int D>
void launch_qprep_d(const DecodeLaunch &a, hipStream_t stream)
{
    // (part, quarter): q_rot and, with QJL rows, Sq
    const dim3 grid(static_cast<unsigned>(a.mf.units), (a.m > 0 && !a.kfmt_block) ? 8 : 4);
    switch (a.mf.gc) {
    case 1: hipLaunchKernelGGL((k_qprep<TIn, D, 1>), grid, dim3(kThreads), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((k_qprep<TIn, D, 2>), grid, dim3(kThreads), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((k_qprep<TIn, D, 4>), grid, dim3(kThreads), 0, stream, a); break;
    default: hipLaunchKernelGGL((k_qprep<TIn, D, 8>), grid, dim3(kThreads), 0, stream, a); break;
    }
}

template <typename TIn>
void launch_qprep_t(const DecodeLaunch &a, hipStream_t stream)
{
    if (a.d == 128) launch_qprep_d<TIn, 128>(a, stream);
    else launch_qprep_d<TIn, 256>(a, stream);
}

}  // namespace

bool mfma_decode_supported(int d, int bits, int G, int vbits, int group)
{
    (void)group;
    const int gc = mfma_query_chunk(G);
    return (d == 128 || d == 256) && bits >= 1 && bits <= 7 && gc >= 1 && (vbits == 2 || vbits == 4);
}

int mfma_query_chunk(int G)
{
    int gc = kMaxG;
    while (gc > 1 && (G % gc) != 0) gc >>= 1;
    return gc;
}

int mfma_row_tiles(int bits, int gc) { return bits <= 2 ? (gc + 3) / 4 : 1; }

int mfma_score_steps(int d, int bits, int m)
{
    // table scores: two code steps per 32 coordinates and one sign step,
    // the sign steps reserved whether or not the format has them
    return bits <= 2 ? 2 * code_dwords(d, bits) + (m > 0 ? 2 * sign_dwords(d) : 0) : 3 * (d / 32);
}

template <int QB, int D>
hipError_t launch_attend_q(const DecodeLaunch &a, hipStream_t s, int64_t chunk)
{
    return a.mf.mt == 1 ? launch_attend_v<ScoreQ<QB, D, 1>, QB, D>(a, s, 0.0f, chunk)
                        : launch_attend_v<ScoreQ<QB, D, 2>, QB, D>(a, s, 0.0f, chunk);
}

hipError_t launch_decode_block(const DecodeLaunch &a, hipStream_t stream)
{
    void *tok;
    prof_begin("tq_qprep", stream, &tok);
    switch (a.dtype) {
    case TQ_F32: launch_qprep_t<float>(a, stream); break;
    case TQ_BF16: launch_qprep_t<bf16_t>(a, stream); break;
    case TQ_F16: launch_qprep_t<f16_t>(a, stream); break;
    }
    prof_end(tok, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t tiles = (a.T + kMfmaTile - 1) / kMfmaTile;
    const int64_t chunk = ((tiles + a.splits - 1) / a.splits) * kMfmaTile;
    if (a.bits == 8) return a.d == 128 ? launch_attend_q<8, 128>(a, stream, chunk) : launch_attend_q<8, 256>(a, stream, chunk);
    return a.d == 128 ? launch_attend_q<4, 128>(a, stream, chunk) : launch_attend_q<4, 256>(a, stream, chunk);
}

template <class SCORE, int BITS, int D>
hipError_t launch_scores_t(const DecodeLaunch &a, hipStream_t stream, float kappa, int64_t chunk)
{
    const dim3 grid(static_cast<unsigned>(a.splits), static_cast<unsigned>(a.mf.units));
    void *tok;
    prof_begin("tq_scores_mfma", stream, &tok);
    hipLaunchKernelGGL((k_attend<SCORE, BITS, D, 4, false, false, true>), grid, dim3(kThreads), 0, stream, a, kappa, chunk);
    prof_end(tok, stream);
    return hipGetLastError();
}

template <int BITS, int D, bool QJL>
hipError_t launch_scores_b(const DecodeLaunch &a, hipStream_t s, float kappa, int64_t chunk)
{
    if constexpr (BITS <= 2) {
        return a.mf.mt == 1 ? launch_scores_t<ScoreBits<BITS, D, 1, QJL>, BITS, D>(a, s, kappa, chunk)
                            : launch_scores_t<ScoreBits<BITS, D, 2, QJL>, BITS, D>(a, s, kappa, chunk);
    } else {
        return launch_scores_t<ScoreLut<BITS, D, QJL>, BITS, D>(a, s, kappa, chunk);
    }
}

template <int D, bool QJL>
hipError_t launch_scores_d(const DecodeLaunch &a, hipStream_t s, float kappa, int64_t chunk)
{
    switch (a.bits) {
    case 1: return launch_scores_b<1, D, QJL>(a, s, kappa, chunk);
    case 2: return launch_scores_b<2, D, QJL>(a, s, kappa, chunk);
    case 3: return launch_scores_b<3, D, QJL>(a, s, kappa, chunk);
    case 4: return launch_scores_b<4, D, QJL>(a, s, kappa, chunk);
    case 5: return launch_scores_b<5, D, QJL>(a, s, kappa, chunk);
    case 6: return launch_scores_b<6, D, QJL>(a, s, kappa, chunk);
    case 7: return launch_scores_b<7, D, QJL>(a, s, kappa, chunk);
    }
    return hipErrorInvalidValue;
}

// q-prep of the matrix-core kernels (score operands and per-query scales)
static hipError_t qprep_mfma(const DecodeLaunch &a, hipStream_t stream)
{
    void *tok;
    prof_begin("tq_qprep", stream, &tok);
    switch (a.dtype) {
    case TQ_F32: launch_qprep_t<float>(a, stream); break;
    case TQ_BF16: launch_qprep_t<bf16_t>(a, stream); break;
    case TQ_F16: launch_qprep_t<f16_t>(a, stream); break;
    }
    prof_end(tok, stream);
    return hipGetLastError();
}

hipError_t launch_decode_mfma(const DecodeLaunch &a, hipStream_t stream)
{
    const hipError_t e = qprep_mfma(a, stream);
    if (e != hipSuccess) return e;
    const float kappa = a.m > 0 ? static_cast<float>(std::sqrt(M_PI / 2.0) / a.m) : 0.0f;
    const int64_t tiles = (a.T + kMfmaTile - 1) / kMfmaTile;
    const int64_t chunk = ((tiles + a.splits - 1) / a.splits) * kMfmaTile;
    if (a.m > 0)
        return a.d == 128 ? launch_attend_d<128, true>(a, stream, kappa, chunk)
                          : launch_attend_d<256, true>(a, stream, kappa, chunk);
    return a.d == 128 ? launch_attend_d<128, false>(a, stream, kappa, chunk)
                      : launch_attend_d<256, false>(a, stream, kappa, chunk);
}

hipError_t launch_scores_mfma(const DecodeLaunch &a, hipStream_t stream)
{
    const hipError_t e = qprep_mfma(a, stream);
    if (e != hipSuccess) return e;
    const float kappa = a.m > 0 ? static_cast<float>(std::sqrt(M_PI / 2.0) / a.m) : 0.0f;
    const int64_t tiles = (a.T + kMfmaTile - 1) / kMfmaTile;
    const int64_t chunk = ((tiles + a.splits - 1) / a.splits) * kMfmaTile;
    if (a.m > 0)
        return a.d == 128 ? launch_scores_d<128, true>(a, stream, kappa, chunk)
                          : launch_scores_d<256, true>(a, stream, kappa, chunk);
    return a.d == 128 ? launch_scores_d<128, false>(a, stream, kappa, chunk)
                      : launch_scores_d<256, false>(a, stream, kappa, chunk);
}

}  // namespace tq

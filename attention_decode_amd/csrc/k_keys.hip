// Key compression for gfx950 on the matrix cores: norm, rotation, Lloyd-Max
// codes, residual norm and QJL signs, packed into the four key planes.
// Method: discosf.com TurboQuant article, section "TurboQuant in one sentence",
// steps 1-3 (y = Pi k/||k||, nearest-centroid codes, signs of S r with
// r = y - c[idx]).
//
// One 256-thread workgroup encodes 64 keys (four 16-key tiles; 32 at d = 256,
// and in launches too small to give every CU two workgroups) and stages them
// in LDS first, in one round trip to HBM.  Both products run
// as v_mfma_f32_16x16x32_bf16 with the keys / residuals as the B operand
// (lane = key column) and the matrix as the A operand, so that every A
// fragment read from L2 serves all keys of the workgroup; the four waves split
// the output rows.
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
// Codes: idx = #{t_i < y}.  Up to 3 bits a binary search of |y| among the
// positive boundaries of the symmetric codebook, in registers (at most two
// comparisons, no LDS reads); from 4 bits a uniform grid over [t_0, t_{L-2}]
// gives a lower bound of the count that is at most two below it, and two
// exact comparisons finish it.
#include "tq_internal.h"
#include "tq_device.h"

namespace tq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
// 16-key tiles per workgroup: four (64 keys), except fp32 keys at d = 256
// (two), whose staged rows would leave room in LDS for one workgroup per CU
template <int D, typename TIn> constexpr int key_tiles() { return D >= 256 ? (sizeof(TIn) == 2 ? 4 : 2) : 4; }
// 16-key tiles whose residual operands share LDS at a time: at d = 256 with
// 2-byte inputs a workgroup takes 64 keys and runs the residual and sign steps
// in two passes of 32 (two workgroups per CU; every A fragment of Pi then
// serves 64 keys instead of 32)
template <int D, typename TIn, int KT> constexpr int key_pass_tiles() { return (D >= 256 && KT == 4) ? 2 : KT; }
template <int D, typename TIn, int KT> constexpr int key_occupancy() { return key_pass_tiles<D, TIn, KT>() < KT ? 2 : 3; }

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

// elements of 16-byte chunk c of a staged key row as fp32 (eight 16-bit
// elements, or four fp32 ones in x[0..3])
template <typename TIn, int N>
__device__ __forceinline__ void chunk_as_f32(const uint4 (&v)[N], int c, float (&x)[8])
{
    const uint32_t u[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
    if constexpr (sizeof(TIn) == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(u[i]);
#pragma unroll
        for (int i = 4; i < 8; ++i) x[i] = 0.0f;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (sizeof(TIn) == 2 && __is_same(TIn, bf16_t)) {
                x[2 * i] = bf16_to_f32(u[i] & 0xffffu);
                x[2 * i + 1] = bf16_to_f32(u[i] >> 16);
            } else {
                x[2 * i] = f16_bits_to_f32(u[i] & 0xffffu);
                x[2 * i + 1] = f16_bits_to_f32(u[i] >> 16);
            }
        }
    }
}

// eight consecutive channels of one staged key (LDS) as NT bf16 B-operand
// terms: a bf16 key is its own single term
template <typename TIn, int NT>
__device__ __forceinline__ void key_frag_lds(const unsigned char *p, uint4 (&t)[NT])
{
    if constexpr (__is_same(TIn, bf16_t)) {
        t[0] = *reinterpret_cast<const uint4 *>(p);
    } else {
        float x[8];
        if constexpr (sizeof(TIn) == 4) {
            const float4 a = reinterpret_cast<const float4 *>(p)[0];
            const float4 b = reinterpret_cast<const float4 *>(p)[1];
            x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
            x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
        } else {
            const uint4 w = *reinterpret_cast<const uint4 *>(p);
            const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[2 * i] = f16_bits_to_f32(u[i] & 0xffffu);
                x[2 * i + 1] = f16_bits_to_f32(u[i] >> 16);
            }
        }
        split_terms<NT>(x, t);
    }
}

// fp32 pair -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t bf16x2(float x0, float x1)
{
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    const bf2 v = {static_cast<__bf16>(x0), static_cast<__bf16>(x1)};
    return __builtin_bit_cast(uint32_t, v);
}

struct KeySmem {
    uint4 *rfrag;       // [KT][KS][2][64]  residual B operands (two bf16 terms)
    uint32_t *cw;       // [KEYS][D * bits / 32]  code words
    uint32_t *sw;       // [KEYS][D / 32]         sign words
    double *rho2;       // [4 waves][KEYS]
    double *nrm2;       // [256 / KEYS threads per key][KEYS]
    float *cent;        // [256]
    float *bnd;         // [256] (+inf after the last boundary)
    uint8_t *grid;      // [kMaxGrid]
};

// LDS row stride of a staged key: the row plus 16 bytes, so that the 16 keys
// one B-fragment read touches start in 16 different 4-bank groups
template <int D, typename TIn>
constexpr int key_stage_stride() { return D * static_cast<int>(sizeof(TIn)) + 16; }

// the workgroup's raw keys (step 0-1) and the residual operands (steps 3-4)
// share one region: the keys are dead before the first residual is written
template <int D, typename TIn, int KT>
constexpr size_t key_union_bytes()
{
    const size_t rfrag = sizeof(uint4) * key_pass_tiles<D, TIn, KT>() * (D / 32) * 2 * 64;
    const size_t stage = static_cast<size_t>(16 * KT) * key_stage_stride<D, TIn>();
    return rfrag > stage ? rfrag : stage;
}

template <int D, typename TIn, int BITS, int KT>
constexpr size_t key_smem_bytes()
{
    constexpr size_t keys = 16 * KT;
    return key_union_bytes<D, TIn, KT>() + sizeof(uint32_t) * keys * (D * BITS / 32 + D / 32)
           + sizeof(double) * (4 * keys + kThreads) + sizeof(float) * 512 + (BITS >= 4 ? kMaxGrid : 0);
}

template <int D, typename TIn, int BITS, int KT>
__global__ __launch_bounds__(kThreads, (key_occupancy<D, TIn, KT>())) void k_compress_keys(KeyLaunch a, int64_t n_total)
{
    constexpr int KS = D / 32;           // k-steps of 32 channels
    constexpr int RTW = D / 64;          // 16-row output tiles per wave
    constexpr int NK = KeyTerms<TIn>::n;
    constexpr int L = 1 << BITS;
    constexpr int CW = D * BITS / 32, SWN = D / 32;
    constexpr int kKT = KT;              // 16-key tiles of the workgroup
    constexpr int kKeys = 16 * kKT;      // keys of the workgroup
    constexpr int KR = key_pass_tiles<D, TIn, KT>();   // key tiles per residual / sign pass
    constexpr int TPK = kThreads / kKeys;                              // threads per staged key
    extern __shared__ __align__(16) unsigned char smem_raw[];
    __shared__ int64_t s_row[kKeys];              // plane row of each key of the workgroup
    KeySmem s;
    {
        unsigned char *p = smem_raw;
        s.rfrag = reinterpret_cast<uint4 *>(p);   p += key_union_bytes<D, TIn, KT>();
        s.rho2 = reinterpret_cast<double *>(p);   p += sizeof(double) * 4 * kKeys;
        s.nrm2 = reinterpret_cast<double *>(p);   p += sizeof(double) * kThreads;
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

    // codebook tables (L <= 128 entries, a grid of at most 4096 bytes in
    // 16-byte pieces): loads issued unconditionally (indices clamped) ahead of
    // the keys, stored to LDS after them, so both share one round trip
    const int ti = tid < L ? tid : L - 1;
    const float cent_v = a.centroids[ti];
    const float bnd_v = a.boundaries[ti];      // entry L - 1 is +inf
    uint4 grid_v = make_uint4(0u, 0u, 0u, 0u);
    if constexpr (BITS >= 4) {
        const int ng16 = a.ngrid / 16;
        grid_v = reinterpret_cast<const uint4 *>(a.grid)[tid < ng16 ? tid : ng16 - 1];
    }
    for (int i = tid; i < kKeys * CW; i += kThreads) s.cw[i] = 0u;
    for (int i = tid; i < kKeys * SWN; i += kThreads) s.sw[i] = 0u;

    // ---- 0. the workgroup's keys into LDS, one HBM round trip: thread
    // (key kk, quarter q) loads quarter q of row kk as 16-byte chunks (rows
    // found with one divide per workgroup, then stepping across sequence /
    // head boundaries) and adds the exact squares of its elements in fp64:
    // partial q of ||k||^2.  Slots past the last key reload that key (loads
    // stay unconditional); their results are never stored.
    constexpr int RSTR = key_stage_stride<D, TIn>();
    constexpr int CH16 = D * static_cast<int>(sizeof(TIn)) / 16;     // 16-byte chunks per row
    constexpr int CPT = CH16 / TPK;                                    // chunks per thread
    unsigned char *kst = reinterpret_cast<unsigned char *>(s.rfrag);
    {
        const int kk = tid / TPK, q = tid % TPK;
        const int last = static_cast<int>(n_total - 1 - n0 < kKeys - 1 ? n_total - 1 - n0 : kKeys - 1);
        const int64_t bh0 = n0 / a.T, t0 = n0 - bh0 * a.T;
        int64_t t = t0 + (kk < last ? kk : last), h = bh0 % a.H, b = bh0 / a.H;
        while (t >= a.T) {          // at most 64 / T + 1 steps
            t -= a.T;
            if (++h == a.H) {
                h = 0;
                ++b;
            }
        }
        const uint4 *src = reinterpret_cast<const uint4 *>(static_cast<const TIn *>(a.k) + b * a.sb + h * a.sh + t * a.st)
                           + q * CPT;
        uint4 v[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) v[c] = src[c];
        uint4 *dst = reinterpret_cast<uint4 *>(kst + kk * RSTR) + q * CPT;
#pragma unroll
        for (int c = 0; c < CPT; ++c) dst[c] = v[c];
        double ss = 0.0;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            float x[8];
            chunk_as_f32<TIn>(v, c, x);
#pragma unroll
            for (int e = 0; e < 16 / static_cast<int>(sizeof(TIn)); ++e)
                ss = fma(static_cast<double>(x[e]), static_cast<double>(x[e]), ss);    // exact squares
        }
        s.nrm2[q * kKeys + kk] = ss;
    }
    if (tid < L) {
        s.cent[tid] = cent_v;
        s.bnd[tid] = bnd_v;
    }
    if constexpr (BITS >= 4)
        if (tid < a.ngrid / 16) reinterpret_cast<uint4 *>(s.grid)[tid] = grid_v;
    __syncthreads();   // staged keys, cleared words, codebook tables

    // ---- 1. y = Pi k (unnormalised), this wave's rows 16 (RTW wave + j) + 4 kb + r
    const uint4 *pif = reinterpret_cast<const uint4 *>(a.pifrag);
    const uint4 *sfr = reinterpret_cast<const uint4 *>(a.sfrag);
    f32x4 acc[RTW][kKT];
#pragma unroll
    for (int j = 0; j < RTW; ++j)
#pragma unroll
        for (int kt = 0; kt < kKT; ++kt) acc[j][kt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const bool three = !a.hadamard;
    const int bits = BITS;
#pragma unroll 2
    for (int ks = 0; ks < KS; ++ks) {
        // A fragments of this k-step (the Hadamard sign matrix is one exact term)
        uint4 af[RTW][3];
#pragma unroll
        for (int j = 0; j < RTW; ++j) {
            const int rt = wave * RTW + j;
            af[j][0] = pif[((rt * KS + ks) * 3 + 0) * 64 + lane];
            if (three) {
                af[j][1] = pif[((rt * KS + ks) * 3 + 1) * 64 + lane];
                af[j][2] = pif[((rt * KS + ks) * 3 + 2) * 64 + lane];
            }
        }
        uint4 kf[kKT][NK];
#pragma unroll
        for (int kt = 0; kt < kKT; ++kt)
            key_frag_lds<TIn, NK>(kst + (16 * kt + col) * RSTR + (32 * ks + 8 * kb) * static_cast<int>(sizeof(TIn)), kf[kt]);
#pragma unroll
        for (int j = 0; j < RTW; ++j) {
#pragma unroll
            for (int pp = 0; pp < 3; ++pp) {
                if (pp > 0 && !three) continue;
#pragma unroll
                for (int kq = 0; kq < NK; ++kq) {
                    if (three && pp + kq > 2) continue;
#pragma unroll
                    for (int kt = 0; kt < kKT; ++kt) acc[j][kt] = mfma_bf16(af[j][pp], kf[kt][kq], acc[j][kt]);
                }
            }
        }
    }
    __syncthreads();   // every wave is done with the staged keys (the region takes the residuals next)
    float inv_n[kKT];
#pragma unroll
    for (int kt = 0; kt < kKT; ++kt) {
        const int key = 16 * kt + col;
        // 1/||k|| only scales y: fp32 rsqrt (about 1 ulp) moves y by ~1e-7 at most,
        // far inside the 1e-5 boundary band; the stored ||k|| is rounded from fp64
        double n2d = 0.0;
#pragma unroll
        for (int q = 0; q < TPK; ++q) n2d += s.nrm2[q * kKeys + key];
        const float n2 = static_cast<float>(n2d);
        inv_n[kt] = (n2 > 0.0f) ? a.rot_scale * __builtin_amdgcn_rsqf(n2) : 0.0f;
    }
    // 1-3 bits: the codebook is exactly symmetric (c[L-1-i] = -c[i], and so
    // the boundaries, with t[L/2-1] = 0), so |y| is placed among the H - 1
    // positive boundaries by a binary search in registers and the centroid
    // taken from the H positive ones; idx and y - c[idx] follow from the sign
    // of y, bit for bit as the full count would give them (up to exact ties)
    constexpr int H = L / 2;
    float tp[H > 1 ? H - 1 : 1], cp[H];
    if constexpr (BITS <= 3) {
#pragma unroll
        for (int i = 0; i < H - 1; ++i) tp[i] = s.bnd[H + i];
#pragma unroll
        for (int i = 0; i < H; ++i) cp[i] = s.cent[H + i];
    }

    const bool qjl = a.m > 0;
#pragma unroll
    for (int kt0 = 0; kt0 < kKT; kt0 += KR) {
    // ---- 3. codes idx = #{boundaries < y}, residual r = y - c[idx], ||r||
    // (key tiles kt0 .. kt0 + KR - 1 of this pass)
#pragma unroll
    for (int kt = kt0; kt < kt0 + KR; ++kt) {
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
                    const float ay = fabsf(y);
                    int cnt = 0;          // positive boundaries below |y|
                    float c = cp[0];
                    if constexpr (BITS == 2) {
                        const bool b0 = ay > tp[0];
                        cnt = b0 ? 1 : 0;
                        c = b0 ? cp[1] : cp[0];
                    } else if constexpr (BITS == 3) {
                        const bool b1 = ay > tp[1];
                        const bool b0 = ay > (b1 ? tp[2] : tp[0]);
                        cnt = (b1 ? 2 : 0) + (b0 ? 1 : 0);
                        const float clo = b0 ? cp[1] : cp[0], chi = b0 ? cp[3] : cp[2];
                        c = b1 ? chi : clo;
                    }
                    const bool up = y > 0.0f;
                    pos = cnt ^ (up ? H : H - 1);     // H + cnt above zero, H - 1 - cnt below (cnt < H)
                    const float dv = ay - c;
                    res[r] = up ? dv : -dv;
                } else {
                    int c = static_cast<int>((y - a.grid_lo) * a.grid_scale);
                    c = c < 0 ? 0 : (c >= a.ngrid ? a.ngrid - 1 : c);
                    pos = s.grid[c];
                    pos += (y > s.bnd[pos]) ? 1 : 0;
                    pos += (y > s.bnd[pos]) ? 1 : 0;
                    res[r] = y - s.cent[pos];
                }
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
            uint32_t *dst = reinterpret_cast<uint32_t *>(&s.rfrag[(((kt - kt0) * KS + rt / 2) * 2 + 0) * 64 + lane]);
            uint32_t *dst1 = reinterpret_cast<uint32_t *>(&s.rfrag[(((kt - kt0) * KS + rt / 2) * 2 + 1) * 64 + lane]);
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
    if (qjl) {
    f32x4 zacc[RTW][KR];
#pragma unroll
    for (int j = 0; j < RTW; ++j)
#pragma unroll
        for (int kt = 0; kt < KR; ++kt) zacc[j][kt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 2
    for (int ks = 0; ks < KS; ++ks) {
        uint4 rf[KR][2];
#pragma unroll
        for (int kt = 0; kt < KR; ++kt) {
            rf[kt][0] = s.rfrag[((kt * KS + ks) * 2 + 0) * 64 + lane];
            rf[kt][1] = s.rfrag[((kt * KS + ks) * 2 + 1) * 64 + lane];
        }
#pragma unroll
        for (int j = 0; j < RTW; ++j) {
            const int rt = wave * RTW + j;
            const uint4 s0 = sfr[((rt * KS + ks) * 2 + 0) * 64 + lane];
            const uint4 s1 = sfr[((rt * KS + ks) * 2 + 1) * 64 + lane];
#pragma unroll
            for (int kt = 0; kt < KR; ++kt) {
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
        for (int kt = 0; kt < KR; ++kt) {
            uint32_t nib = 0;
#pragma unroll
            for (int r = 0; r < 4; ++r) nib |= (zacc[j][kt][r] >= 0.0f ? 1u : 0u) << r;
            atomicOr(&s.sw[(16 * (kt0 + kt) + col) * SWN + (off >> 5)], nib << (off & 31));
        }
    }
    __syncthreads();   // (also: this pass's residual operands are read before the next pass writes them)
    }
    }   // passes

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
        double n2 = 0.0;
#pragma unroll
        for (int q = 0; q < TPK; ++q) n2 += s.nrm2[q * kKeys + tid];
        a.out.knorm[r] = static_cast<float>(sqrt(n2));
        if (qjl) {
            const double r2 = s.rho2[tid] + s.rho2[kKeys + tid] + s.rho2[2 * kKeys + tid] + s.rho2[3 * kKeys + tid];
            a.out.rnorm[r] = static_cast<float>(sqrt(r2));
        }
    }
}

template <int D, typename TIn, int BITS, int KT>
hipError_t launch_keys_k(const KeyLaunch &a, hipStream_t stream)
{
    const int64_t n = static_cast<int64_t>(a.B) * a.H * a.T;
    constexpr size_t smem = key_smem_bytes<D, TIn, BITS, KT>();
    auto kern = k_compress_keys<D, TIn, BITS, KT>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    constexpr int keys = 16 * KT;
    const int64_t blocks = (n + keys - 1) / keys;
    void *tok;
    prof_begin("tq_compress_keys", stream, &tok);
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), smem, stream, a, n);
    prof_end(tok, stream);
    return hipGetLastError();
}

// Small launches (a few thousand keys, as in one decode step's append or a
// short cache): with 64 keys per workgroup the grid would not reach two
// workgroups per CU and each workgroup's dependent chain (staging, two
// products, the code and residual work on one wave per SIMD) sets the time;
// 32 keys per workgroup halves the per-wave work and doubles the grid.
constexpr int64_t kSmallKeyGrid = 512;

template <int D, typename TIn, int BITS>
hipError_t launch_keys_t(const KeyLaunch &a, hipStream_t stream)
{
    constexpr int KT = key_tiles<D, TIn>();
    if constexpr (KT > 2) {
        const int64_t n = static_cast<int64_t>(a.B) * a.H * a.T;
        if ((n + 16 * KT - 1) / (16 * KT) < kSmallKeyGrid) return launch_keys_k<D, TIn, BITS, 2>(a, stream);
    }
    return launch_keys_k<D, TIn, BITS, KT>(a, stream);
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

// Key compression for gfx950 on the matrix cores: norm, rotation, Lloyd-Max
// codes, residual norm and QJL signs, packed into the four key planes.
// Method: discosf.com TurboQuant article, section "TurboQuant in one sentence",
// steps 1-3 (y = Pi k/||k||, nearest-centroid codes, signs of S r with
// r = y - c[idx]).
//
// One 256-thread workgroup encodes 64 keys (four 16-key tiles; 32 for fp32
// keys at d = 256 and in launches too small to give every CU two workgroups)
// and stages them in LDS first, in one round trip to HBM.  Both products run
// as 16x16x32 MFMAs (bf16, or fp16 for the y product of 2-byte keys under a
// dense rotation) with the keys / residuals as the B operand (lane = key
// column) and the matrix as the A operand, so that every A fragment read from
// L2 serves all keys of the workgroup; the four waves split the output rows.
//
// Accuracy: the 16-bit operands are made exact or near-fp32 by splitting.
//   * y, 2-byte keys, dense Pi:  Pi 2^14 = F0 + F1 (two fp16 terms, about 22
//         significant bits) against the key times 2^ex, one exact fp16 term
//         (key_half_y).
//   * y otherwise:  Pi = P0 + P1 + P2 (three bf16 terms, about 24 significant
//         bits); an fp32 key is three terms.  The products kept are those whose
//         term ranks sum to at most 2, i.e. every product down to about 2^-24
//         of the leading one.  The Hadamard sign matrix H D is exact in one
//         term and its 1/sqrt(d) joins 1/||k||.
//   * z:  S = S0 + S1, r = R0 + R1 (16 bits each); S0 R0 + S0 R1 + S1 R0 leaves
//         an error near 2^-16 of |z| per term, far inside the resolution at
//         which a sign can legitimately flip.
// All sums accumulate in fp32 inside the MFMA.  ||k||^2 is summed in fp32
// along one fixed tree per key; ||r|| in fp32 per lane and fp64 across lanes.
//
// Codes: idx = #{t_i < y}.  Up to 2 bits a comparison of |y| with the
// positive boundary of the symmetric codebook, in registers (no LDS reads);
// from 3 bits (kCellBits) one 16-byte LDS read of the cell of
// a uniform grid over [t_0, t_{L-2}] that holds y: the count below the cell,
// the one boundary inside it and the centroids on either side, so one exact
// comparison finishes the code and picks the centroid.
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

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma_f16(const uint4 &a, const uint4 &b, const f32x4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Dense rotations of 2-byte keys run y = Pi k on fp16 operands: Pi 2^kPiHalfExp
// as two fp16 terms (22 significant bits; the bf16 form needs three terms for
// 24) against the key times a power of two 2^ex of its own, chosen so that
// 2^(kKeyHalfExp - 1) <= ||k|| 2^ex < 2^kKeyHalfExp.  A bf16 or fp16 element
// then fits fp16's 11-bit significand exactly unless it falls below fp16's
// normal range, i.e. below ||k|| 2^-27, where it is rounded on the subnormal
// grid (an error under ||k|| 2^-37).  Two products per fragment instead of
// three.
constexpr int kKeyHalfExp = 14;
template <int NP, typename TIn> constexpr bool key_half_y() { return NP == 3 && sizeof(TIn) == 2; }

// the eight 16-bit elements of a staged chunk times 2^ex, as packed fp16
// (v_cvt_pkrtz_f16_f32: exact for normal fp16 results, toward zero below)
template <typename TIn>
__device__ __forceinline__ uint4 chunk_as_f16(const uint4 &v, int ex)
{
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float x0, x1;
        if constexpr (__is_same(TIn, bf16_t)) {
            x0 = __uint_as_float(u[i] << 16);
            x1 = __uint_as_float(u[i] & 0xffff0000u);
        } else {
            x0 = f16_bits_to_f32(u[i] & 0xffffu);
            x1 = f16_bits_to_f32(u[i] >> 16);
        }
        o[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__builtin_amdgcn_ldexpf(x0, ex),
                                                                      __builtin_amdgcn_ldexpf(x1, ex)));
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
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

// x0^2 + x1^2 + acc for the bf16 pair (x0, x1) packed in u (v_dot2c_f32_bf16)
__device__ __forceinline__ float sq2_bf16(uint32_t u, float acc)
{
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    const bf2 x = __builtin_bit_cast(bf2, u);
    return __builtin_amdgcn_fdot2_f32_bf16(x, x, acc, false);
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

// r0, r1 as two bf16 terms each (hardware round to nearest even), packed in
// pairs: hi = (bf16(r0), bf16(r1)), lo = bf16 of the remainders.  The hi
// terms come back to fp32 by a byte permute of the low half and a mask of the
// high half (written as a shift, the compiler converts r0 a second time)
__device__ __forceinline__ void split_bf16x2(float r0, float r1, uint32_t &hi, uint32_t &lo)
{
    hi = bf16x2(r0, r1);
    const float h0 = __uint_as_float(__builtin_amdgcn_perm(hi, 0u, 0x05040c0cu));
    const float h1 = __uint_as_float(hi & 0xffff0000u);
    lo = bf16x2(r0 - h0, r1 - h1);
}

// LDS row strides of the code and sign words: one word past the row, an odd
// stride, so that the 16 keys of one atomicOr (lanes 0-15 of a row of the
// wave) land in 16 different banks (an even row of 8, 12 or 56 words puts
// them in 2 to 8 banks)
template <int D, int BITS> constexpr int cw_stride() { return D * BITS / 32 + 1; }
template <int D> constexpr int sw_stride() { return D / 32 + 1; }

struct KeySmem {
    uint4 *rfrag;       // [KT][KS][2][64]  residual B operands (two bf16 terms)
    uint32_t *cw;       // [KEYS][cw_stride]  code words
    uint32_t *sw;       // [KEYS][sw_stride]  sign words
    double *rho2;       // [4 waves][KEYS]
    double *nrm2;       // [256 / KEYS threads per key][KEYS]
    float *cent;        // [256]
    float *bnd;         // [256] (+inf after the last boundary)
    float4 *grid;       // [kGridLds] code cells {t, c_lo, c_hi, below}
};

// LDS row stride of a staged key: the row plus 16 bytes, so that the 16 keys
// one B-fragment read touches start in 16 different 4-bank groups
template <int D, typename TIn>
constexpr int key_stage_stride() { return D * static_cast<int>(sizeof(TIn)) + 16; }

// d = 256: the matrix compressor writes its code and sign words straight to
// the planes (each lane holds 16 consecutive coordinates of a key, two lanes
// one run of whole words), so no LDS holds them and the residual operands of
// all the workgroup's keys fit beside the staged keys: one sign product
template <int D> constexpr bool key_direct_words() { return D == 256; }

// the workgroup's raw keys (step 0-1) and the residual operands of all its
// key tiles (steps 3-4) share one region: the keys are dead before the first
// residual is written
template <int D, typename TIn, int KT>
constexpr size_t key_union_bytes()
{
    const size_t rfrag = sizeof(uint4) * KT * (D / 32) * 2 * 64;
    const size_t stage = static_cast<size_t>(16 * KT) * key_stage_stride<D, TIn>();
    return rfrag > stage ? rfrag : stage;
}

template <int D, typename TIn, int BITS, int KT>
constexpr size_t key_smem_bytes()
{
    constexpr size_t keys = 16 * KT;
    constexpr size_t words = key_direct_words<D>() ? 0 : sizeof(uint32_t) * keys * (cw_stride<D, BITS>() + sw_stride<D>());
    return key_union_bytes<D, TIn, KT>() + words + sizeof(double) * (4 * keys + kThreads) + sizeof(float) * 512
           + (BITS >= kCellBits ? sizeof(float4) * kGridLds : 0);
}


// Code idx = #{t_i < y} of one rotated coordinate and its residual y - c[idx].
// Up to 2 bits (encode_reg): |y| placed among the positive boundaries tp of
// the exactly symmetric codebook in registers, the centroid taken from the
// positive ones cp, idx and the residual fixed by the sign of y (bit for bit
// what the full count gives, up to exact ties; y = 0 takes the code just below
// zero).  From 3 bits (encode_cell, kCellBits): the cell of the uniform
// grid that holds y gives the count below it and its one boundary t, so the
// code is below + [y > t], the centroid c_lo or c_hi.
// encode_reg takes the coordinate as y = v scale (scale > 0, one per key, or
// 0 for a zero key) and the positive boundary as tv = tp / scale, so that no
// product v scale is formed for the comparisons (their rounding differs from
// y's by an ulp, far inside the 1e-5 band) and the residual is one fma.
template <int BITS>
__device__ __forceinline__ uint32_t encode_reg(float v, float scale, float tv, const float (&cp)[(1 << BITS) / 2],
                                               float &res)
{
    static_assert(BITS <= 2, "register codes: one positive boundary at most");
    constexpr uint32_t H = (1u << BITS) / 2;
    const bool up = v > 0.0f;
    float c = cp[0];
    uint32_t cnt = 0u;                  // positive boundaries below |y|
    if constexpr (BITS == 2) {
        const bool b0 = fabsf(v) > tv;
        c = b0 ? cp[1] : cp[0];
        cnt = b0 ? 1u : 0u;
    }
    res = fmaf(v, scale, up ? -c : c);  // y - c[idx]: the centroid's sign is the side of zero
    return cnt ^ (up ? H : H - 1);      // H + cnt above zero, H - 1 - cnt below (cnt < H)
}

// tp / scale for encode_reg from ||k||^2 (scale = rot_scale / ||k||), or 0 for
// a zero key (whose v are all 0)
__device__ __forceinline__ float reg_bound(float tp, float n2, float inv_rot_scale)
{
    return n2 > 0.0f ? tp * __builtin_amdgcn_sqrtf(n2) * inv_rot_scale : 0.0f;
}

__device__ __forceinline__ int encode_cell(float y, const KeySmem &s, const KeyLaunch &a, float &res)
{
    // cell index (y - lo) / w as one fma, clamped to [0, ngrid - 1] before
    // the conversion; its rounding (about 1e-5 of a cell) is inside the
    // cells' 2 % widening
    const float cf = __builtin_amdgcn_fmed3f(fmaf(y, a.grid_scale, a.grid_off), 0.0f, a.grid_max);
    const float4 e = s.grid[static_cast<int>(cf)];
    const bool up = y > e.x;
    res = y - (up ? e.z : e.y);
    return __float_as_int(e.w) + (up ? 1 : 0);
}

// The A-fragment tables of Pi and S are read through buffer loads: the
// lane's 16-byte slot is the one vector offset, the fragment's place in the
// table a scalar offset (wave-uniform), so a fragment load costs no vector
// address arithmetic and no address registers.  Records past the table's
// size read as zero.
static_assert(kGridLds <= kThreads, "one code cell per thread");
constexpr int kBufWord3 = 0x00020000;     // raw 32-bit access, no format conversion

__device__ __forceinline__ __amdgpu_buffer_rsrc_t frag_table(const void *p, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, bytes, kBufWord3);
}

__device__ __forceinline__ uint4 frag_load(__amdgpu_buffer_rsrc_t t, int lane, int frag)
{
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(t, lane * 16, frag * 1024, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// bytes of a table of A fragments for D rows x D columns with NT terms
template <int D, int NT> constexpr int frag_table_bytes() { return (D / 16) * (D / 32) * NT * 1024; }

// Rows 16 (RTW wave + j) .. + 15 of S, k-step ks, as the two bf16 A terms
template <int D>
__device__ __forceinline__ void load_s_frag(__amdgpu_buffer_rsrc_t st, int wave, int lane, int ks,
                                            uint4 (&sf)[D / 64][2])
{
    constexpr int KS = D / 32, RTW = D / 64;
#pragma unroll
    for (int j = 0; j < RTW; ++j) {
        const int rt = wave * RTW + j;
        sf[j][0] = frag_load(st, lane, (rt * KS + ks) * 2 + 0);
        sf[j][1] = frag_load(st, lane, (rt * KS + ks) * 2 + 1);
    }
}

// Row order of the compressor's fragment tables.  Wave w's row tile j, MFMA
// output row 4 kb + r (lane col + 16 kb, element r) holds coordinate
// SEGC (4 w + kb) + 4 j + r, SEGC = d / 16: each lane ends with SEGC
// consecutive coordinates of each of its keys (the host orders the rows of
// Pi and S so; at d = 64 this is the natural order).
template <int D> constexpr int seg_coords() { return D / 16; }

// z = S r for the residual operands of key tiles kt0 .. kt0 + KR - 1 (LDS,
// B-operand order) on this wave's rows of S; sign bits [z >= 0] of the
// lane's SEGC consecutive rows OR-ed into the LDS sign words, or (DIRECT,
// d = 256) paired with the next lane's 16 into one word stored to the key's
// row of the sign plane (rows: the plane row of each of the workgroup's keys,
// -1 to skip).  sf0 holds the first k-step's S fragments, loaded by the
// caller ahead of the residual work; each later k-step's fragments are in
// flight while the previous k-step's products run.  Without DIRECT, ends with
// a workgroup barrier (the pass's residual operands are read before the next
// pass writes them).
template <int D, int KR, bool DIRECT>
__device__ __forceinline__ void qjl_signs(__amdgpu_buffer_rsrc_t st, const KeySmem &s, const KeyLaunch &a,
                                          const int64_t *rows, int kt0, int wave, int lane,
                                          const uint4 (&sf0)[D / 64][2])
{
    constexpr int KS = D / 32, RTW = D / 64, SWN = D / 32, SWS = sw_stride<D>(), SEGC = seg_coords<D>();
    static_assert(!DIRECT || SEGC == 16, "direct sign words pair two lanes of 16 rows");
    const int col = lane & 15, kb = lane >> 4;
    const int qb = SEGC * (4 * wave + kb);      // first row of S this lane holds
    f32x4 zacc[RTW][KR];
#pragma unroll
    for (int j = 0; j < RTW; ++j)
#pragma unroll
        for (int kt = 0; kt < KR; ++kt) zacc[j][kt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    uint4 sf[2][RTW][2];
#pragma unroll
    for (int j = 0; j < RTW; ++j) {
        sf[0][j][0] = sf0[j][0];
        sf[0][j][1] = sf0[j][1];
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS) load_s_frag<D>(st, wave, lane, ks + 1, sf[(ks + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);     // keep the prefetch ahead of this k-step's products
        uint4 rf[KR][2];
#pragma unroll
        for (int kt = 0; kt < KR; ++kt) {
            rf[kt][0] = s.rfrag[((kt * KS + ks) * 2 + 0) * 64 + lane];
            rf[kt][1] = s.rfrag[((kt * KS + ks) * 2 + 1) * 64 + lane];
        }
#pragma unroll
        for (int j = 0; j < RTW; ++j) {
            const uint4 &s0 = sf[ks & 1][j][0], &s1 = sf[ks & 1][j][1];
#pragma unroll
            for (int kt = 0; kt < KR; ++kt) {
                zacc[j][kt] = mfma_bf16(s0, rf[kt][0], zacc[j][kt]);
                zacc[j][kt] = mfma_bf16(s0, rf[kt][1], zacc[j][kt]);
                zacc[j][kt] = mfma_bf16(s1, rf[kt][0], zacc[j][kt]);
            }
        }
    }
#pragma unroll
    for (int kt = 0; kt < KR; ++kt) {
        uint32_t bits = 0;        // bit 4 j + r: row qb + 4 j + r
#pragma unroll
        for (int j = 0; j < RTW; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) bits |= (zacc[j][kt][r] >= 0.0f ? 1u : 0u) << (4 * j + r);
        const int key = 16 * (kt0 + kt) + col;
        if constexpr (DIRECT) {
            const uint32_t other = static_cast<uint32_t>(__shfl_xor(static_cast<int>(bits), 16));
            const int64_t row = rows[key];
            if (!(kb & 1) && row >= 0)
                reinterpret_cast<uint32_t *>(a.out.signs)[row * SWN + (qb >> 5)] = bits | (other << 16);
        } else {
            atomicOr(&s.sw[key * SWS + (qb >> 5)], bits << (qb & 31));
        }
    }
    if constexpr (!DIRECT) __syncthreads();
}

// The code words of one lane's SEGC consecutive codes (seg: bit BITS e holds
// the code of coordinate qb + e), for the key at plane row `row`.
//   LDS (not DIRECT): OR-ed into the key's LDS code words at bit BITS qb.
//   DIRECT (d = 256, SEGC = 16): straight to the plane.  With BITS even the
//   lane's 16 codes are BITS / 2 whole words; with BITS odd the lanes kb, kb
//   + 1 (kb even) hold one run of BITS words, the first lane's segment ending
//   and the second's starting in the middle of word BITS / 2, so the second
//   lane's low 16 bits move to the first (one lane shuffle).
template <int D, int BITS, bool DIRECT, int NSEG>
__device__ __forceinline__ void put_code_words(const KeySmem &s, const KeyLaunch &a, const uint32_t (&seg)[NSEG + 1],
                                               int key, int64_t row, int qb, int kb)
{
    constexpr int CW = D * BITS / 32, CWS = cw_stride<D, BITS>();
    if constexpr (DIRECT) {
        static_assert(seg_coords<D>() == 16, "direct code words pair two lanes of 16 codes");
        uint32_t *plane = reinterpret_cast<uint32_t *>(a.out.codes);
        constexpr int NW = BITS / 2;
        if constexpr (BITS % 2 == 0) {
            if (row >= 0) {
                uint32_t *dst = plane + row * CW + (BITS * qb >> 5);
#pragma unroll
                for (int i = 0; i < NW; ++i) dst[i] = seg[i];
            }
        } else {
            const uint32_t other = static_cast<uint32_t>(__shfl_xor(static_cast<int>(seg[0]), 16));
            if (row >= 0) {
                uint32_t *dst = plane + row * CW + BITS * (qb >> 5);      // the pair's first word
                if (kb & 1) {
#pragma unroll
                    for (int i = 0; i < NW; ++i) dst[NW + 1 + i] = (seg[i] >> 16) | (seg[i + 1] << 16);
                } else {
#pragma unroll
                    for (int i = 0; i < NW; ++i) dst[i] = seg[i];
                    dst[NW] = (seg[NW] & 0xffffu) | (other << 16);
                }
            }
        }
    } else {
        const int bit0 = BITS * qb, w0 = bit0 >> 5, sh = bit0 & 31;
#pragma unroll
        for (int i = 0; i <= NSEG; ++i) {
            const uint32_t word = sh ? ((seg[i] << sh) | (i ? seg[i - 1] >> (32 - sh) : 0u)) : seg[i];
            if (word != 0u && w0 + i < CW) atomicOr(&s.cw[key * CWS + w0 + i], word);
        }
    }
}

// ||k||^2 of key kk from its NPN partials (fp32 values; NPN a power of two),
// each an aligned subtree of one fixed pairwise tree over the key's groups of
// eight elements, finished in that same tree, so that every tiling of the
// keys gives the same bits
template <int NPN>
__device__ __forceinline__ float key_norm2(const double *nrm2, int stride, int kk)
{
    static_assert((NPN & (NPN - 1)) == 0, "partials of a power-of-two tree");
    float p[NPN];
#pragma unroll
    for (int i = 0; i < NPN; ++i) p[i] = static_cast<float>(nrm2[i * stride + kk]);
#pragma unroll
    for (int w = 1; w < NPN; w *= 2)
#pragma unroll
        for (int i = 0; i < NPN; i += 2 * w) p[i] += p[i + w];
    return p[0];
}

// The workgroup's KEYS packed keys to the planes, each at its row s_row[key]
// (-1: skipped): the code and sign words from LDS (WORDS; otherwise already
// stored), ||k|| from NPN partials of the key_norm2 tree and ||r|| from NPR
// fp64 partial sums per key.
template <int D, int BITS, int KEYS, int NPN, int NPR, bool WORDS>
__device__ __forceinline__ void store_keys(const KeyLaunch &a, const KeySmem &s, const int64_t *s_row, bool qjl)
{
    constexpr int CW = D * BITS / 32, SWN = D / 32, CWS = cw_stride<D, BITS>(), SWS = sw_stride<D>();
    constexpr int TPK = kThreads / KEYS;            // threads per key
    const int tid = threadIdx.x, kk = tid / TPK, q = tid % TPK;
    const int64_t row = s_row[kk];
    if (row < 0) return;
    if constexpr (WORDS) {
        // the TPK threads of a key copy its words round-robin (fixed offsets
        // from one base per thread)
        {
            uint32_t *dst = reinterpret_cast<uint32_t *>(a.out.codes) + row * CW + q;
            const uint32_t *src = s.cw + kk * CWS + q;
#pragma unroll
            for (int it = 0; it < (CW + TPK - 1) / TPK; ++it)
                if (CW % TPK == 0 || q + it * TPK < CW) dst[it * TPK] = src[it * TPK];
        }
        if (qjl) {
            uint32_t *dst = reinterpret_cast<uint32_t *>(a.out.signs) + row * SWN + q;
            const uint32_t *src = s.sw + kk * SWS + q;
#pragma unroll
            for (int it = 0; it < (SWN + TPK - 1) / TPK; ++it)
                if (SWN % TPK == 0 || q + it * TPK < SWN) dst[it * TPK] = src[it * TPK];
        }
    }
    if (q == 0) {
        a.out.knorm[row] = static_cast<float>(sqrt(static_cast<double>(key_norm2<NPN>(s.nrm2, KEYS, kk))));
        if (qjl) {
            double r2 = 0.0;
#pragma unroll
            for (int p = 0; p < NPR; ++p) r2 += s.rho2[p * KEYS + kk];
            a.out.rnorm[row] = static_cast<float>(sqrt(r2));
        }
    }
}

// Rows 16 (RTW wave + j) .. + 15 of Pi, k-step ks: the first NP of the NT
// terms that each fragment of the table holds
template <int D, int NP, int NT>
__device__ __forceinline__ void load_pi_frag(__amdgpu_buffer_rsrc_t pt, int wave, int lane, int ks,
                                             uint4 (&af)[D / 64][NP])
{
    constexpr int KS = D / 32, RTW = D / 64;
#pragma unroll
    for (int j = 0; j < RTW; ++j) {
        const int rt = wave * RTW + j;
#pragma unroll
        for (int p = 0; p < NP; ++p) af[j][p] = frag_load(pt, lane, (rt * KS + ks) * NT + p);
    }
}

// NP = 3: a dense Pi as three bf16 terms (two fp16 terms for 2-byte keys,
// key_half_y); NP = 1: the Hadamard sign matrix, exact in one term
template <int D, typename TIn, int BITS, int KT, int NP>
__global__ __launch_bounds__(kThreads, (key_occupancy<D, TIn, KT>())) void k_compress_keys(KeyLaunch a, int64_t n_total)
{
    constexpr int KS = D / 32;           // k-steps of 32 channels
    constexpr int RTW = D / 64;          // 16-row output tiles per wave
    constexpr bool HALF = key_half_y<NP, TIn>();
    constexpr int NPA = HALF ? 2 : NP;   // A terms of Pi per fragment
    constexpr int NTAB = HALF ? 2 : 3;   // terms per fragment in Pi's table
    constexpr int NK = HALF ? 1 : KeyTerms<TIn>::n;
    constexpr int L = 1 << BITS;
    constexpr bool DIRECT = key_direct_words<D>();
    constexpr int CWS = DIRECT ? 0 : cw_stride<D, BITS>(), SWS = DIRECT ? 0 : sw_stride<D>();
    constexpr int kKT = KT;              // 16-key tiles of the workgroup
    constexpr int kKeys = 16 * kKT;      // keys of the workgroup
    constexpr int TPK = kThreads / kKeys;                              // threads per staged key
    constexpr int SEGC = seg_coords<D>();                              // consecutive coordinates per lane
    constexpr int NSEG = (SEGC * BITS + 31) / 32;                      // words of a lane's codes
    extern __shared__ __align__(16) unsigned char smem_raw[];
    __shared__ int64_t s_row[kKeys];              // plane row of each key of the workgroup (-1: none)
    __shared__ int s_kexp[HALF ? kKeys : 1];      // each key's staging exponent ex (fp16 y product)
    KeySmem s;
    {
        unsigned char *p = smem_raw;
        s.rfrag = reinterpret_cast<uint4 *>(p);   p += key_union_bytes<D, TIn, KT>();
        s.rho2 = reinterpret_cast<double *>(p);   p += sizeof(double) * 4 * kKeys;
        s.nrm2 = reinterpret_cast<double *>(p);   p += sizeof(double) * kThreads;
        s.cw = reinterpret_cast<uint32_t *>(p);   p += sizeof(uint32_t) * kKeys * CWS;
        s.sw = reinterpret_cast<uint32_t *>(p);   p += sizeof(uint32_t) * kKeys * SWS;
        s.cent = reinterpret_cast<float *>(p);    p += sizeof(float) * 256;
        s.bnd = reinterpret_cast<float *>(p);     p += sizeof(float) * 256;
        s.grid = reinterpret_cast<float4 *>(p);
    }
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, kb = lane >> 4;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kKeys;

    // codebook tables (L <= 128 entries, at most kGridLds = kThreads code
    // cells of 16 bytes): loads issued unconditionally (indices clamped) ahead of
    // the keys, stored to LDS after them, so both share one round trip
    const int ti = tid < L ? tid : L - 1;
    const float cent_v = a.centroids[ti];
    const float bnd_v = a.boundaries[ti];      // entry L - 1 is +inf
    float4 grid_v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if constexpr (BITS >= kCellBits) grid_v = a.grid[tid < a.ngrid ? tid : a.ngrid - 1];
    for (int i = tid; i < kKeys * CWS; i += kThreads) s.cw[i] = 0u;
    for (int i = tid; i < kKeys * SWS; i += kThreads) s.sw[i] = 0u;
    if (tid < kKeys) s_row[tid] = n0 + tid < n_total ? out_row(a.map, a.H, a.T, n0 + tid) : -1;
    // Pi's fragments of the first k-step, in flight with the keys
    const __amdgpu_buffer_rsrc_t pt = frag_table(HALF ? a.pihfrag : a.pifrag, frag_table_bytes<D, NTAB>());
    const __amdgpu_buffer_rsrc_t st = frag_table(a.sfrag, a.m > 0 ? frag_table_bytes<D, 2>() : 0);
    uint4 af[2][RTW][NPA];
    load_pi_frag<D, NPA, NTAB>(pt, wave, lane, 0, af[0]);

    // ---- 0. the workgroup's keys into LDS, one HBM round trip: thread
    // (key kk, quarter q) loads quarter q of row kk as 16-byte chunks (row n
    // at n d for densely packed inputs; otherwise found with one divide per
    // workgroup, then stepping across sequence / head boundaries) and sums
    // the squares of its elements: partial q of ||k||^2.  Slots past the last
    // key reload that key (loads stay unconditional); their results are never
    // stored.
    constexpr int RSTR = key_stage_stride<D, TIn>();
    constexpr int CH16 = D * static_cast<int>(sizeof(TIn)) / 16;     // 16-byte chunks per row
    constexpr int CPT = CH16 / TPK;                                    // chunks per thread
    unsigned char *kst = reinterpret_cast<unsigned char *>(s.rfrag);
    {
        const int kk = tid / TPK, q = tid % TPK;
        const int last = static_cast<int>(n_total - 1 - n0 < kKeys - 1 ? n_total - 1 - n0 : kKeys - 1);
        const int kr = kk < last ? kk : last;
        const TIn *row;
        if (a.contig) {
            row = static_cast<const TIn *>(a.k) + (n0 + kr) * D;
        } else {
            const int64_t bh0 = n0 / a.T, t0 = n0 - bh0 * a.T;
            int64_t t = t0 + kr, h = bh0 % a.H, b = bh0 / a.H;
            while (t >= a.T) {      // at most 64 / T + 1 steps
                t -= a.T;
                if (++h == a.H) {
                    h = 0;
                    ++b;
                }
            }
            row = static_cast<const TIn *>(a.k) + b * a.sb + h * a.sh + t * a.st;
        }
        const uint4 *src = reinterpret_cast<const uint4 *>(row) + q * CPT;
        uint4 v[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) v[c] = src[c];
        uint4 *dst = reinterpret_cast<uint4 *>(kst + kk * RSTR) + q * CPT;
        if constexpr (!HALF) {
#pragma unroll
            for (int c = 0; c < CPT; ++c) dst[c] = v[c];
        }
        // partial q of ||k||^2 in fp32, one subtree of a fixed tree: each
        // group of eight consecutive elements is one fma chain and the groups
        // are summed pairwise (key_norm2 finishes the tree over the TPK
        // partials).  A term passes through at most 7 + log2(D / 8) roundings
        // of sums of non-negative terms (one more for an fp32 input's square;
        // bf16 and fp16 squares are exact): 13 * 2^-24 < 8e-7 relative at
        // d = 256, 4e-7 in ||k||
        // (bf16 keys: one v_dot2c_f32_bf16 per element pair, x0^2 + x1^2 + acc,
        // at most two roundings per step, so still at most 8 in a group)
        constexpr int EPC = 16 / static_cast<int>(sizeof(TIn));     // elements per chunk
        constexpr int NG = CPT * EPC / 8;                              // groups of this thread
        static_assert(NG >= 1 && (NG & (NG - 1)) == 0, "whole groups, a power of two per thread");
        float gs[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) gs[g] = 0.0f;
        if constexpr (__is_same(TIn, bf16_t)) {
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                const uint32_t u[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) gs[c] = sq2_bf16(u[i], gs[c]);
            }
        } else {
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                float x[8];
                chunk_as_f32<TIn>(v, c, x);
#pragma unroll
                for (int e = 0; e < EPC; ++e) gs[(c * EPC + e) / 8] = fmaf(x[e], x[e], gs[(c * EPC + e) / 8]);
            }
        }
#pragma unroll
        for (int w = 1; w < NG; w *= 2)
#pragma unroll
            for (int g = 0; g < NG; g += 2 * w) gs[g] += gs[g + w];
        s.nrm2[q * kKeys + kk] = static_cast<double>(gs[0]);
        if constexpr (HALF) {
            // the key's ||k||^2 from its TPK threads (consecutive lanes; each
            // xor step adds the same two values in either order, so every
            // thread of the key gets the same bits and the same exponent):
            // ||k||^2 < 2^E, so ||k|| < 2^ceil(E/2) and ||k|| 2^ex < 2^kKeyHalfExp
            float n2 = gs[0];
#pragma unroll
            for (int o = 1; o < TPK; o *= 2) n2 += __shfl_xor(n2, o);
            const int ex = kKeyHalfExp - ((__builtin_amdgcn_frexp_expf(n2) + 1) >> 1);
#pragma unroll
            for (int c = 0; c < CPT; ++c) dst[c] = chunk_as_f16<TIn>(v[c], ex);
            if (q == 0) s_kexp[kk] = ex;
        }
    }
    if (tid < L) {
        s.cent[tid] = cent_v;
        s.bnd[tid] = bnd_v;
    }
    if constexpr (BITS >= kCellBits)
        if (tid < a.ngrid) s.grid[tid] = grid_v;
    __syncthreads();   // staged keys, cleared words, codebook tables

    // ---- 1. y = Pi k (unnormalised): acc[j][kt][r] of lane (col, kb) is
    // coordinate SEGC (4 wave + kb) + 4 j + r of key 16 kt + col (the row order
    // of the fragment table).
    // Pi's A fragments come from L2, double-buffered: the next k-step's are
    // in flight while this k-step's products run.
    f32x4 acc[RTW][kKT];
#pragma unroll
    for (int j = 0; j < RTW; ++j)
#pragma unroll
        for (int kt = 0; kt < kKT; ++kt) acc[j][kt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS) load_pi_frag<D, NPA, NTAB>(pt, wave, lane, ks + 1, af[(ks + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);     // keep the prefetch ahead of this k-step's products
        uint4 kf[kKT][NK];
#pragma unroll
        for (int kt = 0; kt < kKT; ++kt) {
            const unsigned char *kp = kst + (16 * kt + col) * RSTR + (32 * ks + 8 * kb) * static_cast<int>(sizeof(TIn));
            if constexpr (HALF) kf[kt][0] = *reinterpret_cast<const uint4 *>(kp);     // staged as fp16
            else key_frag_lds<TIn, NK>(kp, kf[kt]);
        }
#pragma unroll
        for (int j = 0; j < RTW; ++j) {
#pragma unroll
            for (int pp = 0; pp < NPA; ++pp) {
#pragma unroll
                for (int kq = 0; kq < NK; ++kq) {
                    if (pp + kq > 2) continue;     // terms below fp32's resolution
#pragma unroll
                    for (int kt = 0; kt < kKT; ++kt) {
                        if constexpr (HALF) acc[j][kt] = mfma_f16(af[ks & 1][j][pp], kf[kt][kq], acc[j][kt]);
                        else acc[j][kt] = mfma_bf16(af[ks & 1][j][pp], kf[kt][kq], acc[j][kt]);
                    }
                }
            }
        }
    }
    __syncthreads();   // every wave is done with the staged keys (the region takes the residuals next)
    // 1-2 bits: the codebook is exactly symmetric (c[L-1-i] = -c[i], and so
    // the boundaries, with t[L/2-1] = 0), so |y| is placed against the one
    // positive boundary in registers and the centroid taken from the H
    // positive ones; idx and y - c[idx] follow from the sign of y, bit for bit
    // as the full count would give them (up to exact ties)
    constexpr int H = L / 2;
    float cp[H];
    const float tp0 = (BITS == 2) ? s.bnd[H] : 0.0f;
    if constexpr (BITS < kCellBits) {
#pragma unroll
        for (int i = 0; i < H; ++i) cp[i] = s.cent[H + i];
    }
    float inv_n[kKT], tv[kKT];
#pragma unroll
    for (int kt = 0; kt < kKT; ++kt) {
        const int key = 16 * kt + col;
        // 1/||k|| only scales y: fp32 rsqrt (about 1 ulp) moves y by ~1e-7 at most,
        // far inside the 1e-5 boundary band; the stored ||k|| is the fp64 root
        // of the same sum, rounded once
        const float n2 = key_norm2<TPK>(s.nrm2, kKeys, key);
        inv_n[kt] = (n2 > 0.0f) ? a.rot_scale * __builtin_amdgcn_rsqf(n2) : 0.0f;
        tv[kt] = reg_bound(tp0, n2, a.inv_rot_scale);
        if constexpr (HALF) {
            // acc is y 2^(kPiHalfExp + ex): both factors are exact powers of two
            const int sh = kPiHalfExp + s_kexp[key];
            inv_n[kt] = __builtin_amdgcn_ldexpf(inv_n[kt], -sh);
            tv[kt] = __builtin_amdgcn_ldexpf(tv[kt], sh);
        }
    }

    const bool qjl = a.m > 0;
    // S's fragments of the first k-step of step 4, in flight with step 3
    uint4 sf0[RTW][2];
    if (qjl) load_s_frag<D>(st, wave, lane, 0, sf0);
    const int qb = SEGC * (4 * wave + kb);      // first coordinate this lane holds
    // ---- 3. codes idx = #{boundaries < y}, residual r = y - c[idx], ||r||
#pragma unroll
    for (int kt = 0; kt < kKT; ++kt) {
        const int key = 16 * kt + col;
        float rr = 0.0f;
        uint32_t seg[NSEG + 1];               // code of coordinate qb + e at bit BITS e
#pragma unroll
        for (int i = 0; i <= NSEG; ++i) seg[i] = 0u;
#pragma unroll
        for (int j = 0; j < RTW; ++j) {
            float res[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int b = BITS * (4 * j + r);
                if constexpr (BITS < kCellBits) {
                    seg[b >> 5] |= encode_reg<BITS>(acc[j][kt][r], inv_n[kt], tv[kt], cp, res[r]) << (b & 31);
                } else {
                    const float y = acc[j][kt][r] * inv_n[kt];
                    const uint32_t pos = static_cast<uint32_t>(encode_cell(y, s, a, res[r]));
                    seg[b >> 5] |= pos << (b & 31);
                    if ((b & 31) + BITS > 32) seg[(b >> 5) + 1] |= pos >> (32 - (b & 31));
                }
                rr = fmaf(res[r], res[r], rr);
            }
            // residual as two bf16 terms (hardware round to nearest even), in
            // the B-operand slots of coordinates q0 .. q0 + 3: k-step q0 / 32,
            // k-block (q0 / 4) % 4 (the lane col + 16 k-block), elements
            // 4 ((q0 / 16) % 2) + r
            uint32_t h01, l01, h23, l23;
            split_bf16x2(res[0], res[1], h01, l01);
            split_bf16x2(res[2], res[3], h23, l23);
            const int q0 = qb + 4 * j, ks = q0 >> 5, bl = col + 16 * ((q0 >> 2) & 3), hw = 2 * ((q0 >> 4) & 1);
            uint32_t *dst = reinterpret_cast<uint32_t *>(&s.rfrag[((kt * KS + ks) * 2 + 0) * 64 + bl]);
            uint32_t *dst1 = reinterpret_cast<uint32_t *>(&s.rfrag[((kt * KS + ks) * 2 + 1) * 64 + bl]);
            *reinterpret_cast<uint2 *>(dst + hw) = make_uint2(h01, h23);
            *reinterpret_cast<uint2 *>(dst1 + hw) = make_uint2(l01, l23);
        }
        put_code_words<D, BITS, DIRECT, NSEG>(s, a, seg, key, s_row[key], qb, kb);
        double rd = static_cast<double>(rr);
        rd += __shfl_xor(rd, 16);
        rd += __shfl_xor(rd, 32);
        if (kb == 0) s.rho2[wave * kKeys + key] = rd;
    }
    __syncthreads();

    // ---- 4. z = S r on this wave's rows; signs [z >= 0] (skipped for the
    // first-stage format, m = 0; the condition is uniform over the launch)
    if (qjl) qjl_signs<D, kKT, DIRECT>(st, s, a, s_row, 0, wave, lane, sf0);

    // ---- 5. the workgroup's norms (and, from LDS, its code and sign words)
    store_keys<D, BITS, kKeys, TPK, 4, !DIRECT>(a, s, s_row, qjl);
}


// ---------------------------------------------------------------------------
// Walsh-Hadamard rotations (TQ_ROT_HADAMARD: y = H D1 k / sqrt(d);
// TQ_ROT_HADAMARD2: y = H D2 H D1 k / d) as a randomized butterfly in
// registers (tproger.ru article, section "Implementations": the Walsh-Hadamard
// transform as the O(d log d) rotation).
//
// A key's d coordinates sit in the 16 lanes of one DPP row, CPL = d / 16
// consecutive coordinates per lane.  The stages over the coordinate bits below
// log2(CPL) are add/sub pairs in registers; the four above them run across the
// row as v_fmac_f32 with a DPP source: self + s * partner, partners along the
// quad swaps (lane ^ 1, lane ^ 2), the half-row mirror (lane ^ 7) and the row
// mirror (lane ^ 15), with s = +-1 per lane and stage (kWhtNeg).  Since the
// mirrors pair lanes along 7 and 15 rather than 4 and 8, the lane stages give
// Sylvester's H_16 up to a fixed relabelling of the lanes and a sign per lane:
// lane p ends with sign(p) * (H_16 v)[out(p)], out(p) the nibble p of
// kWhtOut, sign(p) = -1 where bit p of kWhtEps is set (H_16 is symmetric in
// that relabelling, so a second round fed with the first round's lanes
// undoes it and ends in natural order).  The lane holding output chunk c
// then encodes coordinates [CPL c, CPL c + CPL) of its key directly: codes,
// residual, and the residual's B-operand slots of the QJL product.
constexpr uint32_t kWhtNeg[4] = {0x5a5au, 0x3c3cu, 0x0ff0u, 0xff00u};
constexpr uint32_t kWhtEps = 0x9696u;
constexpr uint64_t kWhtOut = 0x8deb7214c9af3650ull;
constexpr int kWhtPartner[4] = {1, 2, 7, 15};    // lane stage k pairs lane p with p ^ kWhtPartner[k]

// Lane permutations within a 16-lane row (quad swaps, half-row and row
// mirrors): every source lane exists, so the move needs no "old" value and
// the compiler folds it into the consuming v_add_f32 as a DPP operand
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// sums over the 16 lanes of a DPP row, left in every lane of the row
__device__ __forceinline__ float row16_sum_f32(float x)
{
    x += dpp_f32<0xB1>(x);
    x += dpp_f32<0x4E>(x);
    x += dpp_f32<0x141>(x);
    return x + dpp_f32<0x140>(x);
}

// One lane stage on four values: x += s * (the partner lane's x), one
// v_fmac_f32 with a DPP source per value (the compiler does not fold a DPP
// move into v_fmac_f32, whose accumulator is tied to the destination, and
// would spend a separate v_mov_b32_dpp on each).  The s_nop gives the two
// wait states a DPP read needs after a VALU write of its source.
#define TQ_WHT_FMAC(N, CTL) "v_fmac_f32_dpp %" #N ", %" #N ", %4 " CTL " row_mask:0xf bank_mask:0xf bound_ctrl:1"
#define TQ_WHT_STAGE4(CTL, X, E, S)                                                                        \
    asm("s_nop 1\n\t" TQ_WHT_FMAC(0, CTL) "\n\t" TQ_WHT_FMAC(1, CTL) "\n\t" TQ_WHT_FMAC(2, CTL) "\n\t"     \
        TQ_WHT_FMAC(3, CTL)                                                                               \
        : "+v"(X[E]), "+v"(X[E + 1]), "+v"(X[E + 2]), "+v"(X[E + 3])                                      \
        : "v"(S))

// one round: the in-register stages, then the four lane stages (partners
// lane ^ 1, lane ^ 2, the half-row mirror and the row mirror)
template <int CPL>
__device__ __forceinline__ void wht_round(float (&x)[CPL], const float (&sg)[4])
{
    static_assert(CPL % 4 == 0, "lane stages take four values at a time");
#pragma unroll
    for (int h = 1; h < CPL; h *= 2)
#pragma unroll
        for (int e = 0; e < CPL; ++e)
            if (!(e & h)) {
                const float u = x[e], v = x[e + h];
                x[e] = u + v;
                x[e + h] = u - v;
            }
#pragma unroll
    for (int e = 0; e < CPL; e += 4) TQ_WHT_STAGE4("quad_perm:[1,0,3,2]", x, e, sg[0]);
#pragma unroll
    for (int e = 0; e < CPL; e += 4) TQ_WHT_STAGE4("quad_perm:[2,3,0,1]", x, e, sg[1]);
#pragma unroll
    for (int e = 0; e < CPL; e += 4) TQ_WHT_STAGE4("row_half_mirror", x, e, sg[2]);
#pragma unroll
    for (int e = 0; e < CPL; e += 4) TQ_WHT_STAGE4("row_mirror", x, e, sg[3]);
}
#undef TQ_WHT_STAGE4
#undef TQ_WHT_FMAC

// CPL consecutive input elements of one lane as loaded: NW = CPL * size / 4
// words, in 16-byte loads (8-byte ones for four 2-byte elements, d = 64)
template <typename TIn, int CPL>
struct LaneChunk {
    static constexpr int NW = CPL * static_cast<int>(sizeof(TIn)) / 4;
    uint32_t w[NW];

    __device__ void load(const TIn *p)
    {
        if constexpr (NW >= 4) {
#pragma unroll
            for (int c = 0; c < NW / 4; ++c) {
                const uint4 u = reinterpret_cast<const uint4 *>(p)[c];
                w[4 * c] = u.x; w[4 * c + 1] = u.y; w[4 * c + 2] = u.z; w[4 * c + 3] = u.w;
            }
        } else {
            const uint2 u = *reinterpret_cast<const uint2 *>(p);
            w[0] = u.x; w[1] = u.y;
        }
    }

    // the elements as fp32
    __device__ void unpack(float (&x)[CPL]) const
    {
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            if constexpr (sizeof(TIn) == 4) {
                x[i] = __uint_as_float(w[i]);
            } else if constexpr (__is_same(TIn, bf16_t)) {
                x[2 * i] = bf16_to_f32(w[i] & 0xffffu);
                x[2 * i + 1] = bf16_to_f32(w[i] >> 16);
            } else {
                x[2 * i] = f16_bits_to_f32(w[i] & 0xffffu);
                x[2 * i + 1] = f16_bits_to_f32(w[i] >> 16);
            }
        }
    }

    // the lane's share of ||k||^2 in fp32: interleaved chains summed pairwise
    // (an fma per element in four chains; for bf16 one v_dot2c_f32_bf16 per
    // pair, in two chains up to four pairs and four beyond)
    __device__ float norm2(const float (&x)[CPL]) const
    {
        float q4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (__is_same(TIn, bf16_t)) {
            constexpr int NCH = NW > 4 ? 4 : 2;
#pragma unroll
            for (int i = 0; i < NW; ++i) q4[i % NCH] = sq2_bf16(w[i], q4[i % NCH]);
        } else {
#pragma unroll
            for (int e = 0; e < CPL; ++e) q4[e & 3] = fmaf(x[e], x[e], q4[e & 3]);
        }
        return (q4[0] + q4[1]) + (q4[2] + q4[3]);
    }
};

template <int D, typename TIn, int KT>
constexpr size_t key_smem_bytes_wht(int bits)
{
    constexpr size_t keys = 16 * KT;
    const size_t rfrag = sizeof(uint4) * key_pass_tiles<D, TIn, KT>() * (D / 32) * 2 * 64;
    return rfrag + sizeof(uint32_t) * keys * ((D * bits / 32 + 1) + sw_stride<D>()) + sizeof(double) * 2 * keys
           + sizeof(float) * 512 + (bits >= kCellBits ? sizeof(float4) * kGridLds : 0);
}

// One 256-thread workgroup encodes 16 KT keys; wave w takes keys 16 t + 4 w + g
// of key tile t in lane row g.  Steps: load (each lane its CPL elements) and
// ||k||^2 (fp32, summed over the row); the butterfly;
// codes, residual and ||r||^2 per lane; then, per pass of KR tiles, the QJL
// product and the store shared with the matrix-core kernel.
template <int D, typename TIn, int BITS, int KT, int ROUNDS>
__global__ __launch_bounds__(kThreads, (key_occupancy<D, TIn, KT>())) void k_compress_keys_wht(KeyLaunch a, int64_t n_total)
{
    constexpr int CPL = D / 16;          // coordinates per lane
    constexpr int KS = D / 32;
    constexpr int L = 1 << BITS;
    constexpr int H = L / 2;
    constexpr int CW = D * BITS / 32, CWS = cw_stride<D, BITS>(), SWS = sw_stride<D>();
    constexpr int kKeys = 16 * KT;
    constexpr int KR = key_pass_tiles<D, TIn, KT>();
    constexpr int NSW = (BITS * CPL + 31) / 32;   // code words of one lane's segment
    extern __shared__ __align__(16) unsigned char smem_raw[];
    __shared__ int64_t s_row[kKeys];
    KeySmem s;
    {
        unsigned char *p = smem_raw;
        s.rfrag = reinterpret_cast<uint4 *>(p);   p += sizeof(uint4) * KR * KS * 2 * 64;
        s.rho2 = reinterpret_cast<double *>(p);   p += sizeof(double) * kKeys;
        s.nrm2 = reinterpret_cast<double *>(p);   p += sizeof(double) * kKeys;
        s.cw = reinterpret_cast<uint32_t *>(p);   p += sizeof(uint32_t) * kKeys * CWS;
        s.sw = reinterpret_cast<uint32_t *>(p);   p += sizeof(uint32_t) * kKeys * SWS;
        s.cent = reinterpret_cast<float *>(p);    p += sizeof(float) * 256;
        s.bnd = reinterpret_cast<float *>(p);     p += sizeof(float) * 256;
        s.grid = reinterpret_cast<float4 *>(p);
    }
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, pl = lane & 15;      // lane row (key of the round) and lane in the row
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kKeys;

    // codebook tables, loaded ahead of the keys
    const int ti = tid < L ? tid : L - 1;
    const float cent_v = a.centroids[ti];
    const float bnd_v = a.boundaries[ti];
    float4 grid_v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if constexpr (BITS >= kCellBits) grid_v = a.grid[tid < a.ngrid ? tid : a.ngrid - 1];
    for (int i = tid; i < kKeys * CWS; i += kThreads) s.cw[i] = 0u;
    for (int i = tid; i < kKeys * SWS; i += kThreads) s.sw[i] = 0u;
    if (tid < kKeys) s_row[tid] = n0 + tid < n_total ? out_row(a.map, a.H, a.T, n0 + tid) : -1;

    // this lane's elements of each of its KT keys (slots past the last key
    // reload that key; their results are never stored)
    const int last = static_cast<int>(n_total - 1 - n0 < kKeys - 1 ? n_total - 1 - n0 : kKeys - 1);
    LaneChunk<TIn, CPL> x[KT];
#pragma unroll
    for (int t = 0; t < KT; ++t) {
        const int kk = 16 * t + 4 * wave + g;
        const int kr = kk < last ? kk : last;
        const TIn *row;
        if (a.contig) {
            row = static_cast<const TIn *>(a.k) + (n0 + kr) * D;
        } else {
            const int64_t bh0 = n0 / a.T, t0 = n0 - bh0 * a.T;
            int64_t tt = t0 + kr, h = bh0 % a.H, b = bh0 / a.H;
            while (tt >= a.T) {
                tt -= a.T;
                if (++h == a.H) {
                    h = 0;
                    ++b;
                }
            }
            row = static_cast<const TIn *>(a.k) + b * a.sb + h * a.sh + tt * a.st;
        }
        x[t].load(row + CPL * pl);
    }
    // round signs of this lane.  The plain butterfly leaves lane p with
    // eps(p) times its output chunk; instead every value the lane holds is kept
    // times eps(p): the input D1 k times eps(p), and each lane stage's
    // coefficient s(p) times eps(p) eps(partner), since eps(p) (x(p) + s x(q))
    // = z(p) + s eps(p) eps(q) z(q) for z = eps x.  A round then ends with the
    // chunk itself.  A second round takes D2 of the coordinates the lane holds
    // after the first, again times eps(p).
    float d1[CPL], d2[ROUNDS == 2 ? CPL : 1];
    const int out1 = static_cast<int>((kWhtOut >> (4 * pl)) & 15);
    const float eps = ((kWhtEps >> pl) & 1u) ? -1.0f : 1.0f;
#pragma unroll
    for (int e = 0; e < CPL; ++e) d1[e] = a.wht[CPL * pl + e] * eps;
    if constexpr (ROUNDS == 2) {
#pragma unroll
        for (int e = 0; e < CPL; ++e) d2[e] = a.wht[D + CPL * out1 + e] * eps;
    }
    float sg[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t neg = (kWhtNeg[k] >> pl) ^ (kWhtEps >> pl) ^ (kWhtEps >> (pl ^ kWhtPartner[k]));
        sg[k] = (neg & 1u) ? -1.0f : 1.0f;
    }
    if (tid < L) {
        s.cent[tid] = cent_v;
        s.bnd[tid] = bnd_v;
    }
    if constexpr (BITS >= kCellBits)
        if (tid < a.ngrid) s.grid[tid] = grid_v;
    __syncthreads();   // cleared words, codebook tables

    float cp[H];
    const float tp0 = (BITS == 2) ? s.bnd[H] : 0.0f;
    if constexpr (BITS < kCellBits) {
#pragma unroll
        for (int i = 0; i < H; ++i) cp[i] = s.cent[H + i];
    }
    // output chunk of this lane (one round: relabelled; two: natural)
    const int chunk = ROUNDS == 1 ? out1 : pl;
    const bool qjl = a.m > 0;
    const __amdgpu_buffer_rsrc_t st = frag_table(a.sfrag, qjl ? frag_table_bytes<D, 2>() : 0);
#pragma unroll
    for (int kt0 = 0; kt0 < KT; kt0 += KR) {
        // S's fragments of the first k-step of the sign product, in flight
        // with the butterflies
        uint4 sf0[D / 64][2];
        if (qjl) load_s_frag<D>(st, wave, lane, 0, sf0);
#pragma unroll
        for (int t = kt0; t < kt0 + KR; ++t) {
            const int key = 16 * t + 4 * wave + g;
            // ||k||^2 in fp32: four interleaved chains per lane, summed
            // pairwise, then over the key's 16 lanes in a DPP tree.  Every
            // term passes through at most CPL / 4 + 6 roundings of sums of
            // non-negative terms (one more for an fp32 input's square;
            // bf16 and fp16 squares are exact; a bf16 pair step rounds at
            // most twice for two elements), so the relative error stays
            // below 11 * 2^-24 < 7e-7 at d = 256: under 4e-7 in ||k||
            float xe[CPL];
            x[t].unpack(xe);
            const float ss = row16_sum_f32(x[t].norm2(xe));
            float v[CPL];
#pragma unroll
            for (int e = 0; e < CPL; ++e) v[e] = xe[e] * d1[e];
            wht_round<CPL>(v, sg);
            if constexpr (ROUNDS == 2) {
#pragma unroll
                for (int e = 0; e < CPL; ++e) v[e] *= d2[e];
                wht_round<CPL>(v, sg);
            }
            const float n2 = ss;
            const float scale = (n2 > 0.0f) ? a.rot_scale * __builtin_amdgcn_rsqf(n2) : 0.0f;
            const float tv = reg_bound(tp0, n2, a.inv_rot_scale);
            // codes and residual of coordinates [CPL chunk, CPL chunk + CPL)
            float res[CPL];
            uint32_t seg[NSW + 1];
#pragma unroll
            for (int i = 0; i <= NSW; ++i) seg[i] = 0u;
            float rr = 0.0f;
#pragma unroll
            for (int e = 0; e < CPL; ++e) {
                const int bo = BITS * e;
                if constexpr (BITS < kCellBits) {
                    seg[bo >> 5] |= encode_reg<BITS>(v[e], scale, tv, cp, res[e]) << (bo & 31);
                } else {
                    const float y = v[e] * scale;
                    const uint32_t pos = static_cast<uint32_t>(encode_cell(y, s, a, res[e]));
                    seg[bo >> 5] |= pos << (bo & 31);
                    if ((bo & 31) + BITS > 32) seg[(bo >> 5) + 1] |= pos >> (32 - (bo & 31));
                }
                rr = fmaf(res[e], res[e], rr);
            }
            // the lane's CPL codes start at bit BITS CPL chunk of the key's row
            const int bit0 = BITS * CPL * chunk, w0 = bit0 >> 5, sh0 = bit0 & 31;
#pragma unroll
            for (int i = 0; i <= NSW; ++i) {
                const uint32_t word = sh0 ? ((seg[i] << sh0) | (i ? seg[i - 1] >> (32 - sh0) : 0u)) : seg[i];
                if (word != 0u && w0 + i < CW) atomicOr(&s.cw[key * CWS + w0 + i], word);
            }
            // residual as bf16 hi + lo terms in the B-operand slots of the QJL
            // product: coordinate l at k-step l / 32, k-block (l / 4) % 4,
            // element 4 ((l / 16) % 2) + l % 4 (the k order of the S fragments)
            const int col = 4 * wave + g;
#pragma unroll
            for (int q = 0; q < CPL / 4; ++q) {
                const int l = CPL * chunk + 4 * q;
                const int rt = l >> 4, kbq = (l >> 2) & 3;
                uint32_t h01, l01, h23, l23;
                split_bf16x2(res[4 * q], res[4 * q + 1], h01, l01);
                split_bf16x2(res[4 * q + 2], res[4 * q + 3], h23, l23);
                const int slot = ((t - kt0) * KS + (rt >> 1)) * 2;
                uint32_t *dst = reinterpret_cast<uint32_t *>(&s.rfrag[(slot + 0) * 64 + col + 16 * kbq]);
                uint32_t *dst1 = reinterpret_cast<uint32_t *>(&s.rfrag[(slot + 1) * 64 + col + 16 * kbq]);
                const int hw = 2 * (rt & 1);
                *reinterpret_cast<uint2 *>(dst + hw) = make_uint2(h01, h23);
                *reinterpret_cast<uint2 *>(dst1 + hw) = make_uint2(l01, l23);
            }
            rr = row16_sum_f32(rr);
            if (pl == 0) {
                s.nrm2[key] = static_cast<double>(ss);
                s.rho2[key] = static_cast<double>(rr);
            }
        }
        __syncthreads();
        if (qjl) qjl_signs<D, KR, false>(st, s, a, s_row, kt0, wave, lane, sf0);
    }
    store_keys<D, BITS, kKeys, 1, 1, true>(a, s, s_row, qjl);
}

template <int D, typename TIn, int BITS, int KT, int ROUNDS>
hipError_t launch_keys_wht(const KeyLaunch &a, hipStream_t stream)
{
    const int64_t n = static_cast<int64_t>(a.B) * a.H * a.T;
    constexpr size_t smem = key_smem_bytes_wht<D, TIn, KT>(BITS);
    auto kern = k_compress_keys_wht<D, TIn, BITS, KT, ROUNDS>;
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

template <int D, typename TIn, int BITS, int KT>
hipError_t launch_keys_k(const KeyLaunch &a, hipStream_t stream)
{
    if (a.wht_kernel && a.wht_rounds == 1) return launch_keys_wht<D, TIn, BITS, KT, 1>(a, stream);
    if (a.wht_kernel && a.wht_rounds == 2) return launch_keys_wht<D, TIn, BITS, KT, 2>(a, stream);
    const int64_t n = static_cast<int64_t>(a.B) * a.H * a.T;
    constexpr size_t smem = key_smem_bytes<D, TIn, BITS, KT>();
    auto kern = a.hadamard ? k_compress_keys<D, TIn, BITS, KT, 1> : k_compress_keys<D, TIn, BITS, KT, 3>;
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

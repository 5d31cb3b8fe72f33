// Internal declarations shared by the C-ABI layer and the HIP kernels of libtq.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <vector>

#include "../../include/tq.h"

struct tq_codebook {
    int d = 0, bits = 0;
    std::vector<double> centroids, boundaries;   // fp64 host tables
    float *d_centroids = nullptr;                // device fp32 [2^bits]
    float *d_boundaries = nullptr;               // device fp32 [2^bits - 1], then +inf
    // codes of kCellBits+ bits: a uniform grid over [first, last boundary] whose cells,
    // widened by 2 % of a cell on each side, hold at most one boundary each.
    // Cell c = {t, c_lo, c_hi, below (int bits)}: every y of the cell has
    // #{t_i < y} = below + [y > t], and centroid c_lo (c_hi above t); t = +inf
    // and c_hi = c_lo where the cell holds no boundary
    float4 *d_grid = nullptr;
    int ngrid = 0;
    float grid_lo = 0.0f, grid_scale = 0.0f;
    int device = 0;
};

struct tq_rotation {
    uint64_t seed = 0;
    int d = 0, m = 0;
    tq_rot_kind kind = TQ_ROT_DENSE;
    // device fp32 tables (one allocation, carved up)
    float *d_pi = nullptr;      // [d][d]  y = Pi u, row-major
    float *d_piT = nullptr;     // [d][d]  transpose of Pi
    float *d_s = nullptr;       // [m][d]  QJL projection
    float *d_sT = nullptr;      // [d][m]  transpose of S
    float *d_dsign = nullptr;   // [d]     Hadamard signs (+-1), dense: unused
    float *d_spiT = nullptr;    // [d][m]  transpose of S Pi (Sq = S Pi q in one product)
    float *d_pisum = nullptr;   // [d]     column sums of Pi: sum_j (Pi q)_j = pisum . q
    float *d_spisum = nullptr;  // [d]     column sums of S Pi
    float *d_wht = nullptr;     // [2][d]  signs D1, D2 of the Walsh-Hadamard rounds (+-1; ones if absent)
    float sq_bound = 0.0f;      // max row norm of S Pi (rounded up): |(S Pi q)_i| <= sq_bound |q|
    double *d_pi64T = nullptr;  // [d][d]  fp64 transpose of Pi (block-format compressor)
    // bf16 operand fragments of the matrix-core key compressor, in lane order
    // (16x16x32 MFMA A operand: lane = row % 16 + 16 * k-block, 8 elements):
    //   pifrag [d/16 row tiles][d/32 k-steps][3 parts][64][8]: Pi = hi + mid + lo
    //   sfrag  [m/16 row tiles][d/32 k-steps][2 parts][64][8]: S = hi + mid, with
    //          k element e of k-block kb at coordinate 16 (2 ks + e/4) + 4 kb + e%4
    //   pihfrag [d/16 row tiles][d/32 k-steps][2 parts][64][8]: fp16 bits,
    //          Pi 2^kPiHalfExp = hi + lo (dense rotations; zeros otherwise)
    uint16_t *d_pifrag = nullptr;
    uint16_t *d_sfrag = nullptr;
    uint16_t *d_pihfrag = nullptr;
    void *d_frag_block = nullptr;
    void *d_block = nullptr;
    int device = 0;
};

namespace tq {

// Where the packed rows of a call live.  Flat: row n of the [B, H, T] call is
// row n of the planes.  Layout (contiguous or paged, tq_cache_layout): token t
// of (b, h) sits at layout_row(); a compress call in layout mode appends its
// token t of (b, h) at position pos[b] + t; a decode call in layout mode reads
// seq_lens[b] tokens of sequence b.
struct CacheMap {
    enum Mode { kFlat = 0, kContig = 1, kPaged = 2 };
    int mode = kFlat;
    int64_t cap = 0;                    // tokens a sequence can hold
    const int32_t *seq_lens = nullptr;  // decode: [B]
    const int32_t *pos = nullptr;       // append: [B]
    const int32_t *bt = nullptr;        // paged: [B][maxb]
    int bs = 0, maxb = 0;
    int64_t nblocks = 0;
};

// ---- host math (host_math.cpp)
uint64_t rng_draw(uint64_t seed, int stream, uint64_t k);
double rng_normal(uint64_t seed, int stream, uint64_t n);
tq_status lloyd_max_codebook(int d, int bits, double *centroids, double *boundaries,
                             double *residual_out, int max_iters = -1);
void dense_rotation(uint64_t seed, int d, double *pi);
void hadamard_signs(uint64_t seed, int d, float *signs, int stream = 1);
void hadamard_rotation(uint64_t seed, int d, double *pi, int stream = 1);
void hadamard2_rotation(uint64_t seed, int d, double *pi);
void qjl_projection(uint64_t seed, int m, int d, double *s);

// ---- kernel launchers.  All return hipSuccess or the launch error.
struct KeyLaunch {
    const void *k;
    tq_dtype dtype;
    int B, H;
    int64_t T, sb, sh, st;      // element strides
    bool contig;                // rows packed densely ([B, H, T, d] contiguous): row n at n d
    int d, bits, m;
    bool hadamard;              // Pi = integer matrix * rot_scale, exact in one bf16 term
    float rot_scale;            // 1/sqrt(d) (one Hadamard round), 1/d (two rounds), else 1
    float inv_rot_scale;        // 1 / rot_scale (sqrt(d), d or 1)
    const float *piT, *sT, *dsign, *centroids, *boundaries;
    const float *wht;           // [2][d] Walsh-Hadamard round signs D1, D2
    int wht_rounds;             // 0 dense, 1 or 2 Walsh-Hadamard rounds
    bool wht_kernel;            // Walsh-Hadamard rounds as the register butterfly (else the +-1 matrix product)
    const float4 *grid;         // code cells (tq_codebook::d_grid)
    int ngrid;
    float grid_lo, grid_scale;
    float grid_off, grid_max;   // -grid_lo grid_scale (rounded once), ngrid - 1
    const uint16_t *pifrag, *sfrag;
    const uint16_t *pihfrag;    // Pi 2^kPiHalfExp as two fp16 terms (dense rotations)
    tq_kcache out;
    CacheMap map;               // flat, or appending into a layout cache
};
hipError_t launch_compress_keys(const KeyLaunch &a, hipStream_t stream);
// power of two that lifts Pi (|entries| <= 1) for its two fp16 terms: the
// leading term stays at or below 2^14 (fp16's largest finite value is
// 65504), and the second one, about 2^-11 of it, stays out of fp16's
// subnormal range for every entry above 2^-17
constexpr int kPiHalfExp = 14;
constexpr int kCellBits = 3;       // codes of kCellBits or more bits are read from code cells
constexpr int kMaxGrid = 8192;     // cells of a codebook's code grid
constexpr int kGridLds = 256;      // cells the key compressor stages in LDS (every codebook of d >= 3, <= 7 bits)

struct ValueLaunch {
    const void *v;
    tq_dtype dtype;
    int B, H;
    int64_t T, sb, sh, st;
    int d, bits, group;
    tq_vcache out;
    CacheMap map;
};
hipError_t launch_compress_values(const ValueLaunch &a, hipStream_t stream);

// rotated block key formats (k_block.hip)
struct BlockLaunch {
    const void *k;
    tq_dtype dtype;
    int B, H;
    int64_t T, sb, sh, st;
    int d, bits;                // bits 8 or 4
    const double *pi64T;        // [d][d], row j = input coordinate
    tq_bcache out;
};
hipError_t launch_compress_keys_block(const BlockLaunch &a, hipStream_t stream);

// explicit key estimates (k_dequant.hip)
struct DequantLaunch {
    int64_t N;                  // keys (B * Hkv * T), rows of every plane
    int d, bits, m;
    float kappa;                // sqrt(pi/2) / m, 0 without QJL rows
    const float *pi, *s, *centroids;    // Pi [d][d] and S [m][d] row-major
    const uint8_t *codes, *signs;
    const float *knorm, *rnorm;
    float *out;                 // [N][d]
};
hipError_t launch_dequant_keys(const DequantLaunch &a, hipStream_t stream);

// extra state of the matrix-core decode path
struct MfmaArgs {
    int gc = 0;                 // query heads per unit (<= 8)
    int nqc = 0;                // query chunks per KV head
    int mt = 0;                 // 4-query row tiles of the score product
    int units = 0;              // B * Hkv * nqc
    uint32_t *aops = nullptr;   // [units][mt][steps][64 lanes][4 dwords] score digit operands
    float *qscal = nullptr;     // [B, Hq, 4] fixed-point scales, constant terms
    float lscale = 0.0f;        // factor on the scores: softmax scale * log2(e), or 1 for raw scores
};

struct DecodeLaunch {
    const void *q;              // [B, Hq, d]
    tq_dtype dtype;
    int B, Hq, Hkv;
    int64_t T;
    int d, bits, m;
    const float *piT, *sT, *centroids;
    const float *spiT;          // (S Pi)^T, [d][m]
    const float *pisum, *spisum;    // column sums of Pi and S Pi
    float sq_bound;             // max row norm of S Pi
    tq_kcache kc;
    // attention only
    int vbits, group;
    tq_vcache vc;
    float scale;
    int splits;
    // workspace carve-up
    float *qprep;               // [B, Hq, d + m]
    float *part_ml;             // [B, Hq, splits, 2]
    float *part_acc;            // [B, Hq, splits, d]
    float *scores;              // tq_scores output [B, Hq, T]
    float *out;                 // [B, Hq, d]
    CacheMap map;               // flat (T tokens each) or a layout cache (T = capacity)
    // rotated block key formats (kfmt_block): planes and per-(query, block) offsets
    bool kfmt_block = false;
    tq_bcache kq;
    float *qaux;                // [B, Hq, d / 32]
    MfmaArgs mf;
};
hipError_t launch_qprep(const DecodeLaunch &a, hipStream_t stream);
hipError_t launch_scores(const DecodeLaunch &a, hipStream_t stream);
hipError_t launch_attend(const DecodeLaunch &a, hipStream_t stream);

// query-chunk size the decode kernels use for a GQA group of G heads
int query_chunk(int G);
constexpr int kDecodeTile = 256;   // keys per decode tile

// matrix-core decode path (k_attend_mfma.hip): d 128/256, any key bits
constexpr int kMfmaTile = 128;     // keys per workgroup step (four waves x 32)
constexpr int kStageBlocks = 512;  // paged caches: block ids of one split staged in LDS
bool mfma_decode_supported(int d, int bits, int G, int vbits, int group);
int mfma_query_chunk(int G);
int mfma_score_steps(int d, int bits, int m);
int mfma_row_tiles(int bits, int gc);
hipError_t launch_decode_mfma(const DecodeLaunch &a, hipStream_t stream);
hipError_t launch_scores_mfma(const DecodeLaunch &a, hipStream_t stream);   // raw scores, tq_scores
hipError_t launch_decode_block(const DecodeLaunch &a, hipStream_t stream);

// ---- profiling hooks (api.cpp)
void prof_begin(const char *name, hipStream_t stream, void **token);
void prof_end(void *token, hipStream_t stream);
// while set on this thread, prof_begin records nothing (the allocation-free
// entry point creates no events)
void prof_suppress(bool on);

// ---- static device scratch (scratch.hip): its size, and its address on the
// current device (looked up once per device)
size_t scratch_capacity();
hipError_t scratch_address(void **out);

}  // namespace tq

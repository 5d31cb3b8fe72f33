/*
 * libtq: TurboQuant KV-cache compression and decode attention for AMD MI355X
 * (gfx950).  C ABI: plain pointers and sizes only.
 *
 * The method (pages "turboquant-pytorch", section "What it does", and the
 * discosf.com TurboQuant article, section "TurboQuant in one sentence",
 * steps 1-4):
 *   keys   : normalise, rotate by a random orthogonal matrix Pi, quantise each
 *            rotated coordinate with a Lloyd-Max codebook, and keep one sign
 *            bit per row of a Gaussian QJL projection S of the residual;
 *   values : min-max quantise each group of g channels to 2 or 4 bits with an
 *            fp16 scale and zero, packed four (or two) codes per byte;
 *   decode : score the query against the packed keys directly (asymmetric
 *            estimator), softmax, and sum the dequantised values.
 *
 * Conventions shared by every call
 *  - Device pointers are caller-owned (allocated by the caller, e.g. PyTorch),
 *    must be 16-byte aligned, and are never freed by libtq.  libtq allocates
 *    device memory only inside tq_build_codebook and tq_make_rotation.
 *  - Calls that launch work are asynchronous on `stream` (a hipStream_t; NULL
 *    is the default stream) and return after the launch.  A device fault shows
 *    up at the caller's next synchronisation.
 *  - Every argument is validated before anything is launched.  On any status
 *    other than TQ_OK nothing was launched, and tq_last_error() returns a
 *    thread-local message.  Nothing throws across this interface.
 *  - Handles are immutable after creation and safe to share across streams;
 *    freeing a handle while a launch that uses it is in flight is an error of
 *    the caller.
 *  - Packed planes are laid out [B, Hkv, T, row] with rows contiguous in T.
 *    Bit-streams are LSB-first: element j of width w occupies bits
 *    [w*j, w*j + w) of the row read as little-endian bytes.
 *  - Grouped-query attention: query head hq reads KV head hq / (Hq / Hkv).
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TQ_OK = 0,
    TQ_EINVAL = 1,        /* an argument is out of range or inconsistent   */
    TQ_EUNSUPPORTED = 2,  /* a valid combination the library does not serve */
    TQ_EALIGN = 3,        /* a device pointer or stride is not 16-B aligned  */
    TQ_ENOMEM = 4,        /* handle allocation failed, or workspace too small*/
    TQ_EHIP = 5,          /* the HIP runtime reported an error                */
    TQ_ENOTCONV = 6       /* the codebook iteration did not converge          */
} tq_status;

typedef enum { TQ_ROT_DENSE = 0, TQ_ROT_HADAMARD = 1, TQ_ROT_HADAMARD2 = 2 } tq_rot_kind;
typedef enum { TQ_F32 = 0, TQ_BF16 = 1, TQ_F16 = 2 } tq_dtype;

typedef struct tq_codebook tq_codebook;   /* opaque, immutable */
typedef struct tq_rotation tq_rotation;   /* opaque, immutable */

/* Key format: d channels, mse_bits Lloyd-Max bits per coordinate, qjl_m sign
   rows, the codebook for (d, mse_bits) and the rotation (Pi and S) for d.
   qjl_m is d (both stages of the two-stage quantiser, "turboquant-pytorch",
   section "What it does") or 0: the first stage alone, no sign or residual
   norm planes, score n sum_j (Pi q)_j c[idx_j] (a biased estimate of <q, k>
   that reads fewer bytes per key). */
typedef struct {
    int d;
    int mse_bits;
    int qjl_m;
    const tq_codebook *cb;
    const tq_rotation *rot;
} tq_key_fmt;

/* Value format: d channels, bits per code (2 or 4), group size g (g | d,
   g in {32, 64, 128}). */
typedef struct {
    int d;
    int bits;
    int group;
} tq_val_fmt;

/* Packed key cache planes (device, caller-owned), per vector:
   codes d*mse_bits/8 B, signs qjl_m/8 B, knorm fp32 ||k||, rnorm fp32 ||r||.
   With qjl_m = 0 the signs and rnorm planes are empty (may be NULL). */
typedef struct {
    uint8_t *codes;
    uint8_t *signs;
    float *knorm;
    float *rnorm;
} tq_kcache;

/* Packed value cache planes (device, caller-owned), per vector:
   codes d*bits/8 B, params d/g pairs of fp16 bit patterns (scale, zero). */
typedef struct {
    uint8_t *codes;
    uint16_t *params;
} tq_vcache;

/* ------------------------------------------------------------------ setup */

/* Lloyd-Max codebook for one coordinate of a uniformly random unit vector in
   R^d, whose density is proportional to (1 - x^2)^((d-3)/2) on [-1, 1]
   ("turboquant-pytorch": build the optimal codebook with the Lloyd-Max
   quantizer for vector dimension d; discosf article step 2).  2^bits
   centroids, 2^bits - 1 boundaries (midpoints).  d in [3, 4096], bits in
   [1, 8].  Host work of a few ms; the tables are copied to the current device.
   *out receives a new handle; free it with tq_codebook_free. */
tq_status tq_build_codebook(int d, int bits, tq_codebook **out);
void tq_codebook_free(tq_codebook *cb);
/* fp64 tables of a handle: centroids[2^bits], boundaries[2^bits - 1] (host). */
tq_status tq_codebook_tables(const tq_codebook *cb, double *centroids, double *boundaries);
/* The same computation without any device: fills the host arrays. */
tq_status tq_codebook_host(int d, int bits, double *centroids, double *boundaries);

/* Random rotation Pi and QJL projection S (m = d rows, iid N(0,1)) from a seed
   ("turboquant-pytorch", random orthogonal rotations and QJL; discosf article
   steps 1 and 3).  TQ_ROT_DENSE: Haar-random orthogonal matrix, the Q factor
   of a Gaussian matrix with a positive-diagonal R.  TQ_ROT_HADAMARD:
   H D / sqrt(d), H the Sylvester Walsh-Hadamard matrix and D random signs (the
   O(d log d) rotation the tproger.ru article, section "Implementations",
   names); d must be a power of two.  TQ_ROT_HADAMARD2: two such rounds,
   Pi = (H D2 / sqrt(d)) (H D1 / sqrt(d)) = H D2 H D1 / d, the multi-round
   form that mixes more like a dense rotation at the same O(d log d) cost
   (D1 as in one round, D2 from its own stream).  Random numbers: SplitMix64
   counter generator, stream 0 = Gaussian matrix for Pi, 1 = signs of D (D1),
   2 = S, 3 = signs of D2;
   Box-Muller, row-major fill.  d in {64, 128, 256}.  Allocates device
   copies on the current device. */
tq_status tq_make_rotation(uint64_t seed, int d, tq_rot_kind kind, tq_rotation **out);
void tq_rotation_free(tq_rotation *rot);
/* Host-only: fp64 Pi [d*d] (y = Pi u, row-major) and S [d*d]; either may be
   NULL.  d in [2, 4096] (power of two for Hadamard). */
tq_status tq_rotation_host(uint64_t seed, int d, tq_rot_kind kind, double *pi, double *s);

/* Bytes of one plane for n_vec vectors.  Key planes: 0 codes, 1 signs,
   2 knorm, 3 rnorm (signs and rnorm are 0 bytes when qjl_m = 0).  Value
   planes: 0 codes, 1 params.  0 on a bad argument. */
size_t tq_key_plane_bytes(const tq_key_fmt *fmt, int64_t n_vec, int plane);
size_t tq_val_plane_bytes(const tq_val_fmt *fmt, int64_t n_vec, int plane);

/* -------------------------------------------------------------- hot path */

/* Compress keys k[B, Hkv, T, d] (element strides sb, sh, st; channel stride
   1; dtype f32/bf16/f16) into the planes of `out` (discosf article steps 1-3):
   n = ||k||, y = Pi k / n, idx_j = #{boundaries < y_j}, r = y - c[idx],
   sign_i = [(S r)_i >= 0], stored with fp32 n and fp32 ||r||.  A zero key
   stores n = 0 and the codes of y = 0.  Keys must be finite with ||k|| in
   (2^-60, 2^64): ||k||^2 is summed in fp32, and bf16 squares below 2^-126
   may be dropped.  T = 0 is a no-op.  Strides must be
   multiples of 16 bytes. */
tq_status tq_compress_keys(const tq_key_fmt *fmt, const void *k, tq_dtype dtype, int B, int Hkv,
                           int64_t T, int64_t sb, int64_t sh, int64_t st, tq_kcache out,
                           void *stream);

/* Compress values v[B, Hkv, T, d] (discosf article step 4): per token and
   group of g channels, fp16 scale = (max - min)/(2^bits - 1) and fp16 zero =
   min (round to nearest even), code = clamp(round_half_even((v - zero) /
   scale), 0, 2^bits - 1), or 0 when the scale is 0. */
tq_status tq_compress_values(const tq_val_fmt *fmt, const void *v, tq_dtype dtype, int B, int Hkv,
                             int64_t T, int64_t sb, int64_t sh, int64_t st, tq_vcache out,
                             void *stream);

/* Asymmetric scores of queries q[B, Hq, d] (contiguous) against the packed
   keys ("turboquant-pytorch": attention scores computed directly on the
   compressed keys):
     score_t = ||k_t|| ( sum_j (Pi q)_j c[idx_tj]
                         + sqrt(pi/2)/m ||r_t|| sum_i (S Pi q)_i (2 s_ti - 1) ).
   scores: device fp32 [B, Hq, T].  ws: device workspace of at least
   tq_scores_workspace_bytes() bytes.  (ws and ws_bytes extend the plain
   queries + packed keys -> scores call: the rotated query operands are built
   once per call into caller-owned memory, so that the call itself allocates
   nothing; a too-small ws returns TQ_ENOMEM before any launch.) */
size_t tq_scores_workspace_bytes(const tq_key_fmt *fmt, int B, int Hq);
tq_status tq_scores(const tq_key_fmt *fmt, const void *q, tq_dtype dtype, int B, int Hq, int Hkv,
                    int64_t T, tq_kcache kc, float *scores, void *ws, size_t ws_bytes,
                    void *stream);

/* Decode attention over the packed cache without dequantising the keys
   ("turboquant-pytorch", example requests: attention over the compressed
   cache without full key dequantisation):
     lambda_t = softmax_scale * score_t, p = softmax(lambda),
     out = sum_t p_t (code_t * scale + zero).
   softmax_scale 0 means 1/sqrt(d).  out: device fp32 [B, Hq, d].  T = 0
   writes zeros.  n_splits 0 picks the split count; otherwise the token axis
   is cut into n_splits ranges whose partial results are merged with a
   log-sum-exp combine.  ws: device workspace of at least
   tq_attend_workspace_bytes() bytes (same n_splits).  (n_splits, ws and
   ws_bytes extend the plain queries + packed K/V -> out call: the split count
   is exposed so that a caller can fix the work partition (identical results
   across calls, or a bounded workspace), and the query operands and split
   partials live in caller-owned memory so that the call allocates nothing.
   n_splits 0 and a workspace of the queried size give the plain call.) */
int tq_attend_splits(const tq_key_fmt *fmt, int B, int Hq, int Hkv, int64_t T);
size_t tq_attend_workspace_bytes(const tq_key_fmt *fmt, int B, int Hq, int Hkv, int64_t T,
                                 int n_splits);
tq_status tq_attend_decode(const tq_key_fmt *kfmt, const tq_val_fmt *vfmt, const void *q,
                           tq_dtype dtype, int B, int Hq, int Hkv, int64_t T, tq_kcache kc,
                           tq_vcache vc, float softmax_scale, int n_splits, void *ws,
                           size_t ws_bytes, float *out, void *stream);

/* tq_attend_decode without a workspace argument, for callers that cannot
   allocate device memory (code under HIP graph capture, serving loops or
   harnesses that forbid hipMalloc).  Same arguments, kernels, split plan and
   results as tq_attend_decode with the same n_splits; the workspace is a
   static device array of 16 MiB that the library holds on each GPU it runs
   on until the process ends (its address is looked up on the first call on
   a device).  The call allocates nothing and records no profiling events.
   Shapes whose workspace (tq_attend_workspace_bytes) exceeds 16 MiB return
   TQ_ENOMEM before anything is launched.  Every call on one GPU shares that
   GPU's array: calls that overlap on one GPU (several streams or host
   threads) race and give undefined results; calls ordered on one stream are
   safe.  Every workspace byte a call reads is written by that call first, so
   nothing left by a previous call needs clearing. */
tq_status tq_attend_decode_noalloc(const tq_key_fmt *kfmt, const tq_val_fmt *vfmt, const void *q,
                                   tq_dtype dtype, int B, int Hq, int Hkv, int64_t T, tq_kcache kc,
                                   tq_vcache vc, float softmax_scale, int n_splits, float *out,
                                   void *stream);

/* ------------------------------------------------- serving-style caches */

/* Layout of a preallocated cache that grows by a few tokens per decode step,
   with sequences of different lengths: the serving integration the pages
   describe (discosf.com article, section on known limitations: new K/V of
   each layer are captured into a paged cache; tproger.ru article, section
   "Implementations": TurboQuant as a KV-cache option of a serving engine).
     seq_lens     device int32 [B]: valid tokens of each sequence.
     block_table  NULL: contiguous planes [B, Hkv, capacity, row]; token t of
                  sequence b, KV head h is row (b * Hkv + h) * capacity + t.
                  Otherwise a device int32 [B, max_blocks] table into a pool of
                  num_blocks blocks of block_size tokens, planes
                  [num_blocks, Hkv, block_size, row]; token t lives in block
                  blk = block_table[b * max_blocks + t / block_size], row
                  (blk * Hkv + h) * block_size + t % block_size.
     capacity     tokens a sequence can hold (max_blocks * block_size when
                  paged).
   block_size is a power of two, at least 32.  The kernels read seq_lens and block_table
   on the device: a length is clamped to [0, capacity], and a token whose
   block id is outside [0, num_blocks) is skipped (not read, not written), so
   no access leaves the planes whatever the tables hold. */
typedef struct {
    int64_t capacity;
    const int32_t *seq_lens;
    const int32_t *block_table;
    int block_size;
    int max_blocks;
    int64_t num_blocks;
} tq_cache_layout;

/* Compress n_new new tokens per sequence, k[B, Hkv, n_new, d] (strides as in
   tq_compress_keys), into positions pos[b] .. pos[b] + n_new - 1 of sequence
   b of a layout cache (pos: device int32 [B], typically the lengths before
   the step; the layout's seq_lens are not read).  Positions outside
   [0, capacity) are skipped.  Each key is encoded exactly as by
   tq_compress_keys. */
tq_status tq_append_keys(const tq_key_fmt *fmt, const void *k, tq_dtype dtype, int B, int Hkv,
                         int n_new, int64_t sb, int64_t sh, int64_t st, const tq_cache_layout *lay,
                         const int32_t *pos, tq_kcache cache, void *stream);
tq_status tq_append_values(const tq_val_fmt *fmt, const void *v, tq_dtype dtype, int B, int Hkv,
                           int n_new, int64_t sb, int64_t sh, int64_t st, const tq_cache_layout *lay,
                           const int32_t *pos, tq_vcache cache, void *stream);

/* tq_attend_decode over a layout cache: sequence b attends its seq_lens[b]
   tokens (a sequence of length 0 gives zeros).  Split planning uses the
   capacity, and raises n_splits where needed so that a split spans at most
   511 blocks; ws: at least tq_attend_paged_workspace_bytes() bytes (same
   n_splits). */
size_t tq_attend_paged_workspace_bytes(const tq_key_fmt *fmt, int B, int Hq, int Hkv,
                                       const tq_cache_layout *lay, int n_splits);
tq_status tq_attend_decode_paged(const tq_key_fmt *kfmt, const tq_val_fmt *vfmt, const void *q,
                                 tq_dtype dtype, int B, int Hq, int Hkv, const tq_cache_layout *lay,
                                 tq_kcache kc, tq_vcache vc, float softmax_scale, int n_splits,
                                 void *ws, size_t ws_bytes, float *out, void *stream);

/* ------------------------------------- rotated block formats (comparison) */

/* Rotated scalar block key formats, the comparison the tproger.ru article
   reports (section "First benchmarks": Q8_0 and Q4_0 with rotation against
   the same formats without it).  The key is rotated, x = Pi k (the rotation
   handle's Pi, no normalisation), and every block of 32 consecutive rotated
   coordinates keeps one fp16 scale = fp16_rne(amax / qmax) (qmax 127 for
   bits = 8, 7 for bits = 4) and the signed codes
   q = clamp(round_half_even(x / scale), -qmax, qmax) (0 where scale = 0):
   one int8 byte each (bits 8) or q + 8 in 4 bits, LSB-first (bits 4).
   The score of a query is sum_j (Pi q)_j scale q_j.  d in {128, 256}. */
typedef struct {
    int d;
    int bits;                   /* 8 or 4 */
    const tq_rotation *rot;
} tq_block_fmt;

/* Planes (device, caller-owned), per vector: codes d*bits/8 B, scales d/32
   fp16 bit patterns. */
typedef struct {
    uint8_t *codes;
    uint16_t *scales;
} tq_bcache;

/* Bytes of one plane (0 codes, 1 scales) for n_vec vectors; 0 on a bad argument. */
size_t tq_block_plane_bytes(const tq_block_fmt *fmt, int64_t n_vec, int plane);
/* Compress keys k[B, Hkv, T, d] (strides as in tq_compress_keys).  The
   rotation is accumulated in fp64, so the codes are those of the exact
   rotated key but for ties. */
tq_status tq_compress_keys_block(const tq_block_fmt *fmt, const void *k, tq_dtype dtype, int B, int Hkv,
                                 int64_t T, int64_t sb, int64_t sh, int64_t st, tq_bcache out,
                                 void *stream);
/* Decode attention over block-format keys and the usual packed values, as
   tq_attend_decode. */
size_t tq_attend_block_workspace_bytes(const tq_block_fmt *fmt, int B, int Hq, int Hkv, int64_t T,
                                       int n_splits);
tq_status tq_attend_decode_block(const tq_block_fmt *kfmt, const tq_val_fmt *vfmt, const void *q,
                                 tq_dtype dtype, int B, int Hq, int Hkv, int64_t T, tq_bcache kc,
                                 tq_vcache vc, float softmax_scale, int n_splits, void *ws,
                                 size_t ws_bytes, float *out, void *stream);

/* Explicit key estimates of a packed cache (dequantisation), fp32
   out[B, Hkv, T, d] (contiguous, device):
     k_hat = ||k|| Pi^T ( c[idx] + sqrt(pi/2)/m ||r|| S^T (2 s - 1) ),
   the vector whose inner product with any query equals the score above
   ("turboquant-pytorch", section "What it does": the inverse of the
   two-stage encoding); with qjl_m = 0, k_hat = ||k|| Pi^T c[idx].  Not on the
   decode path, which never forms k_hat.  T = 0 is a no-op. */
tq_status tq_dequantize_keys(const tq_key_fmt *fmt, int B, int Hkv, int64_t T, tq_kcache kc,
                             float *out, void *stream);

/* ------------------------------------------------------------- utilities */

/* Thread-local message describing the last non-OK status of this thread. */
const char *tq_last_error(void);

/* Kernel timing for measurement.  While enabled, libtq records a pair of HIP
   events around every launch of its kernels on the launch stream.
   tq_profile_read synchronises on those events and returns, for kernels whose
   name contains `name`, the summed duration in ms and the launch count, then
   clears their records.  Off by default; enabling it adds two event records
   per launch. */
tq_status tq_profile_enable(int on);
tq_status tq_profile_read(const char *name, double *total_ms, int64_t *launches);

#ifdef __cplusplus
}
#endif
#endif /* TQ_H */

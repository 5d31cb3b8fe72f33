// C ABI of libtq: argument validation, handle lifetime, workspace carve-up and
// the launch of the HIP kernels.  Nothing here computes on the data path.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "tq_internal.h"

namespace {

thread_local std::string g_error;

// bf16 bits of a value, round to nearest even (finite inputs)
uint16_t bf16_rne(double x)
{
    const float f = static_cast<float>(x);
    uint32_t u;
    std::memcpy(&u, &f, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

double bf16_value(uint16_t h)
{
    const uint32_t u = static_cast<uint32_t>(h) << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

// split x into `parts` bf16 terms, each the rounding of what is left
void bf16_split(double x, int parts, uint16_t *out)
{
    for (int p = 0; p < parts; ++p) {
        out[p] = bf16_rne(x);
        x -= bf16_value(out[p]);
    }
}

// split x into `parts` fp16 terms, each the rounding (to nearest even) of what
// is left
void f16_split(double x, int parts, uint16_t *out)
{
    for (int p = 0; p < parts; ++p) {
        const _Float16 h = static_cast<_Float16>(x);
        std::memcpy(&out[p], &h, 2);
        x -= static_cast<double>(h);
    }
}

tq_status fail(tq_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
tq_status fail(tq_status st, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_error = buf;
    return st;
}

tq_status hip_fail(hipError_t e, const char *what)
{
    return fail(TQ_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The integer a C caller passed for an enum parameter.  C lets any int travel
// in an enum type; in C++ loading a value outside the enumerators' range is
// undefined, so arguments are read through their bytes and range-checked
// before they are used as the enum.
template <class E>
int enum_arg(const E &e)
{
    static_assert(sizeof(E) == sizeof(int), "C enums are int-sized here");
    int v;
    std::memcpy(&v, &e, sizeof v);
    return v;
}

// Failure injection for the failure-path tests, read from the environment
// variable TQ_TEST_HOOK at each set-up call and before each launch (unset in
// normal use):
//   "codebook_iters=N"  caps the Lloyd-Max sweeps and Newton steps at N
//                       (N = 0 leaves the start point: TQ_ENOTCONV)
//   "host_alloc"        the host allocation of a new handle fails (TQ_ENOMEM)
//   "launch"            an entry point that would launch kernels reports a
//                       launch failure (TQ_EHIP) after its argument checks,
//                       with nothing launched
struct TestHook {
    int codebook_iters = -1;
    bool host_alloc = false, launch = false;
};

TestHook test_hook()
{
    TestHook h;
    const char *s = std::getenv("TQ_TEST_HOOK");
    if (!s) return h;
    if (std::strncmp(s, "codebook_iters=", 15) == 0) h.codebook_iters = std::atoi(s + 15);
    h.host_alloc = std::strcmp(s, "host_alloc") == 0;
    h.launch = std::strcmp(s, "launch") == 0;
    return h;
}

size_t dtype_size(tq_dtype t)
{
    switch (t) {
    case TQ_F32: return 4;
    case TQ_BF16: return 2;
    case TQ_F16: return 2;
    }
    return 0;
}

bool supported_d(int d) { return d == 64 || d == 128 || d == 256; }

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// ---------------------------------------------------------------- profiling
struct ProfRecord {
    const char *name;
    hipEvent_t start, stop;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
thread_local bool g_prof_suppressed = false;
std::vector<ProfRecord> g_prof_live;
std::vector<ProfRecord> g_prof_free;

}  // namespace

namespace tq {

void prof_suppress(bool on) { g_prof_suppressed = on; }

void prof_begin(const char *name, hipStream_t stream, void **token)
{
    *token = nullptr;
    if (g_prof_suppressed) return;
    std::lock_guard<std::mutex> lock(g_prof_mu);
    if (!g_prof_on) return;
    ProfRecord r;
    if (!g_prof_free.empty()) {
        r = g_prof_free.back();
        g_prof_free.pop_back();
    } else {
        if (hipEventCreate(&r.start) != hipSuccess) return;
        if (hipEventCreate(&r.stop) != hipSuccess) return;
    }
    r.name = name;
    hipEventRecord(r.start, stream);
    g_prof_live.push_back(r);
    *token = reinterpret_cast<void *>(g_prof_live.size());   // 1-based index
}

void prof_end(void *token, hipStream_t stream)
{
    if (!token) return;
    std::lock_guard<std::mutex> lock(g_prof_mu);
    const size_t idx = reinterpret_cast<size_t>(token) - 1;
    if (idx < g_prof_live.size()) hipEventRecord(g_prof_live[idx].stop, stream);
}

}  // namespace tq

namespace {

// Coordinate that row R of the compressor's fragment tables (Pi, S) holds:
// wave w's row tile j, MFMA output row 4 kb + r takes coordinate
// (d / 16)(4 w + kb) + 4 j + r, so that each lane of the key kernel ends with
// d / 16 consecutive coordinates of a key (the natural order at d = 64).
int compressor_row(int d, int R)
{
    const int rtw = d / 64, rt = R / 16, rho = R % 16;
    const int w = rt / rtw, j = rt % rtw, kb = rho / 4, r = rho % 4;
    return (d / 16) * (4 * w + kb) + 4 * j + r;
}

}  // namespace

extern "C" {

const char *tq_last_error(void) { return g_error.c_str(); }

tq_status tq_profile_enable(int on)
{
    std::lock_guard<std::mutex> lock(g_prof_mu);
    g_prof_on = on != 0;
    return TQ_OK;
}

tq_status tq_profile_read(const char *name, double *total_ms, int64_t *launches)
{
    if (!name || !total_ms || !launches) return fail(TQ_EINVAL, "tq_profile_read: NULL argument");
    std::lock_guard<std::mutex> lock(g_prof_mu);
    double sum = 0.0;
    int64_t count = 0;
    std::vector<ProfRecord> keep;
    for (ProfRecord &r : g_prof_live) {
        if (std::strstr(r.name, name) == nullptr) {
            keep.push_back(r);
            continue;
        }
        hipError_t e = hipEventSynchronize(r.stop);
        if (e != hipSuccess) return hip_fail(e, "tq_profile_read: hipEventSynchronize");
        float ms = 0.0f;
        e = hipEventElapsedTime(&ms, r.start, r.stop);
        if (e != hipSuccess) return hip_fail(e, "tq_profile_read: hipEventElapsedTime");
        sum += ms;
        ++count;
        g_prof_free.push_back(r);
    }
    g_prof_live.swap(keep);
    *total_ms = sum;
    *launches = count;
    return TQ_OK;
}

// ------------------------------------------------------------------ codebook
tq_status tq_codebook_host(int d, int bits, double *centroids, double *boundaries)
{
    if (d < 3 || d > 4096) return fail(TQ_EINVAL, "codebook: d=%d outside [3, 4096]", d);
    if (bits < 1 || bits > 8) return fail(TQ_EINVAL, "codebook: bits=%d outside [1, 8]", bits);
    if (!centroids || !boundaries) return fail(TQ_EINVAL, "codebook: NULL output");
    double res = 0.0;
    const tq_status st = tq::lloyd_max_codebook(d, bits, centroids, boundaries, &res, test_hook().codebook_iters);
    if (st != TQ_OK) return fail(st, "codebook: Lloyd-Max residual %.3g after the iteration cap", res);
    return TQ_OK;
}

tq_status tq_build_codebook(int d, int bits, tq_codebook **out)
{
    if (!out) return fail(TQ_EINVAL, "tq_build_codebook: NULL out");
    *out = nullptr;
    auto *cb = test_hook().host_alloc ? nullptr : new (std::nothrow) tq_codebook;
    if (!cb) return fail(TQ_ENOMEM, "tq_build_codebook: host allocation failed");
    cb->d = d;
    cb->bits = bits;
    const int L = 1 << (bits < 1 ? 1 : bits > 8 ? 8 : bits);
    cb->centroids.assign(L, 0.0);
    cb->boundaries.assign(L - 1, 0.0);
    tq_status st = tq_codebook_host(d, bits, cb->centroids.data(), cb->boundaries.data());
    if (st != TQ_OK) {
        delete cb;
        return st;
    }
    std::vector<float> host(2 * L);
    for (int i = 0; i < L; ++i) host[i] = static_cast<float>(cb->centroids[i]);
    for (int i = 0; i < L - 1; ++i) host[L + i] = static_cast<float>(cb->boundaries[i]);
    host[2 * L - 1] = INFINITY;
    hipError_t e = hipGetDevice(&cb->device);
    if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void **>(&cb->d_centroids), sizeof(float) * 2 * L);
    if (e == hipSuccess)
        e = hipMemcpy(cb->d_centroids, host.data(), sizeof(float) * 2 * L, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        if (cb->d_centroids) hipFree(cb->d_centroids);
        delete cb;
        return hip_fail(e, "tq_build_codebook: device upload");
    }
    cb->d_boundaries = cb->d_centroids + L;
    if (L >= (1 << tq::kCellBits)) {
        // code cells over the fp32 boundaries the kernel compares with: the
        // coarsest uniform grid (from 64 cells, doubling) whose cells, widened by
        // 2 % of a cell on each side to absorb the rounding of the cell index,
        // hold at most one boundary each
        const double lo = host[L], hi = host[L + L - 2];
        std::vector<float4> cells;
        int ng = 0;
        for (int n = 64; n <= tq::kMaxGrid && ng == 0; n *= 2) {
            const double w = (hi - lo) / n;
            cells.assign(n, float4{});
            bool ok = true;
            for (int c = 0; c < n && ok; ++c) {
                const double a = lo + (c - 0.02) * w, b = lo + (c + 1.02) * w;
                int below = 0, inside = 0, first = -1;
                for (int i = 0; i < L - 1; ++i) {
                    if (host[L + i] < a) {
                        ++below;
                    } else if (host[L + i] < b) {
                        if (first < 0) first = i;
                        ++inside;
                    }
                }
                ok = inside <= 1;
                float4 &e = cells[c];
                e.x = inside ? host[L + first] : INFINITY;
                e.y = host[below];
                e.z = host[inside ? below + 1 : below];
                int32_t bw = below;
                std::memcpy(&e.w, &bw, sizeof(bw));
            }
            if (ok) ng = n;
        }
        if (ng == 0) {
            hipFree(cb->d_centroids);
            delete cb;
            return fail(TQ_EUNSUPPORTED, "tq_build_codebook: no code grid up to %d cells", tq::kMaxGrid);
        }
        cb->ngrid = ng;
        cb->grid_lo = static_cast<float>(lo);
        cb->grid_scale = static_cast<float>(ng / (hi - lo));
        e = hipMalloc(reinterpret_cast<void **>(&cb->d_grid), sizeof(float4) * ng);
        if (e == hipSuccess) e = hipMemcpy(cb->d_grid, cells.data(), sizeof(float4) * ng, hipMemcpyHostToDevice);
        if (e != hipSuccess) {
            if (cb->d_grid) hipFree(cb->d_grid);
            hipFree(cb->d_centroids);
            delete cb;
            return hip_fail(e, "tq_build_codebook: grid upload");
        }
    }
    *out = cb;
    return TQ_OK;
}

void tq_codebook_free(tq_codebook *cb)
{
    if (!cb) return;
    if (cb->d_centroids) hipFree(cb->d_centroids);
    if (cb->d_grid) hipFree(cb->d_grid);
    delete cb;
}

tq_status tq_codebook_tables(const tq_codebook *cb, double *centroids, double *boundaries)
{
    if (!cb || !centroids || !boundaries) return fail(TQ_EINVAL, "tq_codebook_tables: NULL argument");
    std::memcpy(centroids, cb->centroids.data(), sizeof(double) * cb->centroids.size());
    std::memcpy(boundaries, cb->boundaries.data(), sizeof(double) * cb->boundaries.size());
    return TQ_OK;
}

// ------------------------------------------------------------------ rotation
tq_status tq_rotation_host(uint64_t seed, int d, tq_rot_kind kind_arg, double *pi, double *s)
{
    if (d < 2 || d > 4096) return fail(TQ_EINVAL, "rotation: d=%d outside [2, 4096]", d);
    const int kv = enum_arg(kind_arg);
    if (kv != TQ_ROT_DENSE && kv != TQ_ROT_HADAMARD && kv != TQ_ROT_HADAMARD2)
        return fail(TQ_EINVAL, "rotation: bad kind %d", kv);
    const tq_rot_kind kind = static_cast<tq_rot_kind>(kv);
    if (kind != TQ_ROT_DENSE && (d & (d - 1)) != 0)
        return fail(TQ_EUNSUPPORTED, "rotation: Hadamard needs a power-of-two d, got %d", d);
    if (pi) {
        if (kind == TQ_ROT_DENSE) tq::dense_rotation(seed, d, pi);
        else if (kind == TQ_ROT_HADAMARD) tq::hadamard_rotation(seed, d, pi);
        else tq::hadamard2_rotation(seed, d, pi);
    }
    if (s) tq::qjl_projection(seed, d, d, s);
    return TQ_OK;
}

tq_status tq_make_rotation(uint64_t seed, int d, tq_rot_kind kind_arg, tq_rotation **out)
{
    if (!out) return fail(TQ_EINVAL, "tq_make_rotation: NULL out");
    *out = nullptr;
    if (!supported_d(d)) return fail(TQ_EUNSUPPORTED, "tq_make_rotation: d=%d not in {64, 128, 256}", d);
    const int kv = enum_arg(kind_arg);
    if (kv != TQ_ROT_DENSE && kv != TQ_ROT_HADAMARD && kv != TQ_ROT_HADAMARD2)
        return fail(TQ_EINVAL, "tq_make_rotation: bad kind %d", kv);
    const tq_rot_kind kind = static_cast<tq_rot_kind>(kv);
    const size_t dd = static_cast<size_t>(d) * d;
    std::vector<double> pi(dd), s(dd);
    tq_status st = tq_rotation_host(seed, d, kind, pi.data(), s.data());
    if (st != TQ_OK) return st;
    std::vector<float> host(5 * dd + 5 * d);
    for (int i = 0; i < d; ++i)
        for (int j = 0; j < d; ++j) {
            host[i * d + j] = static_cast<float>(pi[i * d + j]);            // Pi
            host[dd + j * d + i] = static_cast<float>(pi[i * d + j]);       // Pi^T
            host[2 * dd + i * d + j] = static_cast<float>(s[i * d + j]);    // S
            host[3 * dd + j * d + i] = static_cast<float>(s[i * d + j]);    // S^T
        }
    // (S Pi)^T in fp64, rounded once: Sq = S (Pi q) = (S Pi) q; with the
    // column sums of Pi and S Pi and the largest row norm of S Pi
    std::vector<double> pisum(d, 0.0), spisum(d, 0.0);
    double rmax = 0.0;
    for (int i = 0; i < d; ++i) {
        double r2 = 0.0;
        for (int j = 0; j < d; ++j) {
            double acc = 0.0;
            for (int k = 0; k < d; ++k) acc += s[static_cast<size_t>(i) * d + k] * pi[static_cast<size_t>(k) * d + j];
            host[4 * dd + static_cast<size_t>(j) * d + i] = static_cast<float>(acc);
            spisum[j] += acc;
            pisum[j] += pi[static_cast<size_t>(i) * d + j];
            r2 += acc * acc;
        }
        rmax = std::max(rmax, std::sqrt(r2));
    }
    for (int j = 0; j < d; ++j) {
        host[5 * dd + d + j] = static_cast<float>(pisum[j]);
        host[5 * dd + 2 * d + j] = static_cast<float>(spisum[j]);
    }
    if (kind == TQ_ROT_HADAMARD) tq::hadamard_signs(seed, d, host.data() + 5 * dd);
    else for (int j = 0; j < d; ++j) host[5 * dd + j] = 1.0f;
    // the sign vectors of the Walsh-Hadamard rounds (D1, then D2 of the second
    // round) for the butterfly compressor; ones where a round is absent
    for (int j = 0; j < 2 * d; ++j) host[5 * dd + 3 * d + j] = 1.0f;
    if (kind != TQ_ROT_DENSE) tq::hadamard_signs(seed, d, host.data() + 5 * dd + 3 * d, 1);
    if (kind == TQ_ROT_HADAMARD2) tq::hadamard_signs(seed, d, host.data() + 5 * dd + 4 * d, 3);
    auto *rot = test_hook().host_alloc ? nullptr : new (std::nothrow) tq_rotation;
    if (!rot) return fail(TQ_ENOMEM, "tq_make_rotation: host allocation failed");
    rot->seed = seed;
    rot->d = d;
    rot->m = d;
    rot->kind = kind;
    hipError_t e = hipGetDevice(&rot->device);
    if (e == hipSuccess) e = hipMalloc(&rot->d_block, sizeof(float) * host.size());
    if (e == hipSuccess) e = hipMemcpy(rot->d_block, host.data(), sizeof(float) * host.size(), hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        if (rot->d_block) hipFree(rot->d_block);
        delete rot;
        return hip_fail(e, "tq_make_rotation: device upload");
    }
    // operand fragments of the matrix-core compressor (rows in the order of
    // compressor_row): Pi as three bf16 terms for fp32 keys and the Hadamard
    // sign matrices
    // (about 24 significant bits, so y keeps fp32 accuracy), S as two (16 bits;
    // the residual is split in two as well, see the key kernel), and for 2-byte
    // keys of a dense rotation Pi 2^kPiHalfExp as two fp16 terms (22 bits)
    const int ks_n = d / 32, rt_n = d / 16;
    const size_t part_n = static_cast<size_t>(rt_n) * ks_n * 512;
    std::vector<uint16_t> frag(part_n * 7);
    uint16_t *pif = frag.data(), *sfr = frag.data() + part_n * 3, *pih = frag.data() + part_n * 5;
    for (int rt = 0; rt < rt_n; ++rt)
        for (int ks = 0; ks < ks_n; ++ks)
            for (int lane = 0; lane < 64; ++lane)
                for (int el = 0; el < 8; ++el) {
                    const int row = compressor_row(d, 16 * rt + lane % 16), kb = lane / 16;
                    uint16_t parts[3];
                    const double pv = pi[static_cast<size_t>(row) * d + 32 * ks + 8 * kb + el];
                    if (kind == TQ_ROT_HADAMARD) {
                        // the +-1 sign matrix H D, exact in one part; 1/sqrt(d) is applied in fp32
                        parts[0] = bf16_rne(pv > 0.0 ? 1.0 : -1.0);
                        parts[1] = parts[2] = 0;
                    } else if (kind == TQ_ROT_HADAMARD2) {
                        // H D2 H D1 has integer entries in [-d, d], exact in one bf16 part
                        // (|entry| <= 256); 1/d is applied in fp32
                        parts[0] = bf16_rne(std::nearbyint(pv * d));
                        parts[1] = parts[2] = 0;
                    } else {
                        bf16_split(pv, 3, parts);
                    }
                    for (int p = 0; p < 3; ++p) pif[(((rt * ks_n + ks) * 3 + p) * 64 + lane) * 8 + el] = parts[p];
                    uint16_t hparts[2] = {0, 0};
                    if (kind == TQ_ROT_DENSE) f16_split(std::ldexp(pv, tq::kPiHalfExp), 2, hparts);
                    for (int p = 0; p < 2; ++p) pih[(((rt * ks_n + ks) * 2 + p) * 64 + lane) * 8 + el] = hparts[p];
                    const int col = 16 * (2 * ks + el / 4) + 4 * kb + el % 4;
                    bf16_split(s[static_cast<size_t>(row) * d + col], 2, parts);
                    for (int p = 0; p < 2; ++p) sfr[(((rt * ks_n + ks) * 2 + p) * 64 + lane) * 8 + el] = parts[p];
                }
    e = hipMalloc(&rot->d_frag_block, sizeof(uint16_t) * frag.size());
    if (e == hipSuccess)
        e = hipMemcpy(rot->d_frag_block, frag.data(), sizeof(uint16_t) * frag.size(), hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        if (rot->d_frag_block) hipFree(rot->d_frag_block);
        hipFree(rot->d_block);
        delete rot;
        return hip_fail(e, "tq_make_rotation: fragment upload");
    }
    // fp64 Pi^T for the block-format compressor
    std::vector<double> pi64T(dd);
    for (int i = 0; i < d; ++i)
        for (int j = 0; j < d; ++j) pi64T[static_cast<size_t>(j) * d + i] = pi[static_cast<size_t>(i) * d + j];
    e = hipMalloc(&rot->d_pi64T, sizeof(double) * dd);
    if (e == hipSuccess) e = hipMemcpy(rot->d_pi64T, pi64T.data(), sizeof(double) * dd, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        if (rot->d_pi64T) hipFree(rot->d_pi64T);
        hipFree(rot->d_frag_block);
        hipFree(rot->d_block);
        delete rot;
        return hip_fail(e, "tq_make_rotation: fp64 upload");
    }
    rot->d_pifrag = static_cast<uint16_t *>(rot->d_frag_block);
    rot->d_sfrag = rot->d_pifrag + part_n * 3;
    rot->d_pihfrag = rot->d_pifrag + part_n * 5;
    float *base = static_cast<float *>(rot->d_block);
    rot->d_pi = base;
    rot->d_piT = base + dd;
    rot->d_s = base + 2 * dd;
    rot->d_sT = base + 3 * dd;
    rot->d_spiT = base + 4 * dd;
    rot->d_dsign = base + 5 * dd;
    rot->d_pisum = base + 5 * dd + d;
    rot->d_spisum = base + 5 * dd + 2 * d;
    rot->d_wht = base + 5 * dd + 3 * d;
    rot->sq_bound = static_cast<float>(rmax * (1.0 + 1e-6));
    *out = rot;
    return TQ_OK;
}

void tq_rotation_free(tq_rotation *rot)
{
    if (!rot) return;
    if (rot->d_block) hipFree(rot->d_block);
    if (rot->d_frag_block) hipFree(rot->d_frag_block);
    if (rot->d_pi64T) hipFree(rot->d_pi64T);
    delete rot;
}

// ------------------------------------------------------------------ sizes
size_t tq_key_plane_bytes(const tq_key_fmt *fmt, int64_t n_vec, int plane)
{
    if (!fmt || n_vec < 0 || fmt->d <= 0 || fmt->mse_bits <= 0 || fmt->qjl_m < 0) return 0;
    const size_t n = static_cast<size_t>(n_vec);
    switch (plane) {
    case 0: return n * ((static_cast<size_t>(fmt->d) * fmt->mse_bits + 7) / 8);
    case 1: return n * ((static_cast<size_t>(fmt->qjl_m) + 7) / 8);
    case 2: return n * sizeof(float);
    case 3: return fmt->qjl_m > 0 ? n * sizeof(float) : 0;
    }
    return 0;
}

size_t tq_val_plane_bytes(const tq_val_fmt *fmt, int64_t n_vec, int plane)
{
    if (!fmt || n_vec < 0 || fmt->d <= 0 || fmt->bits <= 0 || fmt->group <= 0 || fmt->d % fmt->group)
        return 0;
    const size_t n = static_cast<size_t>(n_vec);
    switch (plane) {
    case 0: return n * ((static_cast<size_t>(fmt->d) * fmt->bits + 7) / 8);
    case 1: return n * (static_cast<size_t>(fmt->d) / fmt->group) * 2 * sizeof(uint16_t);
    }
    return 0;
}

}  // extern "C"

namespace {

tq_status check_key_fmt(const tq_key_fmt *f, const char *who)
{
    if (!f) return fail(TQ_EINVAL, "%s: NULL key format", who);
    if (!f->cb || !f->rot) return fail(TQ_EINVAL, "%s: key format without codebook or rotation", who);
    if (!supported_d(f->d)) return fail(TQ_EUNSUPPORTED, "%s: d=%d not in {64, 128, 256}", who, f->d);
    if (f->mse_bits < 1 || f->mse_bits > 7)
        return fail(TQ_EUNSUPPORTED, "%s: mse_bits=%d not in [1, 7]", who, f->mse_bits);
    if (f->qjl_m != f->d && f->qjl_m != 0)
        return fail(TQ_EUNSUPPORTED, "%s: qjl_m=%d must be d=%d or 0", who, f->qjl_m, f->d);
    if (f->cb->d != f->d || f->cb->bits != f->mse_bits)
        return fail(TQ_EINVAL, "%s: codebook is for (d=%d, bits=%d), format wants (%d, %d)", who,
                    f->cb->d, f->cb->bits, f->d, f->mse_bits);
    if (f->rot->d != f->d || (f->qjl_m > 0 && f->rot->m != f->qjl_m))
        return fail(TQ_EINVAL, "%s: rotation is for d=%d, format wants %d", who, f->rot->d, f->d);
    return TQ_OK;
}

tq_status check_val_fmt(const tq_val_fmt *f, const char *who)
{
    if (!f) return fail(TQ_EINVAL, "%s: NULL value format", who);
    if (!supported_d(f->d)) return fail(TQ_EUNSUPPORTED, "%s: d=%d not in {64, 128, 256}", who, f->d);
    if (f->bits != 2 && f->bits != 4) return fail(TQ_EUNSUPPORTED, "%s: value bits=%d not in {2, 4}", who, f->bits);
    if (f->group != 32 && f->group != 64 && f->group != 128)
        return fail(TQ_EUNSUPPORTED, "%s: group=%d not in {32, 64, 128}", who, f->group);
    if (f->group > f->d || f->d % f->group) return fail(TQ_EINVAL, "%s: group=%d does not divide d=%d", who, f->group, f->d);
    return TQ_OK;
}

tq_status check_dtype(const tq_dtype &t, const char *who)
{
    const int v = enum_arg(t);
    if (v != TQ_F32 && v != TQ_BF16 && v != TQ_F16) return fail(TQ_EINVAL, "%s: bad dtype %d", who, v);
    return TQ_OK;
}

tq_status check_input(const void *x, tq_dtype dt, int B, int H, int64_t T, int64_t sb, int64_t sh,
                      int64_t st, int d, const char *who)
{
    if (B < 1 || H < 1 || T < 0) return fail(TQ_EINVAL, "%s: bad shape B=%d H=%d T=%lld", who, B, H, (long long)T);
    if (T > 0 && !x) return fail(TQ_EINVAL, "%s: NULL input", who);
    if (sb < 0 || sh < 0 || st < 0) return fail(TQ_EINVAL, "%s: negative stride", who);
    if (T > 0 && st < d) return fail(TQ_EINVAL, "%s: token stride %lld overlaps a %d-channel row", who, (long long)st, d);
    const size_t es = dtype_size(dt);
    if (!aligned16(x) || (sb * es) % 16 || (sh * es) % 16 || (st * es) % 16)
        return fail(TQ_EALIGN, "%s: input pointer and strides must be 16-byte aligned", who);
    if (static_cast<int64_t>(B) * H * T > (int64_t(1) << 40))
        return fail(TQ_EINVAL, "%s: too many vectors", who);
    return TQ_OK;
}

// the signs and rnorm planes exist only with QJL rows (m > 0)
tq_status check_kcache(const tq_kcache &kc, int m, const char *who)
{
    if (!kc.codes || !kc.knorm || (m > 0 && (!kc.signs || !kc.rnorm)))
        return fail(TQ_EINVAL, "%s: NULL key plane", who);
    if (!aligned16(kc.codes) || !aligned16(kc.knorm) || (m > 0 && (!aligned16(kc.signs) || !aligned16(kc.rnorm))))
        return fail(TQ_EALIGN, "%s: key planes must be 16-byte aligned", who);
    return TQ_OK;
}

tq_status check_vcache(const tq_vcache &vc, const char *who)
{
    if (!vc.codes || !vc.params) return fail(TQ_EINVAL, "%s: NULL value plane", who);
    if (!aligned16(vc.codes) || !aligned16(vc.params)) return fail(TQ_EALIGN, "%s: value planes must be 16-byte aligned", who);
    return TQ_OK;
}

#define TQ_TRY(expr)                         \
    do {                                     \
        const tq_status st_ = (expr);        \
        if (st_ != TQ_OK) return st_;        \
    } while (0)

// Implementation of the Walsh-Hadamard rotations in the key compressor
// (TQ_HADAMARD_KERNEL, read at each call): "butterfly" (default) runs the
// randomized butterfly in registers, "matrix" the +-1 sign matrix as one exact
// bf16 term on the matrix cores.  Both compute the same rotation; their
// roundings differ only in fp32 summation order.
bool hadamard_butterfly()
{
    const char *s = std::getenv("TQ_HADAMARD_KERNEL");
    return !(s && std::strcmp(s, "matrix") == 0);
}

// the "launch" test hook: report a launch failure where kernels would be launched
#define TQ_LAUNCH_HOOK(who)                                                       \
    do {                                                                          \
        if (test_hook().launch) return hip_fail(hipErrorLaunchFailure, (who));    \
    } while (0)

// Decode path and split count for a shape: the matrix-core path when the key
// format allows it, else the general kernel.
// the matrix-core kernels run the softmax in base 2: scores leave the score
// stage multiplied by scale log2(e)
constexpr float kLog2e = 1.4426950408889634f;

// compute units of the target GPU (MI355X) the decode plan fills
constexpr int64_t kDecodeCUs = 256;

struct DecodePlan {
    bool mfma = false;
    int gc = 0, nqc = 0, mt = 0, units = 0, splits = 0, steps = 0;
};

// paged_bs > 0: a paged cache with that block size, whose splits must each
// span at most kStageBlocks blocks (their ids are staged in LDS).
// scores_only: the plan of tq_scores, whose kernel (no value stage) fits at
// least two workgroups per CU at d = 256 as at d = 128 and writes raw scores
// per token (no merge), so it takes the d = 128 rule.
DecodePlan decode_plan(const tq_key_fmt *fmt, int B, int Hq, int Hkv, int64_t T, int n_splits, int paged_bs = 0,
                       bool scores_only = false)
{
    DecodePlan p;
    const int G = Hq / Hkv;
    p.mfma = tq::mfma_decode_supported(fmt->d, fmt->mse_bits, G, 2, 32);
    p.gc = p.mfma ? tq::mfma_query_chunk(G) : tq::query_chunk(G);
    const int tile = p.mfma ? tq::kMfmaTile : tq::kDecodeTile;
    const int64_t tiles = (T + tile - 1) / tile;
    // a grid too small to give every CU a workgroup even at one tile per split
    // (short caches with few KV heads): smaller query chunks, more units
    while (p.mfma && p.gc > 1 && static_cast<int64_t>(B) * Hkv * (G / p.gc) * tiles < 256) p.gc /= 2;
    p.nqc = G / p.gc;
    p.mt = p.mfma ? tq::mfma_row_tiles(fmt->mse_bits, p.gc) : (p.gc + 3) / 4;
    p.units = B * Hkv * p.nqc;
    p.steps = p.mfma ? tq::mfma_score_steps(fmt->d, fmt->mse_bits, fmt->qjl_m) : 0;
    // workgroups per launch: about eight per CU for the d = 128 matrix-core
    // kernels (short enough splits that the last round is cheap), four for the
    // scalar kernels; d = 256 below
    const int64_t target = p.mfma ? 2048 : 1024;
    int64_t want = (target + p.units - 1) / p.units;
    if (p.mfma && fmt->d >= 256 && !scores_only) {
        // the split count that minimises the rounds of workgroups times the
        // tokens of each (ties to fewer splits, which need no or a smaller
        // merge).  A round is one workgroup per CU, or two for the table-score
        // kernels of at most two query heads per unit (3+ bit keys), which fit
        // two per CU at d = 256 when the value groups allow their spread
        // operand; for value formats that do not, the extra splits only cost
        // the merge.
        const int64_t slots = kDecodeCUs * (fmt->mse_bits >= 3 && p.gc <= 2 ? 2 : 1);
        want = 1;
        double best = 1e300;
        const int64_t smax = std::max<int64_t>(16, 2 * ((slots + p.units - 1) / p.units));
        for (int64_t s = 1; s <= smax && s <= 1024; ++s) {
            const double rounds = static_cast<double>((p.units * s + slots - 1) / slots);
            const double cost = rounds / static_cast<double>(s) * (1.0 + 1e-3 * static_cast<double>(s));
            if (cost < best) {
                best = cost;
                want = s;
            }
        }
    }
    if (want > tiles) want = tiles;
    if (want > 1024) want = 1024;
    p.splits = n_splits > 0 ? n_splits : static_cast<int>(want < 1 ? 1 : want);
    if (paged_bs > 0 && p.mfma) {
        const int64_t max_tiles = static_cast<int64_t>(tq::kStageBlocks - 1) * paged_bs / tile;
        const int64_t need = (tiles + max_tiles - 1) / max_tiles;
        if (p.splits < need) p.splits = static_cast<int>(need);
    }
    return p;
}

struct AttendLayout {
    size_t qprep, aops, qscal, qaux, ml, acc, total;
};

// d channels, m QJL rows (0 for the block formats)
AttendLayout attend_layout(int d, int m, int B, int Hq, const DecodePlan &p)
{
    AttendLayout L;
    const size_t rows = static_cast<size_t>(B) * Hq;
    size_t off = 0;
    L.qprep = off;
    off += align256(rows * (d + m) * sizeof(float));
    L.aops = off;
    off += align256(static_cast<size_t>(p.units) * p.mt * p.steps * 64 * 16);
    L.qscal = off;
    off += align256(rows * 4 * sizeof(float));
    L.qaux = off;
    off += align256(rows * (d / 32) * sizeof(float));
    L.ml = off;
    off += align256(rows * p.splits * 2 * sizeof(float));
    L.acc = off;
    off += align256(rows * p.splits * d * sizeof(float));
    L.total = off;
    return L;
}

// A layout cache (tq_cache_layout) as the kernels' row map; seq_lens are
// required for decode, pos for appends.
tq_status layout_map(const tq_cache_layout *lay, const int32_t *pos, bool decode, const char *who, tq::CacheMap &m)
{
    if (!lay) return fail(TQ_EINVAL, "%s: NULL cache layout", who);
    if (lay->capacity < 1 || lay->capacity > (int64_t(1) << 31))
        return fail(TQ_EINVAL, "%s: capacity %lld outside [1, 2^31]", who, (long long)lay->capacity);
    auto al4 = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; };
    if (decode && (!lay->seq_lens || !al4(lay->seq_lens)))
        return fail(TQ_EINVAL, "%s: seq_lens must be a 4-byte aligned device array", who);
    if (!decode && (!pos || !al4(pos))) return fail(TQ_EINVAL, "%s: pos must be a 4-byte aligned device array", who);
    m = tq::CacheMap{};
    m.cap = lay->capacity;
    m.seq_lens = lay->seq_lens;
    m.pos = pos;
    if (lay->block_table) {
        if (!al4(lay->block_table)) return fail(TQ_EINVAL, "%s: block_table must be 4-byte aligned", who);
        if (lay->block_size < 32 || (lay->block_size & (lay->block_size - 1)))
            return fail(TQ_EUNSUPPORTED, "%s: block_size=%d is not a power of two >= 32", who, lay->block_size);
        if (lay->max_blocks < 1 || lay->num_blocks < 1)
            return fail(TQ_EINVAL, "%s: max_blocks=%d, num_blocks=%lld", who, lay->max_blocks, (long long)lay->num_blocks);
        if (static_cast<int64_t>(lay->max_blocks) * lay->block_size != lay->capacity)
            return fail(TQ_EINVAL, "%s: capacity %lld != max_blocks * block_size", who, (long long)lay->capacity);
        m.mode = tq::CacheMap::kPaged;
        m.bt = lay->block_table;
        m.bs = lay->block_size;
        m.maxb = lay->max_blocks;
        m.nblocks = lay->num_blocks;
    } else {
        m.mode = tq::CacheMap::kContig;
    }
    return TQ_OK;
}

tq_status compress_keys_impl(const tq_key_fmt *fmt, const void *k, const tq_dtype &dtype, int B, int Hkv, int64_t T,
                             int64_t sb, int64_t sh, int64_t st, tq_kcache out, const tq::CacheMap &map,
                             void *stream, const char *who)
{
    TQ_TRY(check_key_fmt(fmt, who));
    TQ_TRY(check_dtype(dtype, who));
    TQ_TRY(check_input(k, dtype, B, Hkv, T, sb, sh, st, fmt->d, who));
    if (T == 0) return TQ_OK;
    TQ_TRY(check_kcache(out, fmt->qjl_m, who));
    if (fmt->mse_bits >= tq::kCellBits && fmt->cb->ngrid > tq::kGridLds)
        return fail(TQ_EUNSUPPORTED, "%s: codebook grid of %d cells exceeds the compressor's %d", who,
                    fmt->cb->ngrid, tq::kGridLds);
    tq::KeyLaunch a{};
    a.k = k;
    a.dtype = dtype;
    a.B = B;
    a.H = Hkv;
    a.T = T;
    a.sb = sb;
    a.sh = sh;
    a.st = st;
    a.contig = st == fmt->d && sh == T * fmt->d && sb == static_cast<int64_t>(Hkv) * T * fmt->d;
    a.d = fmt->d;
    a.bits = fmt->mse_bits;
    a.m = fmt->qjl_m;
    a.hadamard = fmt->rot->kind != TQ_ROT_DENSE;
    a.rot_scale = fmt->rot->kind == TQ_ROT_HADAMARD2 ? 1.0f / fmt->d
                : fmt->rot->kind == TQ_ROT_HADAMARD ? static_cast<float>(1.0 / std::sqrt(double(fmt->d))) : 1.0f;
    a.inv_rot_scale = fmt->rot->kind == TQ_ROT_HADAMARD2 ? static_cast<float>(fmt->d)
                    : fmt->rot->kind == TQ_ROT_HADAMARD ? static_cast<float>(std::sqrt(double(fmt->d))) : 1.0f;
    a.piT = fmt->rot->d_piT;
    a.sT = fmt->rot->d_sT;
    a.dsign = fmt->rot->d_dsign;
    a.wht = fmt->rot->d_wht;
    a.wht_rounds = fmt->rot->kind == TQ_ROT_HADAMARD2 ? 2 : fmt->rot->kind == TQ_ROT_HADAMARD ? 1 : 0;
    a.wht_kernel = hadamard_butterfly();
    a.centroids = fmt->cb->d_centroids;
    a.boundaries = fmt->cb->d_boundaries;
    a.grid = fmt->cb->d_grid;
    a.ngrid = fmt->cb->ngrid;
    a.grid_lo = fmt->cb->grid_lo;
    a.grid_scale = fmt->cb->grid_scale;
    a.grid_off = static_cast<float>(-static_cast<double>(fmt->cb->grid_lo) * fmt->cb->grid_scale);
    a.grid_max = static_cast<float>(fmt->cb->ngrid > 0 ? fmt->cb->ngrid - 1 : 0);
    a.pifrag = fmt->rot->d_pifrag;
    a.sfrag = fmt->rot->d_sfrag;
    a.pihfrag = fmt->rot->d_pihfrag;
    a.out = out;
    a.map = map;
    TQ_LAUNCH_HOOK(who);
    const hipError_t e = tq::launch_compress_keys(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TQ_OK : hip_fail(e, who);
}

tq_status compress_values_impl(const tq_val_fmt *fmt, const void *v, const tq_dtype &dtype, int B, int Hkv, int64_t T,
                               int64_t sb, int64_t sh, int64_t st, tq_vcache out, const tq::CacheMap &map,
                               void *stream, const char *who)
{
    TQ_TRY(check_val_fmt(fmt, who));
    TQ_TRY(check_dtype(dtype, who));
    TQ_TRY(check_input(v, dtype, B, Hkv, T, sb, sh, st, fmt->d, who));
    if (T == 0) return TQ_OK;
    TQ_TRY(check_vcache(out, who));
    tq::ValueLaunch a{};
    a.v = v;
    a.dtype = dtype;
    a.B = B;
    a.H = Hkv;
    a.T = T;
    a.sb = sb;
    a.sh = sh;
    a.st = st;
    a.d = fmt->d;
    a.bits = fmt->bits;
    a.group = fmt->group;
    a.out = out;
    a.map = map;
    TQ_LAUNCH_HOOK(who);
    const hipError_t e = tq::launch_compress_values(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TQ_OK : hip_fail(e, who);
}

}  // namespace

extern "C" {

tq_status tq_compress_keys(const tq_key_fmt *fmt, const void *k, tq_dtype dtype, int B, int Hkv,
                           int64_t T, int64_t sb, int64_t sh, int64_t st, tq_kcache out, void *stream)
{
    return compress_keys_impl(fmt, k, dtype, B, Hkv, T, sb, sh, st, out, tq::CacheMap{}, stream, "tq_compress_keys");
}

tq_status tq_compress_values(const tq_val_fmt *fmt, const void *v, tq_dtype dtype, int B, int Hkv,
                             int64_t T, int64_t sb, int64_t sh, int64_t st, tq_vcache out, void *stream)
{
    return compress_values_impl(fmt, v, dtype, B, Hkv, T, sb, sh, st, out, tq::CacheMap{}, stream,
                                "tq_compress_values");
}

tq_status tq_append_keys(const tq_key_fmt *fmt, const void *k, tq_dtype dtype, int B, int Hkv, int n_new,
                         int64_t sb, int64_t sh, int64_t st, const tq_cache_layout *lay, const int32_t *pos,
                         tq_kcache cache, void *stream)
{
    const char *who = "tq_append_keys";
    tq::CacheMap m;
    TQ_TRY(layout_map(lay, pos, false, who, m));
    return compress_keys_impl(fmt, k, dtype, B, Hkv, n_new, sb, sh, st, cache, m, stream, who);
}

tq_status tq_append_values(const tq_val_fmt *fmt, const void *v, tq_dtype dtype, int B, int Hkv, int n_new,
                           int64_t sb, int64_t sh, int64_t st, const tq_cache_layout *lay, const int32_t *pos,
                           tq_vcache cache, void *stream)
{
    const char *who = "tq_append_values";
    tq::CacheMap m;
    TQ_TRY(layout_map(lay, pos, false, who, m));
    return compress_values_impl(fmt, v, dtype, B, Hkv, n_new, sb, sh, st, cache, m, stream, who);
}

static tq_status check_decode_common(const tq_key_fmt *fmt, const void *q, const tq_dtype &dtype, int B, int Hq,
                                     int Hkv, int64_t T, const tq_kcache &kc, const char *who)
{
    TQ_TRY(check_key_fmt(fmt, who));
    TQ_TRY(check_dtype(dtype, who));
    if (B < 1 || Hq < 1 || Hkv < 1 || T < 0) return fail(TQ_EINVAL, "%s: bad shape", who);
    if (Hq % Hkv) return fail(TQ_EINVAL, "%s: Hq=%d is not a multiple of Hkv=%d", who, Hq, Hkv);
    if (!q) return fail(TQ_EINVAL, "%s: NULL query", who);
    if (!aligned16(q)) return fail(TQ_EALIGN, "%s: query must be 16-byte aligned", who);
    if (static_cast<int64_t>(B) * Hkv * T > (int64_t(1) << 40)) return fail(TQ_EINVAL, "%s: too many keys", who);
    if (T > 0) TQ_TRY(check_kcache(kc, fmt->qjl_m, who));
    return TQ_OK;
}

size_t tq_scores_workspace_bytes(const tq_key_fmt *fmt, int B, int Hq)
{
    if (!fmt || B < 1 || Hq < 1) return 0;
    const size_t rows = static_cast<size_t>(B) * Hq;
    // the scalar kernel: the prepared queries; the matrix-core kernel also the
    // score operands of every unit (units * row tiles <= B * Hq for any GQA
    // group) and the per-query scales
    const size_t scalar = align256(rows * (fmt->d + fmt->qjl_m) * sizeof(float));
    const int steps = tq::mfma_score_steps(fmt->d, fmt->mse_bits, fmt->qjl_m);
    const size_t mfma = scalar + align256(rows * steps * 64 * 16) + align256(rows * 4 * sizeof(float));
    return mfma > scalar ? mfma : scalar;
}

tq_status tq_scores(const tq_key_fmt *fmt, const void *q, tq_dtype dtype, int B, int Hq, int Hkv,
                    int64_t T, tq_kcache kc, float *scores, void *ws, size_t ws_bytes, void *stream)
{
    const char *who = "tq_scores";
    TQ_TRY(check_decode_common(fmt, q, dtype, B, Hq, Hkv, T, kc, who));
    if (T == 0) return TQ_OK;
    if (!scores || !ws) return fail(TQ_EINVAL, "%s: NULL scores or workspace", who);
    if (!aligned16(scores) || !aligned16(ws)) return fail(TQ_EALIGN, "%s: scores/workspace must be 16-byte aligned", who);
    const size_t need = tq_scores_workspace_bytes(fmt, B, Hq);
    if (ws_bytes < need) return fail(TQ_ENOMEM, "%s: workspace %zu B < %zu B", who, ws_bytes, need);
    tq::DecodeLaunch a{};
    a.q = q;
    a.dtype = dtype;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.T = T;
    a.d = fmt->d;
    a.bits = fmt->mse_bits;
    a.m = fmt->qjl_m;
    a.piT = fmt->rot->d_piT;
    a.sT = fmt->rot->d_sT;
    a.spiT = fmt->rot->d_spiT;
    a.pisum = fmt->rot->d_pisum;
    a.spisum = fmt->rot->d_spisum;
    a.sq_bound = fmt->rot->sq_bound;
    a.centroids = fmt->cb->d_centroids;
    a.kc = kc;
    a.scores = scores;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const DecodePlan plan = decode_plan(fmt, B, Hq, Hkv, T, 0, 0, true);
    if (plan.mfma) {
        // the matrix-core decode kernel with its value and softmax stages
        // compiled out: same tiles, same score products, raw scores out
        const AttendLayout L = attend_layout(fmt->d, fmt->qjl_m, B, Hq, plan);
        char *base = static_cast<char *>(ws);
        a.qprep = reinterpret_cast<float *>(base + L.qprep);
        a.splits = plan.splits;
        a.mf.gc = plan.gc;
        a.mf.nqc = plan.nqc;
        a.mf.mt = plan.mt;
        a.mf.units = plan.units;
        a.mf.aops = reinterpret_cast<uint32_t *>(base + L.aops);
        a.mf.qscal = reinterpret_cast<float *>(base + L.qscal);
        a.mf.lscale = 1.0f;
        TQ_LAUNCH_HOOK(who);
        const hipError_t e = tq::launch_scores_mfma(a, s);
        return e == hipSuccess ? TQ_OK : hip_fail(e, who);
    }
    a.qprep = static_cast<float *>(ws);
    TQ_LAUNCH_HOOK(who);
    hipError_t e = tq::launch_qprep(a, s);
    if (e == hipSuccess) e = tq::launch_scores(a, s);
    return e == hipSuccess ? TQ_OK : hip_fail(e, who);
}

}  // extern "C"

namespace {

tq_status check_block_fmt(const tq_block_fmt *f, const char *who)
{
    if (!f) return fail(TQ_EINVAL, "%s: NULL block format", who);
    if (!f->rot) return fail(TQ_EINVAL, "%s: block format without rotation", who);
    if (f->d != 128 && f->d != 256) return fail(TQ_EUNSUPPORTED, "%s: d=%d not in {128, 256}", who, f->d);
    if (f->bits != 8 && f->bits != 4) return fail(TQ_EUNSUPPORTED, "%s: bits=%d not in {4, 8}", who, f->bits);
    if (f->rot->d != f->d) return fail(TQ_EINVAL, "%s: rotation is for d=%d, format wants %d", who, f->rot->d, f->d);
    return TQ_OK;
}

tq_status check_bcache(const tq_bcache &c, const char *who)
{
    if (!c.codes || !c.scales) return fail(TQ_EINVAL, "%s: NULL block plane", who);
    if (!aligned16(c.codes) || !aligned16(c.scales)) return fail(TQ_EALIGN, "%s: block planes must be 16-byte aligned", who);
    return TQ_OK;
}

DecodePlan block_plan(int d, int B, int Hq, int Hkv, int64_t T, int n_splits)
{
    DecodePlan p;
    const int G = Hq / Hkv;
    p.mfma = true;
    p.gc = tq::mfma_query_chunk(G);
    p.nqc = G / p.gc;
    p.mt = (p.gc + 3) / 4;
    p.units = B * Hkv * p.nqc;
    p.steps = d / 64;                      // 16-byte operand slots per row tile (two blocks each)
    const int64_t tiles = (T + tq::kMfmaTile - 1) / tq::kMfmaTile;
    const int64_t target = d >= 256 ? 512 : 2048;
    int64_t want = (target + p.units - 1) / p.units;
    if (want > tiles) want = tiles;
    if (want > 1024) want = 1024;
    p.splits = n_splits > 0 ? n_splits : static_cast<int>(want < 1 ? 1 : want);
    return p;
}

}  // namespace

extern "C" {

size_t tq_block_plane_bytes(const tq_block_fmt *fmt, int64_t n_vec, int plane)
{
    if (!fmt || n_vec < 0 || fmt->d <= 0 || fmt->d % 32 || (fmt->bits != 8 && fmt->bits != 4)) return 0;
    const size_t n = static_cast<size_t>(n_vec);
    switch (plane) {
    case 0: return n * (static_cast<size_t>(fmt->d) * fmt->bits / 8);
    case 1: return n * (static_cast<size_t>(fmt->d) / 32) * sizeof(uint16_t);
    }
    return 0;
}

tq_status tq_compress_keys_block(const tq_block_fmt *fmt, const void *k, tq_dtype dtype, int B, int Hkv, int64_t T,
                                 int64_t sb, int64_t sh, int64_t st, tq_bcache out, void *stream)
{
    const char *who = "tq_compress_keys_block";
    TQ_TRY(check_block_fmt(fmt, who));
    TQ_TRY(check_dtype(dtype, who));
    TQ_TRY(check_input(k, dtype, B, Hkv, T, sb, sh, st, fmt->d, who));
    if (T == 0) return TQ_OK;
    TQ_TRY(check_bcache(out, who));
    tq::BlockLaunch a{};
    a.k = k;
    a.dtype = dtype;
    a.B = B;
    a.H = Hkv;
    a.T = T;
    a.sb = sb;
    a.sh = sh;
    a.st = st;
    a.d = fmt->d;
    a.bits = fmt->bits;
    a.pi64T = fmt->rot->d_pi64T;
    a.out = out;
    TQ_LAUNCH_HOOK(who);
    const hipError_t e = tq::launch_compress_keys_block(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TQ_OK : hip_fail(e, who);
}

size_t tq_attend_block_workspace_bytes(const tq_block_fmt *fmt, int B, int Hq, int Hkv, int64_t T, int n_splits)
{
    if (!fmt || B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || T < 0) return 0;
    return attend_layout(fmt->d, 0, B, Hq, block_plan(fmt->d, B, Hq, Hkv, T, n_splits)).total;
}

tq_status tq_attend_decode_block(const tq_block_fmt *kfmt, const tq_val_fmt *vfmt, const void *q, tq_dtype dtype,
                                 int B, int Hq, int Hkv, int64_t T, tq_bcache kc, tq_vcache vc, float softmax_scale,
                                 int n_splits, void *ws, size_t ws_bytes, float *out, void *stream)
{
    const char *who = "tq_attend_decode_block";
    TQ_TRY(check_block_fmt(kfmt, who));
    TQ_TRY(check_dtype(dtype, who));
    TQ_TRY(check_val_fmt(vfmt, who));
    if (B < 1 || Hq < 1 || Hkv < 1 || T < 0) return fail(TQ_EINVAL, "%s: bad shape", who);
    if (Hq % Hkv) return fail(TQ_EINVAL, "%s: Hq=%d is not a multiple of Hkv=%d", who, Hq, Hkv);
    if (static_cast<int64_t>(B) * Hkv * T > (int64_t(1) << 40)) return fail(TQ_EINVAL, "%s: too many keys", who);
    if (vfmt->d != kfmt->d) return fail(TQ_EINVAL, "%s: key d=%d and value d=%d differ", who, kfmt->d, vfmt->d);
    if (!q || !out) return fail(TQ_EINVAL, "%s: NULL query or output", who);
    if (!aligned16(q) || !aligned16(out)) return fail(TQ_EALIGN, "%s: query and output must be 16-byte aligned", who);
    if (n_splits < 0 || n_splits > 65535) return fail(TQ_EINVAL, "%s: n_splits=%d outside [0, 65535]", who, n_splits);
    if (!(softmax_scale >= 0.0f) || !std::isfinite(softmax_scale))
        return fail(TQ_EINVAL, "%s: softmax_scale must be finite and >= 0", who);
    tq::DecodeLaunch a{};
    a.q = q;
    a.dtype = dtype;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.T = T;
    a.d = kfmt->d;
    a.bits = kfmt->bits;
    a.m = 0;
    a.out = out;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (T == 0) {
        TQ_LAUNCH_HOOK(who);
        const hipError_t e = tq::launch_attend(a, s);
        return e == hipSuccess ? TQ_OK : hip_fail(e, who);
    }
    TQ_TRY(check_bcache(kc, who));
    TQ_TRY(check_vcache(vc, who));
    if (!ws) return fail(TQ_EINVAL, "%s: NULL workspace", who);
    if (!aligned16(ws)) return fail(TQ_EALIGN, "%s: workspace must be 16-byte aligned", who);
    const DecodePlan plan = block_plan(kfmt->d, B, Hq, Hkv, T, n_splits);
    const AttendLayout L = attend_layout(kfmt->d, 0, B, Hq, plan);
    if (ws_bytes < L.total) return fail(TQ_ENOMEM, "%s: workspace %zu B < %zu B", who, ws_bytes, L.total);
    a.piT = kfmt->rot->d_piT;
    a.spiT = kfmt->rot->d_spiT;
    a.pisum = kfmt->rot->d_pisum;
    a.spisum = kfmt->rot->d_spisum;
    a.sq_bound = kfmt->rot->sq_bound;
    a.kfmt_block = true;
    a.kq = kc;
    a.vbits = vfmt->bits;
    a.group = vfmt->group;
    a.vc = vc;
    a.scale = softmax_scale > 0.0f ? softmax_scale : static_cast<float>(1.0 / std::sqrt(double(kfmt->d)));
    a.splits = plan.splits;
    char *base = static_cast<char *>(ws);
    a.qprep = reinterpret_cast<float *>(base + L.qprep);
    a.part_ml = reinterpret_cast<float *>(base + L.ml);
    a.part_acc = reinterpret_cast<float *>(base + L.acc);
    a.mf.gc = plan.gc;
    a.mf.nqc = plan.nqc;
    a.mf.mt = plan.mt;
    a.mf.units = plan.units;
    a.mf.aops = reinterpret_cast<uint32_t *>(base + L.aops);
    a.mf.qscal = reinterpret_cast<float *>(base + L.qscal);
    a.qaux = reinterpret_cast<float *>(base + L.qaux);
    a.mf.lscale = a.scale * kLog2e;
    TQ_LAUNCH_HOOK(who);
    const hipError_t e = tq::launch_decode_block(a, s);
    return e == hipSuccess ? TQ_OK : hip_fail(e, who);
}

tq_status tq_dequantize_keys(const tq_key_fmt *fmt, int B, int Hkv, int64_t T, tq_kcache kc, float *out,
                             void *stream)
{
    const char *who = "tq_dequantize_keys";
    TQ_TRY(check_key_fmt(fmt, who));
    if (B < 1 || Hkv < 1 || T < 0) return fail(TQ_EINVAL, "%s: bad shape B=%d Hkv=%d T=%lld", who, B, Hkv, (long long)T);
    if (static_cast<int64_t>(B) * Hkv * T > (int64_t(1) << 40)) return fail(TQ_EINVAL, "%s: too many keys", who);
    if (T == 0) return TQ_OK;
    TQ_TRY(check_kcache(kc, fmt->qjl_m, who));
    if (!out) return fail(TQ_EINVAL, "%s: NULL output", who);
    if (!aligned16(out)) return fail(TQ_EALIGN, "%s: output must be 16-byte aligned", who);
    tq::DequantLaunch a{};
    a.N = static_cast<int64_t>(B) * Hkv * T;
    a.d = fmt->d;
    a.bits = fmt->mse_bits;
    a.m = fmt->qjl_m;
    a.kappa = a.m > 0 ? static_cast<float>(std::sqrt(M_PI / 2.0) / a.m) : 0.0f;
    a.pi = fmt->rot->d_pi;
    a.s = fmt->rot->d_s;
    a.centroids = fmt->cb->d_centroids;
    a.codes = kc.codes;
    a.signs = kc.signs;
    a.knorm = kc.knorm;
    a.rnorm = kc.rnorm;
    a.out = out;
    TQ_LAUNCH_HOOK(who);
    const hipError_t e = tq::launch_dequant_keys(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TQ_OK : hip_fail(e, who);
}

int tq_attend_splits(const tq_key_fmt *fmt, int B, int Hq, int Hkv, int64_t T)
{
    if (!fmt || B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || T < 0) return 0;
    return decode_plan(fmt, B, Hq, Hkv, T, 0).splits;
}

size_t tq_attend_workspace_bytes(const tq_key_fmt *fmt, int B, int Hq, int Hkv, int64_t T, int n_splits)
{
    if (!fmt || B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || T < 0) return 0;
    const DecodePlan p = decode_plan(fmt, B, Hq, Hkv, T, n_splits);
    return attend_layout(fmt->d, fmt->qjl_m, B, Hq, p).total;
}

size_t tq_attend_paged_workspace_bytes(const tq_key_fmt *fmt, int B, int Hq, int Hkv, const tq_cache_layout *lay,
                                       int n_splits)
{
    if (!fmt || !lay || lay->capacity < 1 || B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv) return 0;
    const DecodePlan p = decode_plan(fmt, B, Hq, Hkv, lay->capacity, n_splits, lay->block_table ? lay->block_size : 0);
    return attend_layout(fmt->d, fmt->qjl_m, B, Hq, p).total;
}

// decode attention over T tokens per sequence (flat map) or over a layout
// cache with T = its capacity
static tq_status attend_impl(const tq_key_fmt *kfmt, const tq_val_fmt *vfmt, const void *q, const tq_dtype &dtype, int B,
                             int Hq, int Hkv, int64_t T, tq_kcache kc, tq_vcache vc, float softmax_scale,
                             int n_splits, void *ws, size_t ws_bytes, float *out, const tq::CacheMap &map,
                             void *stream, const char *who, bool use_scratch = false)
{
    TQ_TRY(check_decode_common(kfmt, q, dtype, B, Hq, Hkv, T, kc, who));
    TQ_TRY(check_val_fmt(vfmt, who));
    if (vfmt->d != kfmt->d) return fail(TQ_EINVAL, "%s: key d=%d and value d=%d differ", who, kfmt->d, vfmt->d);
    if (!out) return fail(TQ_EINVAL, "%s: NULL output", who);
    if (!aligned16(out)) return fail(TQ_EALIGN, "%s: output must be 16-byte aligned", who);
    if (n_splits < 0 || n_splits > 65535) return fail(TQ_EINVAL, "%s: n_splits=%d outside [0, 65535]", who, n_splits);
    if (!(softmax_scale >= 0.0f) || !std::isfinite(softmax_scale))
        return fail(TQ_EINVAL, "%s: softmax_scale must be finite and >= 0", who);
    tq::DecodeLaunch a{};
    a.q = q;
    a.dtype = dtype;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.T = T;
    a.d = kfmt->d;
    a.bits = kfmt->mse_bits;
    a.m = kfmt->qjl_m;
    a.out = out;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (T == 0) {
        TQ_LAUNCH_HOOK(who);
        const hipError_t e = tq::launch_attend(a, s);
        return e == hipSuccess ? TQ_OK : hip_fail(e, who);
    }
    TQ_TRY(check_vcache(vc, who));
    if (!use_scratch) {
        if (!ws) return fail(TQ_EINVAL, "%s: NULL workspace", who);
        if (!aligned16(ws)) return fail(TQ_EALIGN, "%s: workspace must be 16-byte aligned", who);
    }
    const DecodePlan plan = decode_plan(kfmt, B, Hq, Hkv, T, n_splits,
                                        map.mode == tq::CacheMap::kPaged ? map.bs : 0);
    const AttendLayout L = attend_layout(kfmt->d, kfmt->qjl_m, B, Hq, plan);
    if (use_scratch) {
        // the device's static scratch instead of a caller workspace
        if (L.total > tq::scratch_capacity())
            return fail(TQ_ENOMEM, "%s: this shape needs %zu B of workspace, more than the %zu B static scratch",
                        who, L.total, tq::scratch_capacity());
        const hipError_t se = tq::scratch_address(&ws);
        if (se != hipSuccess) return hip_fail(se, "tq_attend_decode_noalloc: scratch address");
        ws_bytes = tq::scratch_capacity();
    }
    if (ws_bytes < L.total) return fail(TQ_ENOMEM, "%s: workspace %zu B < %zu B", who, ws_bytes, L.total);
    a.piT = kfmt->rot->d_piT;
    a.sT = kfmt->rot->d_sT;
    a.spiT = kfmt->rot->d_spiT;
    a.pisum = kfmt->rot->d_pisum;
    a.spisum = kfmt->rot->d_spisum;
    a.sq_bound = kfmt->rot->sq_bound;
    a.centroids = kfmt->cb->d_centroids;
    a.kc = kc;
    a.vbits = vfmt->bits;
    a.group = vfmt->group;
    a.vc = vc;
    a.scale = softmax_scale > 0.0f ? softmax_scale : static_cast<float>(1.0 / std::sqrt(double(kfmt->d)));
    a.splits = plan.splits;
    char *base = static_cast<char *>(ws);
    a.qprep = reinterpret_cast<float *>(base + L.qprep);
    a.part_ml = reinterpret_cast<float *>(base + L.ml);
    a.part_acc = reinterpret_cast<float *>(base + L.acc);
    a.mf.gc = plan.gc;
    a.mf.nqc = plan.nqc;
    a.mf.mt = plan.mt;
    a.mf.units = plan.units;
    a.mf.aops = reinterpret_cast<uint32_t *>(base + L.aops);
    a.mf.qscal = reinterpret_cast<float *>(base + L.qscal);
    a.qaux = reinterpret_cast<float *>(base + L.qaux);
    a.mf.lscale = a.scale * kLog2e;
    a.map = map;
    TQ_LAUNCH_HOOK(who);
    hipError_t e;
    if (plan.mfma) {
        e = tq::launch_decode_mfma(a, s);
    } else {
        e = tq::launch_qprep(a, s);
        if (e == hipSuccess) e = tq::launch_attend(a, s);
    }
    return e == hipSuccess ? TQ_OK : hip_fail(e, who);
}

tq_status tq_attend_decode(const tq_key_fmt *kfmt, const tq_val_fmt *vfmt, const void *q, tq_dtype dtype,
                           int B, int Hq, int Hkv, int64_t T, tq_kcache kc, tq_vcache vc, float softmax_scale,
                           int n_splits, void *ws, size_t ws_bytes, float *out, void *stream)
{
    return attend_impl(kfmt, vfmt, q, dtype, B, Hq, Hkv, T, kc, vc, softmax_scale, n_splits, ws, ws_bytes, out,
                       tq::CacheMap{}, stream, "tq_attend_decode");
}

tq_status tq_attend_decode_noalloc(const tq_key_fmt *kfmt, const tq_val_fmt *vfmt, const void *q, tq_dtype dtype,
                                   int B, int Hq, int Hkv, int64_t T, tq_kcache kc, tq_vcache vc,
                                   float softmax_scale, int n_splits, float *out, void *stream)
{
    // the same kernels and split plan as tq_attend_decode; no event records
    // either, even with the profiling hook on
    struct Suppress {
        Suppress() { tq::prof_suppress(true); }
        ~Suppress() { tq::prof_suppress(false); }
    } suppress;
    return attend_impl(kfmt, vfmt, q, dtype, B, Hq, Hkv, T, kc, vc, softmax_scale, n_splits, nullptr, 0, out,
                       tq::CacheMap{}, stream, "tq_attend_decode_noalloc", true);
}

tq_status tq_attend_decode_paged(const tq_key_fmt *kfmt, const tq_val_fmt *vfmt, const void *q, tq_dtype dtype,
                                 int B, int Hq, int Hkv, const tq_cache_layout *lay, tq_kcache kc, tq_vcache vc,
                                 float softmax_scale, int n_splits, void *ws, size_t ws_bytes, float *out,
                                 void *stream)
{
    const char *who = "tq_attend_decode_paged";
    tq::CacheMap m;
    TQ_TRY(layout_map(lay, nullptr, true, who, m));
    return attend_impl(kfmt, vfmt, q, dtype, B, Hq, Hkv, lay->capacity, kc, vc, softmax_scale, n_splits, ws,
                       ws_bytes, out, m, stream, who);
}

}  // extern "C"

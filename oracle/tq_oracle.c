/*
 * fp64 CPU oracle for TurboQuant KV-cache compression and decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library.  It shares no
 * code, header or table with the GPU library; it is a plain, slow statement of
 * what the method computes, written from the method's description on the pages
 * "turboquant-pytorch" (section "What it does": random orthogonal rotation,
 * Lloyd-Max quantizer, 1-bit QJL residual correction, asymmetric scores taken
 * directly on compressed keys) and the discosf.com TurboQuant article (section
 * "TurboQuant in one sentence", steps 1-4: rotation, Lloyd-Max key codes,
 * 1-bit QJL signs of the residual, grouped 2/4-bit value codes packed four to
 * a byte).  Everything is fp64 scalar loops; OpenMP only splits independent
 * vectors across threads and never changes an arithmetic order.
 *
 * Readings of points the pages leave open (stated once here, used below):
 *  - a key is stored as (Lloyd-Max index per rotated coordinate, one QJL sign
 *    per projection row, ||k|| as fp32, ||r|| as fp32);
 *  - the residual r lives in the rotated unit-vector domain, so the query is
 *    projected as S * (Pi q);
 *  - a coordinate equal to a boundary goes to the lower cell; sign(0) = +1;
 *  - codes and signs are LSB-first bit-streams per vector;
 *  - values: per (token, group of g consecutive channels) fp16 scale =
 *    (max-min)/(2^b-1) and fp16 zero = min, both round-to-nearest-even,
 *    code = clamp(round_half_even((v-zero)/scale)), 0 when scale is 0.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef M_PI
#define M_PI 3.14159265358979323846
#endif

/* ------------------------------------------------------------------------ */
/* Random numbers: SplitMix64 (Steele, Lea & Flood, OOPSLA 2014) used as a   */
/* counter generator.  Draw k of a stream is the (k+1)-th output of the      */
/* SplitMix64 sequence started from state seed ^ (stream << 56).            */
/* ------------------------------------------------------------------------ */
uint64_t orc_splitmix_draw(uint64_t seed, int stream, uint64_t k)
{
    uint64_t z = (seed ^ ((uint64_t)stream << 56)) + (k + 1) * 0x9e3779b97f4a7c15ULL;
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
}

/* uniform on (0, 1]: top 53 bits, plus one, times 2^-53 */
double orc_uniform(uint64_t seed, int stream, uint64_t k)
{
    return ((double)(orc_splitmix_draw(seed, stream, k) >> 11) + 1.0) / 9007199254740992.0;
}

/* n-th standard normal of a stream: Box-Muller on uniforms 2p and 2p+1,
   cos output for even n, sin output for odd n. */
double orc_gauss(uint64_t seed, int stream, uint64_t n)
{
    uint64_t p = n >> 1;
    double u1 = orc_uniform(seed, stream, 2 * p);
    double u2 = orc_uniform(seed, stream, 2 * p + 1);
    double rad = sqrt(-2.0 * log(u1));
    double ang = 2.0 * M_PI * u2;
    return (n & 1) ? rad * sin(ang) : rad * cos(ang);
}

/* ------------------------------------------------------------------------ */
/* IEEE binary16, round to nearest even, straight from a double.            */
/* ------------------------------------------------------------------------ */
uint16_t orc_f64_to_f16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x)) return 0x7e00;
    if (a == 0.0) return sign;
    if (a >= 65520.0) return sign | 0x7c00;          /* rounds to infinity */
    int e;
    frexp(a, &e);                                      /* a = f * 2^e, f in [0.5,1) */
    int exp_unbiased = e - 1;                          /* a = 1.x * 2^exp_unbiased */
    double ulp;
    if (exp_unbiased < -14) ulp = ldexp(1.0, -24);     /* subnormal spacing */
    else ulp = ldexp(1.0, exp_unbiased - 10);
    double q = a / ulp;                                /* exact: power-of-two scale */
    double r = nearbyint(q);                           /* default mode: half to even */
    double v = r * ulp;                                /* rounded magnitude */
    /* encode v */
    if (v >= 65536.0) return sign | 0x7c00;
    if (v < ldexp(1.0, -14)) {                         /* subnormal (or became normal min) */
        uint32_t mant = (uint32_t)(v / ldexp(1.0, -24));
        return sign | (uint16_t)mant;                  /* 0x400 encodes the smallest normal */
    }
    int ev;
    double fv = frexp(v, &ev);                         /* v = fv * 2^ev */
    int eb = ev - 1 + 15;
    uint32_t mant = (uint32_t)((fv * 2.0 - 1.0) * 1024.0);
    return sign | (uint16_t)(eb << 10) | (uint16_t)mant;
}

double orc_f16_to_f64(uint16_t h)
{
    int s = (h >> 15) & 1, e = (h >> 10) & 0x1f, m = h & 0x3ff;
    double v;
    if (e == 0) v = ldexp((double)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp(1.0 + m / 1024.0, e - 15);
    return s ? -v : v;
}

/* ------------------------------------------------------------------------ */
/* Rotations.  Dense: Haar-random orthogonal matrix from the QR factors of a */
/* Gaussian matrix (stream 0, row-major), Pi = Q * diag(sign(diag R)), so    */
/* that the R factor has a positive diagonal.  Hadamard: Pi = H D / sqrt(d)  */
/* with H the Sylvester-ordered Walsh-Hadamard matrix and D a diagonal of    */
/* random signs (stream 1, bit 0 set -> -1).  Pi is applied as y = Pi u.     */
/* ------------------------------------------------------------------------ */
void orc_rotation_dense(uint64_t seed, int d, double *pi)
{
    double *a = (double *)malloc(sizeof(double) * d * d);     /* working copy of G */
    double *vs = (double *)calloc((size_t)d * d, sizeof(double)); /* Householder vectors */
    double *rdiag = (double *)malloc(sizeof(double) * d);
    for (int i = 0; i < d; i++)
        for (int j = 0; j < d; j++)
            a[i * d + j] = orc_gauss(seed, 0, (uint64_t)i * d + j);

    for (int k = 0; k < d; k++) {
        double norm2 = 0.0;
        for (int i = k; i < d; i++) norm2 += a[i * d + k] * a[i * d + k];
        double nrm = sqrt(norm2);
        double x0 = a[k * d + k];
        double alpha = (x0 >= 0.0) ? -nrm : nrm;       /* R[k][k] = alpha */
        double *v = vs + (size_t)k * d;
        for (int i = k; i < d; i++) v[i] = a[i * d + k];
        v[k] -= alpha;
        double vn2 = 0.0;
        for (int i = k; i < d; i++) vn2 += v[i] * v[i];
        if (vn2 > 0.0) {
            double inv = 1.0 / sqrt(vn2);
            for (int i = k; i < d; i++) v[i] *= inv;
            /* A[k:, k:] -= 2 v (v^T A[k:, k:]) */
            for (int j = k; j < d; j++) {
                double dot = 0.0;
                for (int i = k; i < d; i++) dot += v[i] * a[i * d + j];
                for (int i = k; i < d; i++) a[i * d + j] -= 2.0 * v[i] * dot;
            }
        }
        rdiag[k] = alpha;
    }
    /* Q = H_0 H_1 ... H_{d-1}: apply to the identity from the right-most one */
    double *q = pi;
    for (int i = 0; i < d; i++)
        for (int j = 0; j < d; j++) q[i * d + j] = (i == j) ? 1.0 : 0.0;
    for (int k = d - 1; k >= 0; k--) {
        double *v = vs + (size_t)k * d;
        for (int j = 0; j < d; j++) {
            double dot = 0.0;
            for (int i = k; i < d; i++) dot += v[i] * q[i * d + j];
            for (int i = k; i < d; i++) q[i * d + j] -= 2.0 * v[i] * dot;
        }
    }
    /* column sign fix */
    for (int j = 0; j < d; j++) {
        if (rdiag[j] < 0.0)
            for (int i = 0; i < d; i++) q[i * d + j] = -q[i * d + j];
    }
    free(a);
    free(vs);
    free(rdiag);
}

static int orc_popcount(unsigned x)
{
    int c = 0;
    while (x) { c += x & 1u; x >>= 1; }
    return c;
}

void orc_hadamard_signs(uint64_t seed, int d, double *dsign)
{
    for (int j = 0; j < d; j++)
        dsign[j] = (orc_splitmix_draw(seed, 1, (uint64_t)j) & 1ULL) ? -1.0 : 1.0;
}

/* Two Hadamard rounds: Pi = (H D2 / sqrt(d)) (H D1 / sqrt(d)), D1 the signs of
   stream 1 (as one round), D2 those of stream 3.  Written as the product of
   the two explicit round matrices. */
void orc_rotation_hadamard2(uint64_t seed, int d, double *pi)
{
    double *a1 = (double *)malloc(sizeof(double) * d * d);
    double *a2 = (double *)malloc(sizeof(double) * d * d);
    double s = 1.0 / sqrt((double)d);
    for (int i = 0; i < d; i++)
        for (int j = 0; j < d; j++) {
            double h = (orc_popcount((unsigned)(i & j)) & 1) ? -1.0 : 1.0;
            double d1 = (orc_splitmix_draw(seed, 1, (uint64_t)j) & 1ULL) ? -1.0 : 1.0;
            double d2 = (orc_splitmix_draw(seed, 3, (uint64_t)j) & 1ULL) ? -1.0 : 1.0;
            a1[i * d + j] = h * d1 * s;
            a2[i * d + j] = h * d2 * s;
        }
    for (int i = 0; i < d; i++)
        for (int j = 0; j < d; j++) {
            double acc = 0.0;
            for (int k = 0; k < d; k++) acc += a2[i * d + k] * a1[k * d + j];
            pi[i * d + j] = acc;
        }
    free(a1);
    free(a2);
}

void orc_rotation_hadamard(uint64_t seed, int d, double *pi)
{
    double *dsign = (double *)malloc(sizeof(double) * d);
    orc_hadamard_signs(seed, d, dsign);
    double s = 1.0 / sqrt((double)d);
    for (int i = 0; i < d; i++)
        for (int j = 0; j < d; j++) {
            double h = (orc_popcount((unsigned)(i & j)) & 1) ? -1.0 : 1.0;
            pi[i * d + j] = h * dsign[j] * s;
        }
    free(dsign);
}

/* QJL projection: m x d iid N(0,1), stream 2, row-major */
void orc_qjl_matrix(uint64_t seed, int m, int d, double *s)
{
    for (int i = 0; i < m; i++)
        for (int j = 0; j < d; j++)
            s[(size_t)i * d + j] = orc_gauss(seed, 2, (uint64_t)i * d + j);
}

/* ------------------------------------------------------------------------ */
/* Lloyd-Max codebook for one coordinate of a uniformly random unit vector   */
/* in R^d.  That coordinate has density                                      */
/*     f_d(x) = C_d (1 - x^2)^((d-3)/2) on [-1, 1],                          */
/*     C_d = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)).                         */
/* An L-level Lloyd-Max quantizer satisfies two conditions: every boundary   */
/* is the midpoint of its two neighbouring centroids, and every centroid is  */
/* the conditional mean of f_d over its cell.  Integrals use composite       */
/* Gauss-Legendre quadrature in the variable phi, x = sin(phi), where the   */
/* integrand g(sin phi) cos(phi)^(d-2) is smooth up to the endpoints.        */
/* The fixed point is reached by Lloyd iteration followed by Newton steps on */
/* the same two conditions.                                                  */
/* ------------------------------------------------------------------------ */
#define ORC_GL_N 16
#define ORC_PANELS 64

/* Legendre P_n and its derivative at z by the three-term recurrence */
static void orc_legendre(int n, double z, double *pn, double *dpn)
{
    double p0 = 1.0, p1 = z;
    for (int k = 2; k <= n; k++) {
        double pk = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
        p0 = p1;
        p1 = pk;
    }
    *pn = p1;
    *dpn = n * (z * p1 - p0) / (z * z - 1.0);
}

/* n-point Gauss-Legendre nodes and weights on [-1, 1] (Newton on P_n) */
static void orc_gauss_legendre(int n, double *x, double *w)
{
    for (int i = 0; i < n; i++) {
        double z = cos(M_PI * (i + 0.75) / (n + 0.5)), p, dp;
        for (int it = 0; it < 100; it++) {
            orc_legendre(n, z, &p, &dp);
            double dz = p / dp;
            z -= dz;
            if (fabs(dz) < 1e-16) break;
        }
        orc_legendre(n, z, &p, &dp);
        x[i] = z;
        w[i] = 2.0 / ((1.0 - z * z) * dp * dp);
    }
}

double orc_density(int d, double x)
{
    if (x <= -1.0 || x >= 1.0) return (d == 3) ? 0.5 : 0.0;
    double logc = lgamma(0.5 * d) - lgamma(0.5 * (d - 1)) - 0.5 * log(M_PI);
    return exp(logc + 0.5 * (d - 3) * log1p(-x * x));
}

/* mass and first moment of f_d over [a, b] */
void orc_cell_moments(int d, double a, double b, double *mass, double *moment)
{
    static int ready = 0;
    static double gx[ORC_GL_N], gw[ORC_GL_N];
    if (!ready) {                                    /* first call is single-threaded */
        orc_gauss_legendre(ORC_GL_N, gx, gw);
        ready = 1;
    }
    double logc = lgamma(0.5 * d) - lgamma(0.5 * (d - 1)) - 0.5 * log(M_PI);
    double cd = exp(logc);
    double pa = asin(a < -1.0 ? -1.0 : a), pb = asin(b > 1.0 ? 1.0 : b);
    double h = (pb - pa) / ORC_PANELS;
    double m0 = 0.0, m1 = 0.0;
    for (int p = 0; p < ORC_PANELS; p++) {
        double lo = pa + p * h;
        for (int i = 0; i < ORC_GL_N; i++) {
            double phi = lo + 0.5 * h * (gx[i] + 1.0);
            double c = cos(phi);
            double wt = 0.5 * h * gw[i] * pow(c, (double)(d - 2));
            m0 += wt;
            m1 += wt * sin(phi);
        }
    }
    *mass = cd * m0;
    *moment = cd * m1;
}

static void orc_boundaries_from_centroids(int L, const double *c, double *t_full)
{
    /* t_full[0] = -1, t_full[L] = 1, t_full[i] = midpoint of c[i-1], c[i] */
    t_full[0] = -1.0;
    t_full[L] = 1.0;
    for (int i = 1; i < L; i++) t_full[i] = 0.5 * (c[i - 1] + c[i]);
}

static void orc_symmetrize(int L, double *c)
{
    for (int i = 0; i < L / 2; i++) {
        double v = 0.5 * (c[L - 1 - i] - c[i]);
        c[i] = -v;
        c[L - 1 - i] = v;
    }
}

/* residual of the centroid condition, F_i = c_i - E[x | cell i] */
static double orc_lloyd_residual(int d, int L, const double *c, double *cond_mean,
                                 double *mass, double *t_full)
{
    orc_boundaries_from_centroids(L, c, t_full);
    double worst = 0.0;
    for (int i = 0; i < L; i++) {
        double m0, m1;
        orc_cell_moments(d, t_full[i], t_full[i + 1], &m0, &m1);
        mass[i] = m0;
        cond_mean[i] = m1 / m0;
        double r = fabs(c[i] - cond_mean[i]);
        if (r > worst) worst = r;
    }
    return worst;
}

/* Returns the number of iterations used, or -1 when not converged.
   centroids: L = 2^bits values; boundaries: L-1 interior boundaries. */
int orc_codebook(int d, int bits, double *centroids, double *boundaries, double *final_residual)
{
    int L = 1 << bits;
    double *c = centroids;
    double *cm = (double *)malloc(sizeof(double) * L);
    double *ms = (double *)malloc(sizeof(double) * L);
    double *tf = (double *)malloc(sizeof(double) * (L + 1));
    double *lo = (double *)malloc(sizeof(double) * L);
    double *di = (double *)malloc(sizeof(double) * L);
    double *up = (double *)malloc(sizeof(double) * L);
    double *rhs = (double *)malloc(sizeof(double) * L);
    double *trial = (double *)malloc(sizeof(double) * L);
    double sigma = 1.0 / sqrt((double)d);
    /* start: evenly spaced over +-2.5 sigma, clipped inside (-1, 1) */
    for (int i = 0; i < L; i++) {
        double v = 2.5 * sigma * (2.0 * i + 1.0 - L) / L;
        if (v > 0.95) v = 0.95;
        if (v < -0.95) v = -0.95;
        c[i] = v;
    }
    int iters = 0;
    double res = 0.0;
    /* Lloyd iteration: c <- E[x | cell(c)] */
    for (int it = 0; it < 300; it++, iters++) {
        res = orc_lloyd_residual(d, L, c, cm, ms, tf);
        for (int i = 0; i < L; i++) c[i] = cm[i];
        orc_symmetrize(L, c);
        if (res < 1e-13) break;
    }
    /* Newton on F(c) = c - m(c) with the tridiagonal Jacobian
       dm_i/dt_i = f(t_i)(m_i - t_i)/P_i,  dm_i/dt_{i+1} = f(t_{i+1})(t_{i+1} - m_i)/P_i,
       t_i = (c_{i-1} + c_i)/2. */
    res = orc_lloyd_residual(d, L, c, cm, ms, tf);
    for (int it = 0; it < 60 && res > 1e-15; it++, iters++) {
        for (int i = 0; i < L; i++) {
            double gl = (i > 0) ? orc_density(d, tf[i]) * (cm[i] - tf[i]) / ms[i] : 0.0;
            double gu = (i < L - 1) ? orc_density(d, tf[i + 1]) * (tf[i + 1] - cm[i]) / ms[i] : 0.0;
            /* row i of I - dm/dc */
            lo[i] = -0.5 * gl;
            up[i] = -0.5 * gu;
            di[i] = 1.0 - 0.5 * gl - 0.5 * gu;
            rhs[i] = -(c[i] - cm[i]);
        }
        /* Thomas algorithm */
        for (int i = 1; i < L; i++) {
            double f = lo[i] / di[i - 1];
            di[i] -= f * up[i - 1];
            rhs[i] -= f * rhs[i - 1];
        }
        rhs[L - 1] /= di[L - 1];
        for (int i = L - 2; i >= 0; i--) rhs[i] = (rhs[i] - up[i] * rhs[i + 1]) / di[i];
        double step = 1.0, new_res = res;
        for (int h = 0; h < 30; h++) {
            for (int i = 0; i < L; i++) trial[i] = c[i] + step * rhs[i];
            orc_symmetrize(L, trial);
            new_res = orc_lloyd_residual(d, L, trial, cm, ms, tf);
            if (new_res < res || new_res < 1e-15) break;
            step *= 0.5;
        }
        if (!(new_res < res) && !(new_res < 1e-15)) break;
        memcpy(c, trial, sizeof(double) * L);
        res = new_res;
    }
    res = orc_lloyd_residual(d, L, c, cm, ms, tf);
    for (int i = 0; i < L - 1; i++) boundaries[i] = tf[i + 1];
    if (final_residual) *final_residual = res;
    free(cm); free(ms); free(tf); free(lo); free(di); free(up); free(rhs); free(trial);
    return (res < 1e-12) ? iters : -1;
}

/* ------------------------------------------------------------------------ */
/* Bit-streams: element j of width w occupies bits [w j, w j + w) of the     */
/* vector's little-endian byte string.                                       */
/* ------------------------------------------------------------------------ */
static void orc_put_bits(uint8_t *row, int j, int w, unsigned value)
{
    for (int q = 0; q < w; q++) {
        int bit = w * j + q;
        if ((value >> q) & 1u) row[bit >> 3] |= (uint8_t)(1u << (bit & 7));
    }
}

static unsigned orc_get_bits(const uint8_t *row, int j, int w)
{
    unsigned v = 0;
    for (int q = 0; q < w; q++) {
        int bit = w * j + q;
        v |= (unsigned)((row[bit >> 3] >> (bit & 7)) & 1u) << q;
    }
    return v;
}

void orc_pack(const uint32_t *vals, int64_t n_vec, int per_vec, int w, uint8_t *out)
{
    int64_t row_bytes = ((int64_t)per_vec * w + 7) / 8;
    memset(out, 0, (size_t)(row_bytes * n_vec));
    for (int64_t t = 0; t < n_vec; t++)
        for (int j = 0; j < per_vec; j++)
            orc_put_bits(out + t * row_bytes, j, w, vals[t * per_vec + j]);
}

void orc_unpack(const uint8_t *in, int64_t n_vec, int per_vec, int w, uint32_t *vals)
{
    int64_t row_bytes = ((int64_t)per_vec * w + 7) / 8;
    for (int64_t t = 0; t < n_vec; t++)
        for (int j = 0; j < per_vec; j++)
            vals[t * per_vec + j] = orc_get_bits(in + t * row_bytes, j, w);
}

/* ------------------------------------------------------------------------ */
/* Key compression (rotation, Lloyd-Max codes, QJL signs of the residual).  */
/* For each key k (given exactly in fp64):                                   */
/*   n = ||k||, u = k / n (u = 0 when n = 0), y = Pi u,                      */
/*   idx_j = #{i : t_i < y_j}, r = y - c[idx], rho = ||r||,                   */
/*   z = S r, sign bit i = [z_i >= 0];                                       */
/* stored: codes (bits per index), signs (1 bit per row), fp32 n, fp32 rho.  */
/* Optional outputs y, z, rho (fp64) let tests measure distances to the     */
/* decision boundaries.                                                      */
/* ------------------------------------------------------------------------ */
void orc_compress_keys(int d, int bits, int m, const double *pi, const double *s,
                       const double *centroids, const double *boundaries,
                       const double *k, int64_t n_vec,
                       uint8_t *codes, uint8_t *signs, float *knorm, float *rnorm,
                       double *y_out, double *z_out, double *rho_out)
{
    int L = 1 << bits;
    int64_t code_bytes = ((int64_t)d * bits + 7) / 8, sign_bytes = ((int64_t)m + 7) / 8;
    memset(codes, 0, (size_t)(code_bytes * n_vec));
    memset(signs, 0, (size_t)(sign_bytes * n_vec));
#pragma omp parallel
    {
        double *u = (double *)malloc(sizeof(double) * d);
        double *y = (double *)malloc(sizeof(double) * d);
        double *r = (double *)malloc(sizeof(double) * d);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < n_vec; t++) {
            const double *kv = k + t * d;
            double n2 = 0.0;
            for (int j = 0; j < d; j++) n2 += kv[j] * kv[j];
            double n = sqrt(n2);
            for (int j = 0; j < d; j++) u[j] = (n > 0.0) ? kv[j] / n : 0.0;
            for (int i = 0; i < d; i++) {
                double acc = 0.0;
                for (int j = 0; j < d; j++) acc += pi[(size_t)i * d + j] * u[j];
                y[i] = acc;
            }
            double rho2 = 0.0;
            for (int j = 0; j < d; j++) {
                int idx = 0;
                for (int i = 0; i < L - 1; i++)
                    if (boundaries[i] < y[j]) idx++;
                orc_put_bits(codes + t * code_bytes, j, bits, (unsigned)idx);
                r[j] = y[j] - centroids[idx];
                rho2 += r[j] * r[j];
            }
            double rho = sqrt(rho2);
            for (int i = 0; i < m; i++) {
                double z = 0.0;
                for (int j = 0; j < d; j++) z += s[(size_t)i * d + j] * r[j];
                if (z >= 0.0) orc_put_bits(signs + t * sign_bytes, i, 1, 1u);
                if (z_out) z_out[t * m + i] = z;
            }
            knorm[t] = (float)n;
            rnorm[t] = (float)rho;
            if (y_out)
                for (int j = 0; j < d; j++) y_out[t * d + j] = y[j];
            if (rho_out) rho_out[t] = rho;
        }
        free(u);
        free(y);
        free(r);
    }
}

/* Residual, QJL signs and ||r|| of one key for a given rotated vector y and a
   given code vector idx (the second half of the key encoder).  Used to derive
   the alternative encoding of a key when a rotated coordinate sits on a
   decision boundary and either adjacent cell is a valid code. */
void orc_key_residual_signs(int d, int m, const double *s, const double *centroids,
                            const double *y, const uint32_t *idx, uint8_t *signs,
                            double *z_out, double *rho_out)
{
    double *r = (double *)malloc(sizeof(double) * d);
    double rho2 = 0.0;
    for (int j = 0; j < d; j++) {
        r[j] = y[j] - centroids[idx[j]];
        rho2 += r[j] * r[j];
    }
    memset(signs, 0, (size_t)((m + 7) / 8));
    for (int i = 0; i < m; i++) {
        double z = 0.0;
        for (int j = 0; j < d; j++) z += s[(size_t)i * d + j] * r[j];
        if (z >= 0.0) orc_put_bits(signs, i, 1, 1u);
        if (z_out) z_out[i] = z;
    }
    *rho_out = sqrt(rho2);
    free(r);
}

/* ------------------------------------------------------------------------ */
/* Value compression: asymmetric min-max quantization per group of `group`   */
/* consecutive channels of one token, fp16 scale and zero, codes packed      */
/* LSB-first (four 2-bit or two 4-bit codes per byte).  params holds         */
/* (scale, zero) fp16 bit patterns per group.  quot_out (optional) receives  */
/* (v - zero) / scale before rounding, for boundary accounting.              */
/* ------------------------------------------------------------------------ */
void orc_compress_values(int d, int bits, int group, const double *v, int64_t n_vec,
                         uint8_t *codes, uint16_t *params, double *quot_out)
{
    int levels = (1 << bits) - 1;
    int64_t code_bytes = ((int64_t)d * bits + 7) / 8;
    int ng = d / group;
    memset(codes, 0, (size_t)(code_bytes * n_vec));
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n_vec; t++) {
        for (int g = 0; g < ng; g++) {
            const double *x = v + t * d + (int64_t)g * group;
            double mn = x[0], mx = x[0];
            for (int j = 1; j < group; j++) {
                if (x[j] < mn) mn = x[j];
                if (x[j] > mx) mx = x[j];
            }
            uint16_t sh = orc_f64_to_f16((mx - mn) / levels);
            uint16_t zh = orc_f64_to_f16(mn);
            double sc = orc_f16_to_f64(sh), ze = orc_f16_to_f64(zh);
            params[(t * ng + g) * 2 + 0] = sh;
            params[(t * ng + g) * 2 + 1] = zh;
            for (int j = 0; j < group; j++) {
                unsigned code = 0;
                double qv = 0.0;
                if (sc > 0.0) {
                    qv = (x[j] - ze) / sc;
                    double rq = nearbyint(qv);
                    if (rq < 0.0) rq = 0.0;
                    if (rq > levels) rq = levels;
                    code = (unsigned)rq;
                }
                if (quot_out) quot_out[t * d + (int64_t)g * group + j] = qv;
                orc_put_bits(codes + t * code_bytes, g * group + j, bits, code);
            }
        }
    }
}

/* v_hat = code * scale + zero */
void orc_dequant_values(int d, int bits, int group, const uint8_t *codes, const uint16_t *params,
                        int64_t n_vec, double *out)
{
    int64_t code_bytes = ((int64_t)d * bits + 7) / 8;
    int ng = d / group;
    for (int64_t t = 0; t < n_vec; t++)
        for (int j = 0; j < d; j++) {
            int g = j / group;
            double sc = orc_f16_to_f64(params[(t * ng + g) * 2 + 0]);
            double ze = orc_f16_to_f64(params[(t * ng + g) * 2 + 1]);
            out[t * d + j] = orc_get_bits(codes + t * code_bytes, j, bits) * sc + ze;
        }
}

/* ------------------------------------------------------------------------ */
/* Asymmetric scores straight from a packed key cache of one KV head:        */
/*   q_rot = Pi q,  Sq = S q_rot,                                            */
/*   score_t = n_t ( sum_j q_rot_j c[idx_tj]                                 */
/*                   + sqrt(pi/2)/m * rho_t * sum_i Sq_i (2 s_ti - 1) ).     */
/* term_mse / term_qjl (optional) receive the two summands times n_t.       */
/* ------------------------------------------------------------------------ */
void orc_scores(int d, int bits, int m, const double *pi, const double *s,
                const double *centroids, const double *q, int nq,
                const uint8_t *codes, const uint8_t *signs, const float *knorm,
                const float *rnorm, int64_t T,
                double *scores, double *term_mse, double *term_qjl)
{
    int64_t code_bytes = ((int64_t)d * bits + 7) / 8, sign_bytes = ((int64_t)m + 7) / 8;
    double *qrot = (double *)malloc(sizeof(double) * d * nq);
    double *sq = (double *)malloc(sizeof(double) * (m > 0 ? m : 1) * nq);
    /* m = 0: the first (MSE) stage alone, no QJL term */
    double kappa = m > 0 ? sqrt(M_PI / 2.0) / m : 0.0;
    for (int h = 0; h < nq; h++) {
        for (int i = 0; i < d; i++) {
            double acc = 0.0;
            for (int j = 0; j < d; j++) acc += pi[(size_t)i * d + j] * q[h * d + j];
            qrot[h * d + i] = acc;
        }
        for (int i = 0; i < m; i++) {
            double acc = 0.0;
            for (int j = 0; j < d; j++) acc += s[(size_t)i * d + j] * qrot[h * d + j];
            sq[h * m + i] = acc;
        }
    }
#pragma omp parallel
    {
        unsigned *idx = (unsigned *)malloc(sizeof(unsigned) * d);
        double *sgn = (double *)malloc(sizeof(double) * (m > 0 ? m : 1));
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; t++) {
            const uint8_t *cr = codes + t * code_bytes, *sr = signs + t * sign_bytes;
            for (int j = 0; j < d; j++) idx[j] = orc_get_bits(cr, j, bits);
            for (int i = 0; i < m; i++) sgn[i] = orc_get_bits(sr, i, 1) ? 1.0 : -1.0;
            double n = (double)knorm[t], rho = (double)rnorm[t];
            for (int h = 0; h < nq; h++) {
                double a = 0.0, b = 0.0;
                for (int j = 0; j < d; j++) a += qrot[h * d + j] * centroids[idx[j]];
                for (int i = 0; i < m; i++) b += sq[h * m + i] * sgn[i];
                double t1 = n * a, t2 = n * kappa * rho * b;
                scores[(int64_t)h * T + t] = t1 + t2;
                if (term_mse) term_mse[(int64_t)h * T + t] = t1;
                if (term_qjl) term_qjl[(int64_t)h * T + t] = t2;
            }
        }
        free(idx);
        free(sgn);
    }
    free(qrot);
    free(sq);
}

/* ------------------------------------------------------------------------ */
/* Explicit estimate of packed keys (dequantisation):                        */
/*   k_hat = n Pi^T ( c[idx] + sqrt(pi/2)/m * rho * S^T (2 s - 1) ),          */
/* the vector whose inner product with any query equals the asymmetric      */
/* score above; with m = 0 (first stage alone) k_hat = n Pi^T c[idx].        */
/* ------------------------------------------------------------------------ */
void orc_dequant_keys(int d, int bits, int m, const double *pi, const double *s,
                      const double *centroids, const uint8_t *codes, const uint8_t *signs,
                      const float *knorm, const float *rnorm, int64_t n_vec, double *out)
{
    int64_t code_bytes = ((int64_t)d * bits + 7) / 8, sign_bytes = ((int64_t)m + 7) / 8;
    double kappa = m > 0 ? sqrt(M_PI / 2.0) / m : 0.0;
#pragma omp parallel
    {
        double *yh = (double *)malloc(sizeof(double) * d);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < n_vec; t++) {
            const uint8_t *cr = codes + t * code_bytes;
            for (int j = 0; j < d; j++) yh[j] = centroids[orc_get_bits(cr, j, bits)];
            if (m > 0) {
                const uint8_t *sr = signs + t * sign_bytes;
                double f = kappa * (double)rnorm[t];
                for (int j = 0; j < d; j++) {
                    double acc = 0.0;
                    for (int i = 0; i < m; i++)
                        acc += s[(size_t)i * d + j] * (orc_get_bits(sr, i, 1) ? 1.0 : -1.0);
                    yh[j] += f * acc;
                }
            }
            double n = (double)knorm[t];
            for (int c = 0; c < d; c++) {
                double acc = 0.0;
                for (int j = 0; j < d; j++) acc += pi[(size_t)j * d + c] * yh[j];
                out[t * d + c] = n * acc;
            }
        }
        free(yh);
    }
}

/* ------------------------------------------------------------------------ */
/* Decode attention of nq query heads over one KV head's T packed tokens:   */
/*   lambda_t = scale * score_t, p = softmax(lambda), out = sum_t p_t v_hat_t */
/* with the max subtracted before exponentiation.  T = 0 gives zeros.        */
/* orc_softmax_values takes the scores [nq][T] (overwritten) and does the    */
/* rest; orc_attend and orc_attend_block differ only in the scores.          */
/* ------------------------------------------------------------------------ */
static void orc_softmax_values(int d, int nq, int64_t T, double *sc, int vbits, int group,
                               const uint8_t *vcodes, const uint16_t *vparams, double scale,
                               double *out);

void orc_attend(int d, int bits, int m, const double *pi, const double *s,
                const double *centroids, const double *q, int nq,
                const uint8_t *codes, const uint8_t *signs, const float *knorm,
                const float *rnorm, int64_t T,
                int vbits, int group, const uint8_t *vcodes, const uint16_t *vparams,
                double scale, double *out)
{
    memset(out, 0, sizeof(double) * d * nq);
    if (T <= 0) return;
    double *sc = (double *)malloc(sizeof(double) * nq * T);
    orc_scores(d, bits, m, pi, s, centroids, q, nq, codes, signs, knorm, rnorm, T, sc, NULL, NULL);
    orc_softmax_values(d, nq, T, sc, vbits, group, vcodes, vparams, scale, out);
    free(sc);
}

static void orc_softmax_values(int d, int nq, int64_t T, double *sc, int vbits, int group,
                               const uint8_t *vcodes, const uint16_t *vparams, double scale,
                               double *out)
{
    int64_t vbytes = ((int64_t)d * vbits + 7) / 8;
    int ng = d / group;
    /* softmax weights per query head (max subtracted) */
    for (int h = 0; h < nq; h++) {
        double *lam = sc + (int64_t)h * T;
        double mx = -INFINITY;
        for (int64_t t = 0; t < T; t++) {
            lam[t] *= scale;
            if (lam[t] > mx) mx = lam[t];
        }
        double den = 0.0;
        for (int64_t t = 0; t < T; t++) {
            lam[t] = exp(lam[t] - mx);
            den += lam[t];
        }
        for (int64_t t = 0; t < T; t++) lam[t] /= den;
    }
    /* out[h][j] = sum_t p[h][t] v_hat[t][j]; channels split across threads, t in order */
#pragma omp parallel for schedule(static)
    for (int j = 0; j < d; j++) {
        int g = j / group;
        for (int64_t t = 0; t < T; t++) {
            double sv = orc_f16_to_f64(vparams[(t * ng + g) * 2 + 0]);
            double zv = orc_f16_to_f64(vparams[(t * ng + g) * 2 + 1]);
            double vh = orc_get_bits(vcodes + t * vbytes, j, vbits) * sv + zv;
            for (int h = 0; h < nq; h++) out[(int64_t)h * d + j] += sc[(int64_t)h * T + t] * vh;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Rotated scalar block formats, the comparison the tproger.ru article      */
/* reports (section "First benchmarks": Q8_0 and Q4_0 with and without      */
/* rotation).  The key is rotated, x = Pi k (no normalisation), and each    */
/* block of 32 consecutive rotated coordinates keeps one fp16 scale and one */
/* signed integer per coordinate:                                           */
/*   scale = fp16_rne(amax / qmax), qmax = 127 (8 bits) or 7 (4 bits),      */
/*   q_j = clamp(round_half_even(x_j / scale), -qmax, qmax), 0 if scale = 0,  */
/* stored as an int8 byte (8 bits) or as q + 8 in 4 bits (LSB-first).       */
/* x_hat_j = scale * q_j, and the score of q is sum_j (Pi q)_j x_hat_j =     */
/* <q, Pi^T x_hat>.  x_out and quot_out (optional) receive x and x / scale    */
/* for tie accounting.                                                      */
/* ------------------------------------------------------------------------ */
static int orc_block_qmax(int bits) { return bits == 8 ? 127 : 7; }

void orc_compress_keys_block(int d, int bits, const double *pi, const double *k, int64_t n_vec,
                             uint8_t *codes, uint16_t *scales, double *x_out, double *quot_out)
{
    const int qmax = orc_block_qmax(bits), nb = d / 32;
    const int64_t code_bytes = (int64_t)d * bits / 8;
    memset(codes, 0, (size_t)(code_bytes * n_vec));
#pragma omp parallel
    {
        double *x = (double *)malloc(sizeof(double) * d);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < n_vec; t++) {
            for (int i = 0; i < d; i++) {
                double acc = 0.0;
                for (int j = 0; j < d; j++) acc += pi[(size_t)i * d + j] * k[t * d + j];
                x[i] = acc;
                if (x_out) x_out[t * d + i] = acc;
            }
            for (int b = 0; b < nb; b++) {
                double amax = 0.0;
                for (int j = 0; j < 32; j++)
                    if (fabs(x[32 * b + j]) > amax) amax = fabs(x[32 * b + j]);
                uint16_t sh = orc_f64_to_f16(amax / qmax);
                double sc = orc_f16_to_f64(sh);
                scales[t * nb + b] = sh;
                for (int j = 0; j < 32; j++) {
                    int c = 32 * b + j;
                    int qv = 0;
                    double qt = 0.0;
                    if (sc > 0.0) {
                        qt = x[c] / sc;
                        double r = nearbyint(qt);
                        if (r > qmax) r = qmax;
                        if (r < -qmax) r = -qmax;
                        qv = (int)r;
                    }
                    if (quot_out) quot_out[t * d + c] = qt;
                    if (bits == 8) codes[t * code_bytes + c] = (uint8_t)(int8_t)qv;
                    else orc_put_bits(codes + t * code_bytes, c, 4, (unsigned)(qv + 8));
                }
            }
        }
        free(x);
    }
}

/* x_hat of one packed block-format row */
static void orc_block_row(int d, int bits, const uint8_t *row, const uint16_t *sc, double *xh)
{
    for (int c = 0; c < d; c++) {
        int qv = bits == 8 ? (int)(int8_t)row[c] : (int)orc_get_bits(row, c, 4) - 8;
        xh[c] = orc_f16_to_f64(sc[c / 32]) * qv;
    }
}

void orc_scores_block(int d, int bits, const double *pi, const double *q, int nq,
                      const uint8_t *codes, const uint16_t *scales, int64_t T, double *scores)
{
    const int64_t code_bytes = (int64_t)d * bits / 8;
    double *qrot = (double *)malloc(sizeof(double) * d * nq);
    for (int h = 0; h < nq; h++)
        for (int i = 0; i < d; i++) {
            double acc = 0.0;
            for (int j = 0; j < d; j++) acc += pi[(size_t)i * d + j] * q[h * d + j];
            qrot[h * d + i] = acc;
        }
#pragma omp parallel
    {
        double *xh = (double *)malloc(sizeof(double) * d);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; t++) {
            orc_block_row(d, bits, codes + t * code_bytes, scales + t * (d / 32), xh);
            for (int h = 0; h < nq; h++) {
                double a = 0.0;
                for (int c = 0; c < d; c++) a += qrot[h * d + c] * xh[c];
                scores[(int64_t)h * T + t] = a;
            }
        }
        free(xh);
    }
    free(qrot);
}

/* k_hat = Pi^T x_hat */
void orc_dequant_keys_block(int d, int bits, const double *pi, const uint8_t *codes,
                            const uint16_t *scales, int64_t n_vec, double *out)
{
    const int64_t code_bytes = (int64_t)d * bits / 8;
#pragma omp parallel
    {
        double *xh = (double *)malloc(sizeof(double) * d);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < n_vec; t++) {
            orc_block_row(d, bits, codes + t * code_bytes, scales + t * (d / 32), xh);
            for (int c = 0; c < d; c++) {
                double acc = 0.0;
                for (int j = 0; j < d; j++) acc += pi[(size_t)j * d + c] * xh[j];
                out[t * d + c] = acc;
            }
        }
        free(xh);
    }
}

void orc_attend_block(int d, int bits, const double *pi, const double *q, int nq,
                      const uint8_t *codes, const uint16_t *scales, int64_t T,
                      int vbits, int group, const uint8_t *vcodes, const uint16_t *vparams,
                      double scale, double *out)
{
    memset(out, 0, sizeof(double) * d * nq);
    if (T <= 0) return;
    double *sc = (double *)malloc(sizeof(double) * nq * T);
    orc_scores_block(d, bits, pi, q, nq, codes, scales, T, sc);
    orc_softmax_values(d, nq, T, sc, vbits, group, vcodes, vparams, scale, out);
    free(sc);
}

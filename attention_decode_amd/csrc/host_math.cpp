// Host-side fp64 construction of the immutable tables libtq uploads once:
// the Lloyd-Max codebook, the rotation Pi and the QJL projection S.
//
// Codebook: moments of f_d(x) = C_d (1 - x^2)^((d-3)/2) in closed form
//   mass   : x^2 ~ Beta(1/2, (d-1)/2), evaluated with the continued fraction
//            of the regularised incomplete beta (DLMF 8.17.22, modified Lentz);
//   moment : int_a^b x f_d = C_d/(d-1) [(1-a^2)^((d-1)/2) - (1-b^2)^((d-1)/2)].
// The two Lloyd-Max conditions (boundaries at midpoints, centroids at cell
// means) are solved on the positive half by Lloyd sweeps and then Newton
// steps, and mirrored, so the codebook is exactly symmetric.
//
// Rotation: the Gaussian matrix is orthonormalised column by column with
// classical Gram-Schmidt applied twice, which yields the Q factor whose R has
// a positive diagonal (the Haar-distributed choice).
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "tq_internal.h"

namespace tq {

// ---------------------------------------------------------------- random
// SplitMix64 output function applied to a counter: draw k of `stream` is the
// (k+1)-th output of the sequence whose state starts at seed ^ (stream << 56).
uint64_t rng_draw(uint64_t seed, int stream, uint64_t k)
{
    uint64_t state = seed ^ (static_cast<uint64_t>(stream) << 56);
    state += (k + 1) * 0x9e3779b97f4a7c15ULL;
    state = (state ^ (state >> 30)) * 0xbf58476d1ce4e5b9ULL;
    state = (state ^ (state >> 27)) * 0x94d049bb133111ebULL;
    return state ^ (state >> 31);
}

static double rng_unit(uint64_t seed, int stream, uint64_t k)
{
    const double two53 = 9007199254740992.0;
    return (static_cast<double>(rng_draw(seed, stream, k) >> 11) + 1.0) / two53;
}

double rng_normal(uint64_t seed, int stream, uint64_t n)
{
    const uint64_t pair = n / 2;
    const double radius = std::sqrt(-2.0 * std::log(rng_unit(seed, stream, 2 * pair)));
    const double angle = 2.0 * M_PI * rng_unit(seed, stream, 2 * pair + 1);
    return (n % 2 == 0) ? radius * std::cos(angle) : radius * std::sin(angle);
}

// --------------------------------------------------------------- codebook
namespace {

// Regularised incomplete beta I_x(a, b) by its continued fraction; the
// fraction converges fast for x < (a+1)/(a+b+2), otherwise use the symmetry
// I_x(a, b) = 1 - I_{1-x}(b, a).
double inc_beta_cf(double a, double b, double x, double inv_beta)
{
    // g = 1 + d_1/(1 + d_2/(1 + ...)) by the modified Lentz method, with
    // d_{2m} = m(b-m)x / ((a+2m-1)(a+2m)),
    // d_{2m+1} = -(a+m)(a+b+m)x / ((a+2m)(a+2m+1));  I = x^a (1-x)^b / (a B(a,b) g).
    const double tiny = 1e-300;
    double g = 1.0, cj = 1.0, dj = 0.0;
    for (int j = 1; j < 4000; ++j) {
        double num;
        if (j % 2 == 0) {
            const int m = j / 2;
            num = m * (b - m) * x / ((a + 2 * m - 1) * (a + 2 * m));
        } else {
            const int m = (j - 1) / 2;
            num = -((a + m) * (a + b + m) * x) / ((a + 2 * m) * (a + 2 * m + 1));
        }
        dj = 1.0 + num * dj;
        if (std::fabs(dj) < tiny) dj = tiny;
        cj = 1.0 + num / cj;
        if (std::fabs(cj) < tiny) cj = tiny;
        dj = 1.0 / dj;
        const double delta = cj * dj;
        g *= delta;
        if (std::fabs(delta - 1.0) < 2e-16) break;
    }
    const double front = std::exp(a * std::log(x) + b * std::log1p(-x)) * inv_beta / a;
    return front / g;
}

// inv_beta = 1 / B(a, b), supplied by the caller (B is symmetric)
double inc_beta(double a, double b, double x, double inv_beta)
{
    if (x <= 0.0) return 0.0;
    if (x >= 1.0) return 1.0;
    if (x < (a + 1.0) / (a + b + 2.0)) return inc_beta_cf(a, b, x, inv_beta);
    return 1.0 - inc_beta_cf(b, a, 1.0 - x, inv_beta);
}

// C_d = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)) = 1 / B(1/2, (d-1)/2), by the
// recurrence r(n+2) = n/(n-1) r(n) on r(n) = Gamma(n/2)/Gamma((n-1)/2) from
// r(2) = 1/sqrt(pi), r(3) = sqrt(pi)/2; avoids the cancellation of two large
// log-gamma values.
double unit_coordinate_constant(int d)
{
    double r = (d % 2 == 0) ? 1.0 / std::sqrt(M_PI) : std::sqrt(M_PI) / 2.0;
    for (int n = (d % 2 == 0) ? 2 : 3; n < d; n += 2) r *= static_cast<double>(n) / (n - 1);
    return r / std::sqrt(M_PI);
}

struct Density {
    int d;
    double cd;   // normalising constant C_d
    explicit Density(int dim) : d(dim), cd(unit_coordinate_constant(dim)) {}
    double pdf(double x) const
    {
        if (x <= -1.0 || x >= 1.0) return d == 3 ? 0.5 : 0.0;
        return cd * std::exp(0.5 * (d - 3) * std::log1p(-x * x));
    }
    // P(X > x) for x >= 0: (1/2) I_{1-x^2}((d-1)/2, 1/2), no cancellation in the tail
    double upper_tail(double x) const
    {
        if (x >= 1.0) return 0.0;
        return 0.5 * inc_beta(0.5 * (d - 1), 0.5, 1.0 - x * x, cd);
    }
    // mass of [a, b] with 0 <= a < b <= 1
    double mass(double a, double b) const { return upper_tail(a) - upper_tail(b); }
    double moment(double a, double b) const
    {
        const double e = 0.5 * (d - 1);
        const double pa = (a >= 1.0) ? 0.0 : std::exp(e * std::log1p(-a * a));
        const double pb = (b >= 1.0) ? 0.0 : std::exp(e * std::log1p(-b * b));
        return cd / (d - 1) * (pa - pb);
    }
};

}  // namespace

// Positive-half unknowns: c[0..K) are the centroids above 0 (K = L/2), the
// cells are [e_i, e_{i+1}] with e_0 = 0, e_i = (c_{i-1}+c_i)/2, e_K = 1.
tq_status lloyd_max_codebook(int d, int bits, double *centroids, double *boundaries,
                             double *residual_out, int max_iters)
{
    // iteration caps: 400 Lloyd sweeps, then 100 Newton steps (max_iters >= 0
    // lowers both, for the host tests of the non-convergence status)
    const int sweeps = max_iters >= 0 && max_iters < 400 ? max_iters : 400;
    const int newton = max_iters >= 0 && max_iters < 100 ? max_iters : 100;
    const int L = 1 << bits, K = L / 2;
    const Density f(d);
    std::vector<double> c(K), e(K + 1), mean(K), mass(K);
    auto evaluate = [&](const std::vector<double> &cc) {
        e[0] = 0.0;
        e[K] = 1.0;
        for (int i = 1; i < K; ++i) e[i] = 0.5 * (cc[i - 1] + cc[i]);
        double worst = 0.0;
        for (int i = 0; i < K; ++i) {
            mass[i] = f.mass(e[i], e[i + 1]);
            mean[i] = f.moment(e[i], e[i + 1]) / mass[i];
            worst = std::fmax(worst, std::fabs(cc[i] - mean[i]));
        }
        return worst;
    };
    // start at the cell means of an equal-width partition of [0, 4/sqrt(d)]
    const double span = std::fmin(4.0 / std::sqrt(static_cast<double>(d)), 0.999);
    for (int i = 0; i < K; ++i) c[i] = span * (i + 0.5) / K;
    double res = evaluate(c);
    for (int sweep = 0; sweep < sweeps && res > 1e-10; ++sweep) {
        c = mean;
        res = evaluate(c);
    }
    // Newton on F = c - mean(c); d mean_i / d e_i = f(e_i)(mean_i - e_i)/mass_i,
    // d mean_i / d e_{i+1} = f(e_{i+1})(e_{i+1} - mean_i)/mass_i, e_0 and e_K fixed.
    std::vector<double> sub(K), dia(K), sup(K), rhs(K), trial(K);
    for (int it = 0; it < newton && res > 1e-15; ++it) {
        for (int i = 0; i < K; ++i) {
            const double lo = (i > 0) ? f.pdf(e[i]) * (mean[i] - e[i]) / mass[i] : 0.0;
            const double hi = (i < K - 1) ? f.pdf(e[i + 1]) * (e[i + 1] - mean[i]) / mass[i] : 0.0;
            sub[i] = -0.5 * lo;
            sup[i] = -0.5 * hi;
            dia[i] = 1.0 - 0.5 * lo - 0.5 * hi;
            rhs[i] = mean[i] - c[i];
        }
        for (int i = 1; i < K; ++i) {
            const double w = sub[i] / dia[i - 1];
            dia[i] -= w * sup[i - 1];
            rhs[i] -= w * rhs[i - 1];
        }
        rhs[K - 1] /= dia[K - 1];
        for (int i = K - 2; i >= 0; --i) rhs[i] = (rhs[i] - sup[i] * rhs[i + 1]) / dia[i];
        double step = 1.0, tres = res;
        bool accepted = false;
        for (int h = 0; h < 40; ++h) {
            bool ordered = true;
            for (int i = 0; i < K; ++i) {
                trial[i] = c[i] + step * rhs[i];
                if (trial[i] <= (i ? trial[i - 1] : 0.0) || trial[i] >= 1.0) ordered = false;
            }
            if (ordered) {
                tres = evaluate(trial);
                if (tres < res) {
                    accepted = true;
                    break;
                }
            }
            step *= 0.5;
        }
        if (!accepted) break;
        c = trial;
        res = tres;
    }
    res = evaluate(c);
    for (int i = 0; i < K; ++i) {
        centroids[K + i] = c[i];
        centroids[K - 1 - i] = -c[i];
    }
    for (int i = 0; i < L - 1; ++i) boundaries[i] = 0.5 * (centroids[i] + centroids[i + 1]);
    boundaries[K - 1] = 0.0;
    if (residual_out) *residual_out = res;
    return (res <= 1e-13) ? TQ_OK : TQ_ENOTCONV;
}

// --------------------------------------------------------------- rotation
void dense_rotation(uint64_t seed, int d, double *pi)
{
    // columns of G, G[i][j] = normal draw i*d + j of stream 0
    std::vector<double> q(static_cast<size_t>(d) * d);   // column-major Q: q[j*d + i]
    std::vector<double> col(d), proj(d);
    for (int j = 0; j < d; ++j) {
        for (int i = 0; i < d; ++i) col[i] = rng_normal(seed, 0, static_cast<uint64_t>(i) * d + j);
        for (int pass = 0; pass < 2; ++pass) {
            for (int p = 0; p < j; ++p) {
                const double *qp = &q[static_cast<size_t>(p) * d];
                double dot = 0.0;
                for (int i = 0; i < d; ++i) dot += qp[i] * col[i];
                proj[p] = dot;
            }
            for (int p = 0; p < j; ++p) {
                const double *qp = &q[static_cast<size_t>(p) * d];
                for (int i = 0; i < d; ++i) col[i] -= proj[p] * qp[i];
            }
        }
        double nrm = 0.0;
        for (int i = 0; i < d; ++i) nrm += col[i] * col[i];
        nrm = std::sqrt(nrm);
        double *qj = &q[static_cast<size_t>(j) * d];
        for (int i = 0; i < d; ++i) qj[i] = col[i] / nrm;
    }
    for (int i = 0; i < d; ++i)
        for (int j = 0; j < d; ++j) pi[static_cast<size_t>(i) * d + j] = q[static_cast<size_t>(j) * d + i];
}

void hadamard_signs(uint64_t seed, int d, float *signs, int stream)
{
    for (int j = 0; j < d; ++j) signs[j] = (rng_draw(seed, stream, j) & 1ULL) ? -1.0f : 1.0f;
}

void hadamard_rotation(uint64_t seed, int d, double *pi, int stream)
{
    std::vector<float> sg(d);
    hadamard_signs(seed, d, sg.data(), stream);
    const double inv = 1.0 / std::sqrt(static_cast<double>(d));
    for (int i = 0; i < d; ++i)
        for (int j = 0; j < d; ++j) {
            const bool odd = __builtin_parity(static_cast<unsigned>(i & j));
            pi[static_cast<size_t>(i) * d + j] = (odd ? -inv : inv) * sg[j];
        }
}

// two rounds: (H D2 / sqrt(d)) (H D1 / sqrt(d)), D1 from stream 1, D2 from stream 3
void hadamard2_rotation(uint64_t seed, int d, double *pi)
{
    std::vector<double> a1(static_cast<size_t>(d) * d), a2(static_cast<size_t>(d) * d);
    hadamard_rotation(seed, d, a1.data(), 1);
    hadamard_rotation(seed, d, a2.data(), 3);
    for (int i = 0; i < d; ++i)
        for (int j = 0; j < d; ++j) {
            double acc = 0.0;
            for (int k = 0; k < d; ++k) acc += a2[static_cast<size_t>(i) * d + k] * a1[static_cast<size_t>(k) * d + j];
            pi[static_cast<size_t>(i) * d + j] = acc;
        }
}

void qjl_projection(uint64_t seed, int m, int d, double *s)
{
    for (int i = 0; i < m; ++i)
        for (int j = 0; j < d; ++j)
            s[static_cast<size_t>(i) * d + j] = rng_normal(seed, 2, static_cast<uint64_t>(i) * d + j);
}

}  // namespace tq

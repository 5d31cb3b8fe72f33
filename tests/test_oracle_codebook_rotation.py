"""Pins of the oracle's random numbers, rotations and Lloyd-Max codebooks.

Each check ties the oracle to something other than itself: a published
reference sequence, a closed form, a library routine (numpy QR, scipy's
incomplete beta and adaptive quadrature, scipy's Hadamard matrix), brute force
on tiny cases, or a Monte-Carlo sample of the distribution the codebook is
built for.
"""
import math
import os

import numpy as np
import pytest
from scipy import integrate, linalg, special, stats

import oracle as O


# ------------------------------------------------------------------ RNG
def test_splitmix_reference_sequence(golden_dir):
    rows = [l for l in open(os.path.join(golden_dir, "splitmix64_seed1234567.txt"))
            if l.strip() and not l.startswith("#")]
    want = [int(x) for x in rows]
    got = [O.splitmix_draw(1234567, 0, k) for k in range(len(want))]
    assert got == want


def test_streams_differ_and_uniform_range():
    a = [O.splitmix_draw(7, 0, k) for k in range(64)]
    b = [O.splitmix_draw(7, 1, k) for k in range(64)]
    assert len(set(a) & set(b)) == 0
    u = np.array([O.uniform(7, 2, k) for k in range(20000)])
    assert u.min() > 0.0 and u.max() <= 1.0
    assert stats.kstest(u, "uniform").pvalue > 1e-3


def test_gaussian_stream_is_standard_normal():
    z = np.array([O.gauss(11, 2, n) for n in range(40000)])
    assert stats.kstest(z, "norm").pvalue > 1e-3
    # cos/sin halves of Box-Muller pairs are uncorrelated
    assert abs(np.corrcoef(z[0::2], z[1::2])[0, 1]) < 0.03


# ------------------------------------------------------------- rotations
@pytest.mark.parametrize("d", [4, 64, 128, 256])
def test_dense_rotation_orthogonal(d):
    pi = O.rotation_dense(1234 + d, d)
    assert np.abs(pi.T @ pi - np.eye(d)).max() < 1e-12
    assert np.abs(pi @ pi.T - np.eye(d)).max() < 1e-12


@pytest.mark.parametrize("d", [8, 128])
def test_dense_rotation_matches_library_qr(d):
    seed = 99
    g = np.array([[O.gauss(seed, 0, i * d + j) for j in range(d)] for i in range(d)])
    q, r = np.linalg.qr(g)
    want = q * np.sign(np.diag(r))[None, :]
    assert np.abs(O.rotation_dense(seed, d) - want).max() < 1e-12


@pytest.mark.parametrize("d", [2, 16, 128, 256])
def test_hadamard_rotation(d):
    seed = 5
    pi = O.rotation_hadamard(seed, d)
    h = linalg.hadamard(d)                       # Sylvester order
    assert np.array_equal(h @ h.T, d * np.eye(d, dtype=h.dtype))
    dsg = O.hadamard_signs(seed, d)
    assert set(np.unique(dsg)) <= {-1.0, 1.0}
    assert np.abs(pi - h * dsg[None, :] / math.sqrt(d)).max() < 1e-15
    assert np.abs(pi.T @ pi - np.eye(d)).max() < 1e-12
    # sign bit is bit 0 of the raw draw of stream 1
    for j in range(d):
        assert dsg[j] == (-1.0 if O.splitmix_draw(seed, 1, j) & 1 else 1.0)


@pytest.mark.parametrize("d", [4, 64, 256])
def test_two_round_hadamard_rotation(d):
    """Pi = (H D2 / sqrt(d)) (H D1 / sqrt(d)): scipy's Hadamard with the sign
    vectors drawn from streams 1 and 3; orthogonal, d Pi integral, and the
    first round is the one-round rotation."""
    seed = 11
    pi = O.rotation_hadamard2(seed, d)
    h = linalg.hadamard(d).astype(np.float64)
    d1 = np.array([-1.0 if O.splitmix_draw(seed, 1, j) & 1 else 1.0 for j in range(d)])
    d2 = np.array([-1.0 if O.splitmix_draw(seed, 3, j) & 1 else 1.0 for j in range(d)])
    want = (h * d2[None, :]) @ (h * d1[None, :]) / d
    assert np.abs(pi - want).max() < 1e-14
    assert np.abs(pi.T @ pi - np.eye(d)).max() < 1e-12
    assert np.abs(pi * d - np.rint(pi * d)).max() < 1e-9
    assert np.abs(pi - (h * d2[None, :] / math.sqrt(d)) @ O.rotation_hadamard(seed, d)).max() < 1e-14
    # at the head dims in use the product is dense-looking (many entry sizes),
    # unlike one round's +-1/sqrt(d) (at d = 4 the two sign draws may cancel)
    if d >= 64:
        assert len(np.unique(np.abs(np.rint(pi * d)))) > 2


def test_qjl_matrix_statistics():
    s = O.qjl_matrix(3, 128, 128)
    assert stats.kstest(s.ravel(), "norm").pvalue > 1e-3
    c = s @ s.T / 128.0
    assert np.abs(np.diag(c) - 1).max() < 0.45
    assert np.abs(c - np.diag(np.diag(c))).max() < 0.45


# ------------------------------------------------------------- codebook
def _closed_mass(d, a, b):
    """P(a < x < b) with x^2 ~ Beta(1/2, (d-1)/2), symmetric in x."""
    def cdf(x):
        return 0.5 + 0.5 * math.copysign(1.0, x) * special.betainc(0.5, (d - 1) / 2.0, x * x)
    return cdf(b) - cdf(a)


def _closed_moment(d, a, b):
    """int_a^b x f_d(x) dx = C_d/(d-1) [(1-a^2)^((d-1)/2) - (1-b^2)^((d-1)/2)]"""
    cd = math.exp(special.gammaln(d / 2.0) - special.gammaln((d - 1) / 2.0)) / math.sqrt(math.pi)
    return cd / (d - 1) * ((1 - a * a) ** ((d - 1) / 2.0) - (1 - b * b) ** ((d - 1) / 2.0))


@pytest.mark.parametrize("d", [3, 8, 128, 256])
def test_cell_moments_match_closed_form(d):
    for a, b in [(-1.0, 1.0), (-0.3, 0.1), (0.05, 0.2), (0.2, 1.0)]:
        m0, m1 = O.cell_moments(d, a, b)
        assert abs(m0 - _closed_mass(d, a, b)) < 1e-13
        assert abs(m1 - _closed_moment(d, a, b)) < 1e-13


@pytest.mark.parametrize("d,bits", [(3, 2), (4, 2), (16, 3), (64, 2), (128, 1), (128, 2),
                                    (128, 3), (128, 4), (256, 2), (256, 7)])
def test_lloyd_max_stationarity_closed_form(d, bits):
    c, t = O.codebook(d, bits)
    L = 1 << bits
    assert np.all(np.diff(c) > 0)
    # symmetric, middle boundary at 0
    assert np.array_equal(c, -c[::-1])
    assert t[L // 2 - 1] == 0.0
    # midpoint condition
    assert np.abs(t - 0.5 * (c[:-1] + c[1:])).max() < 1e-15
    # centroid condition, evaluated with the closed-form numerator and the
    # incomplete-beta mass instead of the oracle's quadrature
    edges = np.concatenate([[-1.0], t, [1.0]])
    for i in range(L):
        mean = _closed_moment(d, edges[i], edges[i + 1]) / _closed_mass(d, edges[i], edges[i + 1])
        assert abs(c[i] - mean) < 1e-12 * max(1.0, math.sqrt(d) * abs(c[i])), (i, c[i], mean)


@pytest.mark.parametrize("bits", [1, 2, 3])
def test_d3_uniform_closed_form(bits):
    # f_3 is uniform on [-1, 1]: levels at -1 + (2i+1)/L
    L = 1 << bits
    c, _ = O.codebook(3, bits)
    assert np.abs(c - (-1.0 + (2 * np.arange(L) + 1) / L)).max() < 1e-13


@pytest.mark.parametrize("d", [3, 4, 17, 128, 256])
def test_one_bit_closed_form(d):
    # b = 1: c = +-E|x| = +-Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2))
    c, t = O.codebook(d, 1)
    want = math.exp(special.gammaln(d / 2) - special.gammaln((d + 1) / 2)) / math.sqrt(math.pi)
    assert abs(c[1] - want) < 1e-14 and abs(c[0] + want) < 1e-14
    assert t[0] == 0.0


def _mse_for_boundary(d, tb):
    """MSE of the symmetric 2-bit quantizer with boundaries (-tb, 0, tb) and
    centroids at the conditional means, by adaptive quadrature."""
    f = lambda x: O.density(d, x) if d != 3 else 0.5
    total = 0.0
    for a, b in [(0.0, tb), (tb, 1.0)]:
        m0 = integrate.quad(f, a, b, epsabs=1e-14, epsrel=1e-13)[0]
        m1 = integrate.quad(lambda x: x * f(x), a, b, epsabs=1e-14, epsrel=1e-13)[0]
        m2 = integrate.quad(lambda x: x * x * f(x), a, b, epsabs=1e-14, epsrel=1e-13)[0]
        total += 2 * (m2 - m1 * m1 / m0)
    return total


@pytest.mark.parametrize("d", [3, 4])
def test_brute_force_two_bit_small_d(d):
    # global search over the one free symmetric boundary, then refine
    grid = np.linspace(0.01, 0.99, 197)
    mse = [_mse_for_boundary(d, g) for g in grid]
    k = int(np.argmin(mse))
    lo, hi = grid[max(k - 1, 0)], grid[min(k + 1, len(grid) - 1)]
    res = __import__("scipy.optimize", fromlist=["x"]).minimize_scalar(
        lambda g: _mse_for_boundary(d, g), bounds=(lo, hi), method="bounded",
        options={"xatol": 1e-10})
    _, t = O.codebook(d, 2)
    assert abs(t[2] - res.x) < 1e-6


@pytest.mark.parametrize("d", [8, 128])
def test_density_matches_random_unit_vectors(d):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((20000, d))
    x = (x / np.linalg.norm(x, axis=1, keepdims=True))[:, 0]
    cdf = np.vectorize(lambda v: O.cell_moments(d, -1.0, v)[0])
    assert stats.kstest(x, cdf).pvalue > 1e-3


def test_large_d_approaches_max_gaussian_table(golden_dir):
    rows = [l.split() for l in open(os.path.join(golden_dir, "max1960_gaussian_lloyd_max.txt"))
            if l.strip() and not l.startswith("#")]
    d = 4096
    for row in rows:
        bits = int(row[0])
        want = np.array([float(v) for v in row[1:]])
        c, _ = O.codebook(d, bits)
        got = math.sqrt(d) * c[len(c) // 2:]
        assert np.abs(got / want - 1).max() < 2e-3, (bits, got, want)

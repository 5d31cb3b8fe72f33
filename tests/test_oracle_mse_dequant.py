"""Pins of the oracle's first-stage (MSE-only, m = 0) key format and of its
explicit key estimates (dequantisation).

The method has two stages ("turboquant-pytorch", section "What it does":
two-stage quantisation): Lloyd-Max codes of the rotated unit key, then one QJL
sign per projection row of the residual.  With m = 0 only the first stage is
stored and the score is n sum_j q_rot_j c[idx_j].  The explicit estimate
k_hat = n Pi^T (c[idx] + sqrt(pi/2)/m rho S^T (2s - 1)) is the vector whose
inner product with a query equals the asymmetric score.
"""
import math

import numpy as np
import pytest

import oracle as O


def _keys(n, d, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal((n, d)) * scale


@pytest.mark.parametrize("d,bits,kind", [(128, 2, "dense"), (64, 3, "hadamard"), (256, 7, "dense")])
def test_first_stage_is_independent_of_qjl(d, bits, kind):
    """Codes and norms do not depend on S; the m = 0 score is the first term of
    the full score on the same packed codes."""
    k = _keys(80, d, 11, 2.0)
    q = np.random.default_rng(12).standard_normal((3, d))
    full = O.rotation(77, d, kind)
    mse = O.rotation(77, d, kind, m=0)
    assert mse.s.shape == (0, d) and np.array_equal(mse.pi, full.pi)
    kf = O.compress_keys(k, bits, full)
    km = O.compress_keys(k, bits, mse)
    assert np.array_equal(kf.codes, km.codes)
    assert np.array_equal(kf.knorm, km.knorm)
    assert km.signs.shape == (80, 0)
    _, t1, _ = O.scores(q, kf, bits, full, terms=True)
    got = O.scores(q, km, bits, mse)
    assert np.all(np.isfinite(got))
    assert np.abs(got - t1).max() <= 1e-13 * np.abs(t1).max()


@pytest.mark.parametrize("d,bits,kind,m", [(128, 2, "dense", None), (128, 3, "hadamard", None),
                                           (64, 4, "dense", None), (256, 7, "dense", None),
                                           (128, 2, "dense", 0), (256, 5, "hadamard", 0)])
def test_dequantised_keys_reproduce_the_scores(d, bits, kind, m):
    """<q, k_hat> equals the oracle's asymmetric score, which the unbiasedness,
    variance and reconstruction pins of the score path fix."""
    rot = O.rotation(21, d, kind, m=m)
    k = _keys(60, d, 5, 4.0)
    q = np.random.default_rng(6).standard_normal((4, d))
    kc = O.compress_keys(k, bits, rot)
    kh = O.dequant_keys(kc, bits, rot)
    got = q @ kh.T
    want = O.scores(q, kc, bits, rot)
    scale = np.linalg.norm(q, axis=1)[:, None] * np.linalg.norm(k, axis=1)[None, :]
    assert np.abs(got - want).max() <= 1e-12 * scale.max()


@pytest.mark.parametrize("d,bits,kind", [(128, 1, "dense"), (128, 3, "dense"), (64, 2, "hadamard"),
                                         (256, 4, "dense")])
def test_first_stage_error_is_the_residual(d, bits, kind):
    """Pi is orthogonal, so k - n Pi^T c[idx] = n Pi^T (y - c[idx]): its norm is
    n rho exactly, and |k_hat| = n |c[idx]|.  A transposed rotation or a wrong
    centroid index fails both."""
    rot = O.rotation(3, d, kind, m=0)
    k = _keys(50, d, 8, 3.0)
    kc = O.compress_keys(k, bits, rot, keep_aux=True)
    kh = O.dequant_keys(kc, bits, rot)
    n = np.linalg.norm(k, axis=1)
    nf = kc.knorm.astype(np.float64)                  # the stored (fp32) norm
    err = np.linalg.norm(k * (nf / n)[:, None] - kh, axis=1)
    assert np.abs(err - nf * kc.rho).max() <= 1e-12 * n.max()
    c, _ = O.codebook(d, bits)
    idx = O.unpack(kc.codes, d, bits)
    assert np.abs(np.linalg.norm(kh, axis=1) - kc.knorm * np.linalg.norm(c[idx], axis=1)).max() <= 1e-12 * n.max()
    # the estimate points along the key: cosine well above that of a random vector
    cos = np.sum(k * kh, axis=1) / (n * np.linalg.norm(kh, axis=1))
    assert cos.min() > (0.7 if bits == 1 else 0.9)       # 1 bit: about sqrt(2/pi)


def test_full_estimate_is_unbiased_per_coordinate():
    """Averaged over independent (Pi, S), the full estimate of one key is the key
    (each coordinate of k_hat is an inner product <e_c, k_hat>, so the QJL
    unbiasedness carries over); the first-stage estimate shrinks towards zero."""
    d, bits, n_seeds = 64, 2, 400
    k = _keys(1, d, 99, 1.0)
    full = np.zeros(d)
    mse = np.zeros(d)
    sq = np.zeros(d)
    for s in range(n_seeds):
        rf = O.rotation(5000 + s, d)
        rm = O.rotation(5000 + s, d, m=0)
        kf = O.dequant_keys(O.compress_keys(k, bits, rf), bits, rf)[0]
        km = O.dequant_keys(O.compress_keys(k, bits, rm), bits, rm)[0]
        full += kf
        sq += kf * kf
        mse += km
    full /= n_seeds
    mse /= n_seeds
    sd = np.sqrt(np.maximum(sq / n_seeds - full * full, 1e-30))
    z = (full - k[0]) / (sd / math.sqrt(n_seeds))
    assert np.abs(z).max() < 4.5, np.abs(z).max()
    # first stage alone: the mean estimate is a shrunk copy of the key
    ratio = float(mse @ k[0]) / float(k[0] @ k[0])
    assert 0.7 < ratio < 0.99, ratio

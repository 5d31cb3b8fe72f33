"""Pins of the oracle's rotated scalar block formats (Q8_0 / Q4_0 with a
rotation, the comparison the tproger.ru article reports in its section
"First benchmarks"): 32-value blocks of the rotated key, one fp16 scale each.

Checks: brute-force nearest integer per coordinate, the scale rule against
numpy float16, the zero key, the score identity against an independent
numpy reconstruction, attention against a numpy softmax, and the page's
qualitative claim that 8-bit blocks with rotation are nearly lossless and
better than without rotation on keys with outlier channels."""
import numpy as np
import pytest

import oracle as O


def _decode_numpy(kc, bits, d):
    """x_hat from the packed planes with numpy only (independent unpacking)."""
    n = kc.codes.shape[0]
    if bits == 8:
        q = kc.codes.view(np.int8).astype(np.float64)
    else:
        lo = (kc.codes & 0x0F).astype(np.int64)
        hi = (kc.codes >> 4).astype(np.int64)
        q = np.empty((n, d))
        q[:, 0::2] = lo - 8
        q[:, 1::2] = hi - 8
    s = kc.scales.view(np.float16).astype(np.float64)
    return q * np.repeat(s, 32, axis=1)


@pytest.mark.parametrize("bits,d,kind", [(8, 128, "dense"), (4, 128, "hadamard"), (8, 256, "dense"),
                                         (4, 64, "dense")])
def test_block_codes_are_the_nearest_integers(bits, d, kind):
    rot = O.rotation(9, d, kind)
    k = np.random.default_rng(bits * d).standard_normal((40, d)) * 3.0
    kc = O.compress_keys_block(k, bits, rot.pi, keep_aux=True)
    x = k @ rot.pi.T
    assert np.abs(x - kc.x).max() < 1e-12 * np.abs(x).max()
    qmax = 127 if bits == 8 else 7
    # the scale: fp16 of the block's largest magnitude over qmax (numpy rounding)
    amax = np.abs(x.reshape(40, d // 32, 32)).max(axis=2)
    assert np.array_equal(kc.scales, (amax / qmax).astype(np.float16).view(np.uint16))
    s = np.repeat(kc.scales.view(np.float16).astype(np.float64), 32, axis=1)
    # brute force over every allowed integer, off exact ties
    cand = np.arange(-qmax, qmax + 1, dtype=np.float64)
    err = np.abs(x[:, :, None] - s[:, :, None] * cand[None, None, :])
    best = cand[np.argmin(err, axis=2)]
    got = _decode_numpy(kc, bits, d) / s
    frac = np.abs(kc.quot - np.floor(kc.quot) - 0.5)
    off_tie = frac > 1e-9
    assert np.array_equal(got[off_tie], best[off_tie])
    assert np.abs(_decode_numpy(kc, bits, d) - x).max() <= 0.5 * s.max() * (1 + 1e-3)


def test_zero_key_and_block():
    d = 128
    rot = O.rotation(3, d)
    k = np.zeros((2, d))
    k[1, :] = 1.0                      # non-zero key, but compare its blocks too
    for bits in (8, 4):
        kc = O.compress_keys_block(k, bits, rot.pi)
        assert np.all(kc.scales[0] == 0)
        assert np.all(_decode_numpy(kc, bits, d)[0] == 0.0)
        assert np.all(O.dequant_keys_block(kc, bits, rot.pi)[0] == 0.0)


@pytest.mark.parametrize("bits,d,kind", [(8, 128, "dense"), (4, 256, "hadamard")])
def test_block_scores_equal_inner_products_with_numpy_reconstruction(bits, d, kind):
    rot = O.rotation(17, d, kind)
    rng = np.random.default_rng(5)
    k = rng.standard_normal((50, d)) * 2.0
    q = rng.standard_normal((3, d))
    kc = O.compress_keys_block(k, bits, rot.pi)
    khat = _decode_numpy(kc, bits, d) @ rot.pi          # Pi^T x_hat, row-wise
    want = q @ khat.T
    got = O.scores_block(q, kc, bits, rot.pi)
    assert np.abs(got - want).max() <= 1e-12 * np.abs(want).max()
    assert np.abs(O.dequant_keys_block(kc, bits, rot.pi) - khat).max() <= 1e-12 * np.abs(khat).max()


def test_block_attention_is_softmax_of_scores():
    d, bits = 128, 8
    rot = O.rotation(23, d)
    rng = np.random.default_rng(6)
    k = rng.standard_normal((90, d))
    v = rng.standard_normal((90, d)).astype(np.float32).astype(np.float64)
    q = rng.standard_normal((4, d))
    kc = O.compress_keys_block(k, bits, rot.pi)
    vc = O.compress_values(v, 4, 32)
    out = O.attend_block(q, kc, bits, rot.pi, vc, 4, 32)
    lam = O.scores_block(q, kc, bits, rot.pi) / np.sqrt(d)
    p = np.exp(lam - lam.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    want = p @ O.dequant_values(vc, d, 4, 32)
    assert np.abs(out - want).max() < 1e-12


def test_rotation_and_block_error_on_outlier_channels():
    """The page reports Q8_0 with rotation as nearly lossless and better than
    Q8_0 without it (model accuracy).  On keys with a few large channels (the
    K-tensor statistics the page describes) the inner-product error of 8-bit
    blocks against random queries drops with rotation and stays below 1 %.
    (The page's 4-bit gain is an accuracy figure of a real model; on these
    synthetic keys rotation does not lower the 4-bit L2 error, so only a
    bound is checked there.)"""
    d, n = 128, 400
    rng = np.random.default_rng(7)
    sig = np.exp(rng.standard_normal(d))
    sig[rng.choice(d, 4, replace=False)] *= 20.0
    k = rng.standard_normal((n, d)) * sig
    q = rng.standard_normal((64, d))
    rot = O.rotation(31, d)
    eye = np.eye(d)

    def ip_err(bits, pi):
        kc = O.compress_keys_block(k, bits, pi)
        kh = O.dequant_keys_block(kc, bits, pi)
        ip, iph = q @ k.T, q @ kh.T
        return np.sqrt(((ip - iph) ** 2).mean() / (ip ** 2).mean())

    e8_plain, e8_rot = ip_err(8, eye), ip_err(8, rot.pi)
    assert e8_rot < e8_plain / 1.4, (e8_rot, e8_plain)
    assert e8_rot < 0.01, e8_rot
    assert ip_err(4, rot.pi) < 0.2

"""Shared helpers of the GPU parity tests: run libtq through its binding, run
the oracle on the same seeded inputs, and compare under the stated bars.

Bars (applied element by element):
  codes, signs  bit-exact, except coordinates within 1e-5 of a decision
                boundary (|y - t_i| for codes, |z_i| for signs); such flips are
                counted and must be at most 1e-4 of all coordinates.  A code
                flipped at a boundary moves to the adjacent cell, which changes
                that key's residual: its signs and ||r|| are then compared with
                the oracle's encoding under that other tie resolution.
  knorm         relative 1e-6;  rnorm  relative 1e-5
  value codes   bit-exact except quotients within 1e-5 of a half-integer;
  value params  bit-exact
  scores        |gpu - oracle| <= 1e-4 ||q|| ||k||, on the oracle's own packed cache
  attention     |gpu - oracle| <= 1e-3, on the oracle's own packed cache
"""
from __future__ import annotations

import numpy as np

import attention_decode_amd as tq
import oracle as O

FLIP_DIST = 1e-5
FLIP_FRAC = 1e-4
SCORE_TOL = 1e-4
ATTN_TOL = 1e-3


def unpack_le(packed: np.ndarray, per_vec: int, width: int) -> np.ndarray:
    packed = packed.reshape(-1, packed.shape[-1])
    bits = np.unpackbits(packed, axis=1, bitorder="little")[:, : per_vec * width]
    bits = bits.reshape(packed.shape[0], per_vec, width).astype(np.uint32)
    return (bits << np.arange(width, dtype=np.uint32)).sum(axis=2)


def f64(t) -> np.ndarray:
    return t.detach().double().cpu().numpy()


class Formats:
    """libtq handles and oracle matrices for one (workload, layer)."""

    def __init__(self, w, layer=0):
        seed = w.rotation_seed(layer)
        self.w = w
        self.cb = tq.tq_build_codebook(w.d, w.k_bits)
        self.rot = tq.tq_make_rotation(seed, w.d, w.rot)
        self.kf = tq.KeyFormat(w.d, w.k_bits, self.cb, self.rot)
        self.vf = tq.ValueFormat(w.d, w.v_bits, w.group)
        self.orot = O.rotation(seed, w.d, w.rot)
        self.centroids, self.boundaries = O.codebook(w.d, w.k_bits)


def gpu_compress(fm: Formats, k, v):
    w = fm.w
    B, H, T, _ = k.shape
    kc = tq.alloc_key_cache(fm.kf, B, H, T, device=k.device)
    vc = tq.alloc_value_cache(fm.vf, B, H, T, device=v.device)
    tq.tq_compress_keys(fm.kf, k, kc)
    tq.tq_compress_values(fm.vf, v, vc)
    return kc, vc


def _rows_of(plane, row_index, ndim: int) -> np.ndarray:
    """Rows of a packed plane (torch, any device) as numpy: the plane viewed
    with `ndim` dimensions (rows first), gathered on the plane's device when
    row_index is given, so that a few rows of a multi-GB plane cost little."""
    import torch
    shape = (-1,) + tuple(plane.shape[-(ndim - 1):]) if ndim > 1 else (-1,)
    flat = plane.reshape(shape)
    if row_index is not None:
        flat = flat.index_select(0, torch.as_tensor(np.asarray(row_index, dtype=np.int64), device=plane.device))
    return flat.cpu().numpy()


def compare_keys(fm: Formats, kc, rows_k: np.ndarray, row_index=None):
    """kc: libtq key planes (torch); rows_k: [N, d] fp64 inputs of the rows to
    check; row_index: flat row numbers of those rows in kc (default: all)."""
    w = fm.w
    d, bits = w.d, w.k_bits
    ok = O.compress_keys(rows_k, bits, fm.orot, keep_aux=True)
    g_codes = _rows_of(kc.codes, row_index, 2)
    g_kn = _rows_of(kc.knorm, row_index, 1)
    n = rows_k.shape[0]
    gi, oi = unpack_le(g_codes, d, bits), unpack_le(ok.codes, d, bits)
    # distance of each rotated coordinate to its nearest boundary, without an
    # [n, d, L - 1] temporary (boundaries are sorted)
    pos = np.searchsorted(fm.boundaries, ok.y)
    lo = fm.boundaries[np.clip(pos - 1, 0, fm.boundaries.size - 1)]
    hi = fm.boundaries[np.clip(pos, 0, fm.boundaries.size - 1)]
    dist = np.minimum(np.abs(ok.y - lo), np.abs(ok.y - hi))
    code_flip = gi != oi
    assert np.all(dist[code_flip] < FLIP_DIST), f"code mismatch away from a boundary: {dist[code_flip].max()}"
    # a boundary coordinate may take either adjacent cell, nothing else
    assert np.all(np.abs(gi[code_flip].astype(np.int64) - oi[code_flip].astype(np.int64)) == 1)
    kn_ref = ok.knorm.astype(np.float64)
    assert np.all(np.abs(g_kn - kn_ref) <= 1e-6 * np.maximum(kn_ref, 1e-30)), "knorm"
    if kc.signs is None:
        # first-stage format: codes and ||k|| only
        flips = int(code_flip.sum())
        assert flips <= FLIP_FRAC * n * d, f"{flips} flips over {n * d} coordinates"
        return {"code_flips": flips, "sign_flips": 0, "flipped_keys": int(code_flip.any(axis=1).sum()),
                "coords": n * d}
    g_signs = _rows_of(kc.signs, row_index, 2)
    g_rn = _rows_of(kc.rnorm, row_index, 1)
    flipped_key = code_flip.any(axis=1)
    # reference signs and ||r||: the oracle's encoding, or for a key with a
    # boundary flip the oracle's encoding under the other tie resolution
    ref_signs = ok.signs.copy()
    ref_z = ok.z.copy()
    ref_rho = ok.rho.copy()
    for r in np.nonzero(flipped_key)[0]:
        alt = oi[r].copy()
        alt[code_flip[r]] = gi[r][code_flip[r]]
        ref_signs[r], ref_z[r], ref_rho[r] = O.key_residual_signs(ok.y[r], alt, bits, fm.orot)
    gs, rs = unpack_le(g_signs, d, 1), unpack_le(ref_signs, d, 1)
    sign_flip = gs != rs
    assert np.all(np.abs(ref_z[sign_flip]) < FLIP_DIST), \
        f"sign mismatch away from z = 0: {np.abs(ref_z[sign_flip]).max()}"
    flips = int(code_flip.sum() + sign_flip.sum())
    assert flips <= FLIP_FRAC * n * d * 2, f"{flips} flips over {n * d * 2} coordinates"
    rel = np.abs(g_rn - ref_rho) / np.maximum(ref_rho, 1e-30)
    assert np.all(rel <= 1e-5), f"rnorm max rel {rel.max()}"
    return {"code_flips": int(code_flip.sum()), "sign_flips": int(sign_flip.sum()),
            "flipped_keys": int(flipped_key.sum()), "coords": n * d * 2}


def compare_keys_chunked(fm: Formats, kc, rows_k: np.ndarray, row_index: np.ndarray, chunk: int = 65536):
    """compare_keys over many rows in pieces (the oracle's auxiliary arrays of
    a whole 2^20-token slice would take gigabytes); flips are summed, and the
    flip budget is checked on each piece and on the total."""
    tot = {"code_flips": 0, "sign_flips": 0, "flipped_keys": 0, "coords": 0}
    for lo in range(0, rows_k.shape[0], chunk):
        st = compare_keys(fm, kc, rows_k[lo:lo + chunk], row_index=row_index[lo:lo + chunk])
        for key in tot:
            tot[key] += st[key]
    assert tot["code_flips"] + tot["sign_flips"] <= FLIP_FRAC * tot["coords"]
    return tot


def compare_values(fm: Formats, vc, rows_v: np.ndarray, row_index=None):
    w = fm.w
    d = w.d
    ov = O.compress_values(rows_v, w.v_bits, w.group, keep_aux=True)
    g_codes = _rows_of(vc.codes, row_index, 2)
    g_par = _rows_of(vc.params.reshape(-1, d // w.group, 2), row_index, 3).view(np.uint16)
    assert np.array_equal(g_par, ov.params), "value scale/zero differ"
    gi, oi = unpack_le(g_codes, d, w.v_bits), unpack_le(ov.codes, d, w.v_bits)
    mism = gi != oi
    halfdist = np.abs(ov.quot - (np.floor(ov.quot) + 0.5))
    assert np.all(halfdist[mism] < FLIP_DIST), "value code mismatch away from a tie"
    assert mism.sum() <= FLIP_FRAC * mism.size
    return int(mism.sum())


def to_device_cache(ok, ov, shape_bht, device):
    """Upload oracle-packed planes as libtq cache tensors."""
    import torch
    B, H, T = shape_bht
    kc = tq.KeyCache(torch.from_numpy(ok.codes).reshape(B, H, T, -1).to(device),
                     torch.from_numpy(ok.signs).reshape(B, H, T, -1).to(device),
                     torch.from_numpy(ok.knorm).reshape(B, H, T).to(device),
                     torch.from_numpy(ok.rnorm).reshape(B, H, T).to(device))
    vc = None
    if ov is not None:
        vc = tq.ValueCache(torch.from_numpy(ov.codes).reshape(B, H, T, -1).to(device),
                           torch.from_numpy(ov.params.view(np.int16)).reshape(B, H, T, -1, 2).to(device))
    return kc, vc


def oracle_units(fm: Formats, q: np.ndarray, ok, ov, shape_bht, want_attn=True):
    """Oracle scores [B, Hq, T] and attention [B, Hq, d] over every (b, h_kv)."""
    w = fm.w
    B, H, T = shape_bht
    G = q.shape[1] // H
    d = w.d
    codes = ok.codes.reshape(B, H, T, -1)
    signs = ok.signs.reshape(B, H, T, -1)
    kn = ok.knorm.reshape(B, H, T)
    rn = ok.rnorm.reshape(B, H, T)
    sc = np.zeros((B, H * G, T))
    at = np.zeros((B, H * G, d))
    for b in range(B):
        for h in range(H):
            kc = O.KeyCache(codes[b, h], signs[b, h], kn[b, h], rn[b, h])
            qq = q[b, h * G:(h + 1) * G]
            sc[b, h * G:(h + 1) * G] = O.scores(qq, kc, w.k_bits, fm.orot)
            if want_attn:
                vc = O.ValueCache(ov.codes.reshape(B, H, T, -1)[b, h],
                                  ov.params.reshape(B, H, T, -1, 2)[b, h])
                at[b, h * G:(h + 1) * G] = O.attend(qq, kc, w.k_bits, fm.orot, vc, w.v_bits, w.group)
    return sc, at


def check_scores(gpu_sc: np.ndarray, ora_sc: np.ndarray, q: np.ndarray, knorm_bht: np.ndarray, H: int):
    B, Hq, T = ora_sc.shape
    G = Hq // H
    qn = np.linalg.norm(q, axis=-1)                                  # [B, Hq]
    kn = np.repeat(knorm_bht.astype(np.float64), G, axis=1)          # [B, Hq, T]
    bound = SCORE_TOL * qn[:, :, None] * kn
    err = np.abs(gpu_sc - ora_sc)
    assert np.all(err <= bound + 1e-30), f"score error {np.max(err / np.maximum(bound, 1e-30))} x bound"
    return float(np.max(err / np.maximum(bound, 1e-30)))


def check_attention(gpu_out: np.ndarray, ora_out: np.ndarray):
    err = np.abs(gpu_out - ora_out)
    assert np.all(err <= ATTN_TOL), f"attention max abs error {err.max()}"
    return float(err.max())


def attention_rel_err(gpu_out: np.ndarray, ora_out: np.ndarray) -> float:
    """Largest error relative to the row's largest output magnitude (reported
    beside the absolute bar: near-uniform softmaxes over long caches give
    outputs of order 1/sqrt(T), where 1e-3 absolute says little)."""
    scale = np.maximum(np.abs(ora_out).max(axis=-1, keepdims=True), 1e-30)
    return float((np.abs(gpu_out - ora_out) / scale).max())

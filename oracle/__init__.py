"""fp64 CPU oracle for the TurboQuant KV-cache hot path (numpy driver).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The arithmetic lives in
``tq_oracle.c`` (plain fp64 scalar loops); this module only builds that file
with gcc, marshals numpy arrays through ctypes and unpacks bit-streams.  It
shares no code with the GPU library and imports nothing from it.

Method (pages "turboquant-pytorch", section "What it does", and the discosf.com
TurboQuant article, section "TurboQuant in one sentence", steps 1-4): keys are
normalised, rotated by a random orthogonal matrix, quantised per coordinate
with a Lloyd-Max codebook, and the residual keeps one QJL sign per projection
row; values are min-max quantised per group to 2 or 4 bits and packed; decode
scores the query directly against the packed keys.

Every function is pinned by tests/test_oracle_*.py against closed forms, brute
force, library routines or figures printed on the pages.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# an instrumented build of tq_oracle.c (sanitizer runs) may stand in for it
_LIB_OVERRIDE = os.environ.get("TQ_ORACLE_LIB")
_lib = None

_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_u32p = np.ctypeslib.ndpointer(dtype=np.uint32, flags="C_CONTIGUOUS")


def build(force: bool = False) -> str:
    """Compile tq_oracle.c with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _l():
    global _lib
    if _lib is not None:
        return _lib
    lib = ctypes.CDLL(_LIB_OVERRIDE or build())
    u64, i32, i64 = ctypes.c_uint64, ctypes.c_int, ctypes.c_int64
    vp = ctypes.c_void_p
    lib.orc_splitmix_draw.restype = u64
    lib.orc_splitmix_draw.argtypes = [u64, i32, u64]
    lib.orc_uniform.restype = ctypes.c_double
    lib.orc_uniform.argtypes = [u64, i32, u64]
    lib.orc_gauss.restype = ctypes.c_double
    lib.orc_gauss.argtypes = [u64, i32, u64]
    lib.orc_f64_to_f16.restype = ctypes.c_uint16
    lib.orc_f64_to_f16.argtypes = [ctypes.c_double]
    lib.orc_f16_to_f64.restype = ctypes.c_double
    lib.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.orc_rotation_dense.argtypes = [u64, i32, _f64p]
    lib.orc_rotation_hadamard.argtypes = [u64, i32, _f64p]
    lib.orc_rotation_hadamard2.argtypes = [u64, i32, _f64p]
    lib.orc_hadamard_signs.argtypes = [u64, i32, _f64p]
    lib.orc_qjl_matrix.argtypes = [u64, i32, i32, _f64p]
    lib.orc_density.restype = ctypes.c_double
    lib.orc_density.argtypes = [i32, ctypes.c_double]
    lib.orc_cell_moments.argtypes = [i32, ctypes.c_double, ctypes.c_double,
                                     ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    lib.orc_codebook.restype = i32
    lib.orc_codebook.argtypes = [i32, i32, _f64p, _f64p, ctypes.POINTER(ctypes.c_double)]
    lib.orc_pack.argtypes = [_u32p, i64, i32, i32, _u8p]
    lib.orc_unpack.argtypes = [_u8p, i64, i32, i32, _u32p]
    lib.orc_compress_keys.argtypes = [i32, i32, i32, _f64p, _f64p, _f64p, _f64p, _f64p, i64,
                                      _u8p, _u8p, _f32p, _f32p, vp, vp, vp]
    lib.orc_key_residual_signs.argtypes = [i32, i32, _f64p, _f64p, _f64p, _u32p, _u8p, _f64p,
                                           ctypes.POINTER(ctypes.c_double)]
    lib.orc_compress_values.argtypes = [i32, i32, i32, _f64p, i64, _u8p, _u16p, vp]
    lib.orc_dequant_values.argtypes = [i32, i32, i32, _u8p, _u16p, i64, _f64p]
    lib.orc_scores.argtypes = [i32, i32, i32, _f64p, _f64p, _f64p, _f64p, i32,
                               _u8p, _u8p, _f32p, _f32p, i64, _f64p, vp, vp]
    lib.orc_dequant_keys.argtypes = [i32, i32, i32, _f64p, _f64p, _f64p, _u8p, _u8p, _f32p, _f32p,
                                     i64, _f64p]
    lib.orc_compress_keys_block.argtypes = [i32, i32, _f64p, _f64p, i64, _u8p, _u16p, vp, vp]
    lib.orc_scores_block.argtypes = [i32, i32, _f64p, _f64p, i32, _u8p, _u16p, i64, _f64p]
    lib.orc_dequant_keys_block.argtypes = [i32, i32, _f64p, _u8p, _u16p, i64, _f64p]
    lib.orc_attend_block.argtypes = [i32, i32, _f64p, _f64p, i32, _u8p, _u16p, i64, i32, i32, _u8p, _u16p,
                                     ctypes.c_double, _f64p]
    lib.orc_attend.argtypes = [i32, i32, i32, _f64p, _f64p, _f64p, _f64p, i32,
                               _u8p, _u8p, _f32p, _f32p, i64, i32, i32, _u8p, _u16p,
                               ctypes.c_double, _f64p]
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# --------------------------------------------------------------------------- RNG
def splitmix_draw(seed: int, stream: int, k: int) -> int:
    return int(_l().orc_splitmix_draw(seed, stream, k))


def uniform(seed: int, stream: int, k: int) -> float:
    return float(_l().orc_uniform(seed, stream, k))


def gauss(seed: int, stream: int, n: int) -> float:
    return float(_l().orc_gauss(seed, stream, n))


# ---------------------------------------------------------------------- fp16
def f64_to_f16_bits(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    f = _l().orc_f64_to_f16
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.uint16).reshape(x.shape)


def f16_bits_to_f64(h) -> np.ndarray:
    h = np.asarray(h, dtype=np.uint16)
    f = _l().orc_f16_to_f64
    return np.array([f(int(v)) for v in h.ravel()], dtype=np.float64).reshape(h.shape)


# ----------------------------------------------------------------- rotations
def rotation_dense(seed: int, d: int) -> np.ndarray:
    pi = np.zeros((d, d))
    _l().orc_rotation_dense(seed, d, pi)
    return pi


def rotation_hadamard(seed: int, d: int) -> np.ndarray:
    pi = np.zeros((d, d))
    _l().orc_rotation_hadamard(seed, d, pi)
    return pi


def rotation_hadamard2(seed: int, d: int) -> np.ndarray:
    pi = np.zeros((d, d))
    _l().orc_rotation_hadamard2(seed, d, pi)
    return pi


def hadamard_signs(seed: int, d: int) -> np.ndarray:
    s = np.zeros(d)
    _l().orc_hadamard_signs(seed, d, s)
    return s


def qjl_matrix(seed: int, m: int, d: int) -> np.ndarray:
    s = np.zeros((m, d))
    _l().orc_qjl_matrix(seed, m, d, s)
    return s


@dataclass
class Rotation:
    seed: int
    d: int
    kind: str          # "dense" | "hadamard" | "hadamard2"
    pi: np.ndarray     # d x d, y = pi @ u
    s: np.ndarray      # m x d QJL projection


def rotation(seed: int, d: int, kind: str = "dense", m: int | None = None) -> Rotation:
    """Pi and S of a seed; m = 0 gives the key format without the QJL stage."""
    m = d if m is None else m
    pi = {"dense": rotation_dense, "hadamard": rotation_hadamard, "hadamard2": rotation_hadamard2}[kind](seed, d)
    return Rotation(seed, d, kind, pi, qjl_matrix(seed, m, d))


# ------------------------------------------------------------------ codebook
def density(d: int, x: float) -> float:
    return float(_l().orc_density(d, x))


def cell_moments(d: int, a: float, b: float):
    m0, m1 = ctypes.c_double(), ctypes.c_double()
    _l().orc_cell_moments(d, a, b, ctypes.byref(m0), ctypes.byref(m1))
    return m0.value, m1.value


_cb_cache: dict = {}


def codebook(d: int, bits: int):
    """(centroids[2^b], boundaries[2^b - 1]) of the Lloyd-Max quantizer for f_d."""
    key = (d, bits)
    if key not in _cb_cache:
        L = 1 << bits
        c = np.zeros(L)
        t = np.zeros(L - 1)
        res = ctypes.c_double()
        it = _l().orc_codebook(d, bits, c, t, ctypes.byref(res))
        if it < 0:
            raise RuntimeError(f"oracle Lloyd-Max did not converge for d={d} b={bits} (res {res.value})")
        _cb_cache[key] = (c, t)
    c, t = _cb_cache[key]
    return c.copy(), t.copy()


# ------------------------------------------------------------------- packing
def pack(vals: np.ndarray, width: int) -> np.ndarray:
    vals = np.ascontiguousarray(vals, dtype=np.uint32)
    n, per = vals.shape
    out = np.zeros((n, (per * width + 7) // 8), dtype=np.uint8)
    _l().orc_pack(vals, n, per, width, out)
    return out


def unpack(packed: np.ndarray, per_vec: int, width: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    n = packed.shape[0]
    out = np.zeros((n, per_vec), dtype=np.uint32)
    _l().orc_unpack(packed, n, per_vec, width, out)
    return out


# ---------------------------------------------------------------------- keys
@dataclass
class KeyCache:
    codes: np.ndarray   # [N, d*b/8] u8
    signs: np.ndarray   # [N, m/8] u8
    knorm: np.ndarray   # [N] f32
    rnorm: np.ndarray   # [N] f32
    y: np.ndarray | None = None    # [N, d] rotated unit vector (fp64)
    z: np.ndarray | None = None    # [N, m] QJL projection of the residual (fp64)
    rho: np.ndarray | None = None  # [N] residual norm before fp32 rounding


def compress_keys(k: np.ndarray, bits: int, rot: Rotation, keep_aux: bool = False) -> KeyCache:
    k = np.ascontiguousarray(k, dtype=np.float64)
    n, d = k.shape
    m = rot.s.shape[0]
    c, t = codebook(d, bits)
    codes = np.zeros((n, (d * bits + 7) // 8), np.uint8)
    signs = np.zeros((n, (m + 7) // 8), np.uint8)
    kn = np.zeros(n, np.float32)
    rn = np.zeros(n, np.float32)
    y = np.zeros((n, d)) if keep_aux else None
    z = np.zeros((n, m)) if keep_aux else None
    rho = np.zeros(n) if keep_aux else None
    _l().orc_compress_keys(d, bits, m, np.ascontiguousarray(rot.pi), np.ascontiguousarray(rot.s),
                           c, t, k, n, codes, signs, kn, rn, _ptr(y), _ptr(z), _ptr(rho))
    return KeyCache(codes, signs, kn, rn, y, z, rho)


def key_residual_signs(y: np.ndarray, idx: np.ndarray, bits: int, rot: Rotation):
    """Signs (packed), z and ||r|| of one key for rotated vector y and codes idx."""
    d = y.shape[0]
    m = rot.s.shape[0]
    c, _ = codebook(d, bits)
    signs = np.zeros((m + 7) // 8, np.uint8)
    z = np.zeros(m)
    rho = ctypes.c_double()
    _l().orc_key_residual_signs(d, m, np.ascontiguousarray(rot.s), c, np.ascontiguousarray(y, np.float64),
                                np.ascontiguousarray(idx, np.uint32), signs, z, ctypes.byref(rho))
    return signs, z, rho.value


# -------------------------------------------------------------------- values
@dataclass
class ValueCache:
    codes: np.ndarray    # [N, d*b/8] u8
    params: np.ndarray   # [N, d/g, 2] u16 fp16 bit patterns (scale, zero)
    quot: np.ndarray | None = None


def compress_values(v: np.ndarray, bits: int, group: int, keep_aux: bool = False) -> ValueCache:
    v = np.ascontiguousarray(v, dtype=np.float64)
    n, d = v.shape
    codes = np.zeros((n, (d * bits + 7) // 8), np.uint8)
    params = np.zeros((n, d // group, 2), np.uint16)
    quot = np.zeros((n, d)) if keep_aux else None
    _l().orc_compress_values(d, bits, group, v, n, codes, params, _ptr(quot))
    return ValueCache(codes, params, quot)


def dequant_values(vc: ValueCache, d: int, bits: int, group: int) -> np.ndarray:
    n = vc.codes.shape[0]
    out = np.zeros((n, d))
    _l().orc_dequant_values(d, bits, group, np.ascontiguousarray(vc.codes),
                            np.ascontiguousarray(vc.params), n, out)
    return out


# ------------------------------------------------------------ scores / attend
def scores(q: np.ndarray, kc: KeyCache, bits: int, rot: Rotation, terms: bool = False):
    """q [nq, d] against one KV head's packed keys -> scores [nq, T] (fp64)."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    nq, d = q.shape
    m = rot.s.shape[0]
    T = kc.codes.shape[0]
    c, _ = codebook(d, bits)
    out = np.zeros((nq, T))
    t1 = np.zeros((nq, T)) if terms else None
    t2 = np.zeros((nq, T)) if terms else None
    _l().orc_scores(d, bits, m, np.ascontiguousarray(rot.pi), np.ascontiguousarray(rot.s), c, q, nq,
                    np.ascontiguousarray(kc.codes), np.ascontiguousarray(kc.signs),
                    np.ascontiguousarray(kc.knorm), np.ascontiguousarray(kc.rnorm), T, out,
                    _ptr(t1), _ptr(t2))
    return (out, t1, t2) if terms else out


def dequant_keys(kc: KeyCache, bits: int, rot: Rotation) -> np.ndarray:
    """Explicit key estimates k_hat [N, d] (fp64) of one packed key plane set:
    the vectors whose inner products with a query are the asymmetric scores;
    a rotation with m = 0 rows of S gives the first (MSE) stage alone."""
    d = rot.d
    m = rot.s.shape[0]
    n = kc.codes.shape[0]
    c, _ = codebook(d, bits)
    out = np.zeros((n, d))
    signs = kc.signs if m > 0 else np.zeros((n, 1), np.uint8)
    _l().orc_dequant_keys(d, bits, m, np.ascontiguousarray(rot.pi), np.ascontiguousarray(rot.s), c,
                          np.ascontiguousarray(kc.codes), np.ascontiguousarray(signs),
                          np.ascontiguousarray(kc.knorm), np.ascontiguousarray(kc.rnorm), n, out)
    return out


def attend(q: np.ndarray, kc: KeyCache, bits: int, rot: Rotation, vc: ValueCache,
           vbits: int, group: int, scale: float | None = None) -> np.ndarray:
    """Decode attention of q [nq, d] over one KV head's packed cache -> [nq, d]."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    nq, d = q.shape
    m = rot.s.shape[0]
    T = kc.codes.shape[0]
    c, _ = codebook(d, bits)
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    out = np.zeros((nq, d))
    _l().orc_attend(d, bits, m, np.ascontiguousarray(rot.pi), np.ascontiguousarray(rot.s), c, q, nq,
                    np.ascontiguousarray(kc.codes), np.ascontiguousarray(kc.signs),
                    np.ascontiguousarray(kc.knorm), np.ascontiguousarray(kc.rnorm), T,
                    vbits, group, np.ascontiguousarray(vc.codes), np.ascontiguousarray(vc.params),
                    float(scale), out)
    return out


# ------------------------------------------------- rotated block formats
@dataclass
class BlockKeyCache:
    codes: np.ndarray    # [N, d*bits/8] u8: int8 codes (8 bits) or q + 8 nibbles (4 bits)
    scales: np.ndarray   # [N, d/32] u16 fp16 bit patterns
    x: np.ndarray | None = None      # [N, d] rotated key (fp64)
    quot: np.ndarray | None = None   # [N, d] x / scale before rounding


def compress_keys_block(k: np.ndarray, bits: int, pi: np.ndarray, keep_aux: bool = False) -> BlockKeyCache:
    """Rotated Q8_0 (bits 8) / Q4_0 (bits 4) keys: x = pi @ k, 32-value blocks."""
    k = np.ascontiguousarray(k, dtype=np.float64)
    n, d = k.shape
    codes = np.zeros((n, d * bits // 8), np.uint8)
    scales = np.zeros((n, d // 32), np.uint16)
    x = np.zeros((n, d)) if keep_aux else None
    quot = np.zeros((n, d)) if keep_aux else None
    _l().orc_compress_keys_block(d, bits, np.ascontiguousarray(pi), k, n, codes, scales, _ptr(x), _ptr(quot))
    return BlockKeyCache(codes, scales, x, quot)


def scores_block(q: np.ndarray, kc: BlockKeyCache, bits: int, pi: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.float64)
    nq, d = q.shape
    T = kc.codes.shape[0]
    out = np.zeros((nq, T))
    _l().orc_scores_block(d, bits, np.ascontiguousarray(pi), q, nq, np.ascontiguousarray(kc.codes),
                          np.ascontiguousarray(kc.scales), T, out)
    return out


def dequant_keys_block(kc: BlockKeyCache, bits: int, pi: np.ndarray) -> np.ndarray:
    n = kc.codes.shape[0]
    d = pi.shape[0]
    out = np.zeros((n, d))
    _l().orc_dequant_keys_block(d, bits, np.ascontiguousarray(pi), np.ascontiguousarray(kc.codes),
                                np.ascontiguousarray(kc.scales), n, out)
    return out


def attend_block(q: np.ndarray, kc: BlockKeyCache, bits: int, pi: np.ndarray, vc: ValueCache,
                 vbits: int, group: int, scale: float | None = None) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.float64)
    nq, d = q.shape
    T = kc.codes.shape[0]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    out = np.zeros((nq, d))
    _l().orc_attend_block(d, bits, np.ascontiguousarray(pi), q, nq, np.ascontiguousarray(kc.codes),
                          np.ascontiguousarray(kc.scales), T, vbits, group, np.ascontiguousarray(vc.codes),
                          np.ascontiguousarray(vc.params), float(scale), out)
    return out


# ------------------------------------------------------------ size accounting
def key_bytes_per_vector(d: int, bits: int, m: int) -> int:
    """codes + signs + fp32 ||k|| + fp32 ||r||; the first-stage format (m = 0)
    stores neither signs nor ||r||, which its score does not use"""
    return (d * bits + 7) // 8 + (m + 7) // 8 + 4 + (4 if m > 0 else 0)


def value_bytes_per_vector(d: int, bits: int, group: int) -> int:
    """codes + (fp16 scale, fp16 zero) per group"""
    return (d * bits + 7) // 8 + 4 * (d // group)

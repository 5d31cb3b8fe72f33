"""attention_decode_amd: Python binding of libtq, the MI355X (gfx950) TurboQuant
KV-cache hot path.

The functions below carry the names of the C entry points in include/tq.h and
do argument marshalling only: torch tensors provide device memory and the
current HIP stream, every computation runs in libtq's HIP kernels.  There is
no CPU path; a missing libtq.so raises ImportError at first use.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np

from . import _lib as L
from ._lib import (TQ_BF16, TQ_F16, TQ_F32, TQ_ROT_DENSE, TQ_ROT_HADAMARD, TQError,  # noqa: F401
                   check, lib)

__all__ = [
    "tq_build_codebook", "tq_make_rotation", "tq_compress_keys", "tq_compress_values",
    "tq_scores", "tq_attend_decode", "tq_codebook_host", "tq_rotation_host",
    "KeyFormat", "ValueFormat", "KeyCache", "ValueCache", "alloc_key_cache", "alloc_value_cache",
    "tq_attend_splits", "tq_attend_workspace_bytes", "tq_scores_workspace_bytes",
    "tq_profile_enable", "tq_profile_read", "TQError", "tq_dequantize_keys",
    "CacheLayout", "alloc_layout_key_cache", "alloc_layout_value_cache", "tq_append_keys", "tq_append_values",
    "tq_attend_paged_workspace_bytes", "tq_attend_decode_paged",
    "BlockFormat", "BlockCache", "alloc_block_cache", "tq_compress_keys_block", "tq_attend_decode_block",
    "tq_attend_block_workspace_bytes",
]

_ROT_KIND = {"dense": TQ_ROT_DENSE, "hadamard": TQ_ROT_HADAMARD, "hadamard2": L.TQ_ROT_HADAMARD2}


def _dptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


# ----------------------------------------------------------------- handles
class Codebook:
    """Owned tq_codebook handle (freed with the object)."""

    def __init__(self, d: int, bits: int):
        h = ctypes.c_void_p()
        check(lib().tq_build_codebook(d, bits, ctypes.byref(h)), "tq_build_codebook")
        self.handle, self.d, self.bits = h, d, bits

    def tables(self):
        n = 1 << self.bits
        c, t = np.zeros(n), np.zeros(n - 1)
        check(lib().tq_codebook_tables(self.handle, _dptr(c), _dptr(t)), "tq_codebook_tables")
        return c, t

    def __del__(self, _L=L):    # the loader module, held past interpreter shutdown
        if getattr(self, "handle", None) and _L._lib is not None:
            _L._lib.tq_codebook_free(self.handle)
            self.handle = None


class Rotation:
    """Owned tq_rotation handle (freed with the object)."""

    def __init__(self, seed: int, d: int, kind: str = "dense"):
        h = ctypes.c_void_p()
        check(lib().tq_make_rotation(seed, d, _ROT_KIND[kind], ctypes.byref(h)), "tq_make_rotation")
        self.handle, self.seed, self.d, self.kind = h, seed, d, kind

    def __del__(self, _L=L):    # the loader module, held past interpreter shutdown
        if getattr(self, "handle", None) and _L._lib is not None:
            _L._lib.tq_rotation_free(self.handle)
            self.handle = None


def tq_build_codebook(d: int, bits: int) -> Codebook:
    return Codebook(d, bits)


def tq_make_rotation(seed: int, d: int, kind: str = "dense") -> Rotation:
    return Rotation(seed, d, kind)


def tq_codebook_host(d: int, bits: int):
    n = 1 << bits
    c, t = np.zeros(n), np.zeros(n - 1)
    check(lib().tq_codebook_host(d, bits, _dptr(c), _dptr(t)), "tq_codebook_host")
    return c, t


def tq_rotation_host(seed: int, d: int, kind: str = "dense"):
    pi, s = np.zeros((d, d)), np.zeros((d, d))
    check(lib().tq_rotation_host(seed, d, _ROT_KIND[kind], _dptr(pi), _dptr(s)), "tq_rotation_host")
    return pi, s


# ------------------------------------------------------------------ formats
@dataclass
class KeyFormat:
    d: int
    mse_bits: int
    cb: Codebook
    rot: Rotation
    qjl_m: int | None = None

    def c(self) -> L.KeyFmt:
        return L.KeyFmt(self.d, self.mse_bits, self.d if self.qjl_m is None else self.qjl_m,
                        self.cb.handle, self.rot.handle)


@dataclass
class ValueFormat:
    d: int
    bits: int
    group: int

    def c(self) -> L.ValFmt:
        return L.ValFmt(self.d, self.bits, self.group)


@dataclass
class KeyCache:
    codes: "torch.Tensor"   # noqa: F821  [B, H, T, d*b/8] uint8
    signs: "torch.Tensor"   # noqa: F821  [B, H, T, m/8] uint8 (None without QJL rows)
    knorm: "torch.Tensor"   # noqa: F821  [B, H, T] float32
    rnorm: "torch.Tensor"   # noqa: F821  [B, H, T] float32 (None without QJL rows)

    def c(self) -> L.KCache:
        ptr = lambda t: None if t is None else t.data_ptr()
        return L.KCache(self.codes.data_ptr(), ptr(self.signs), self.knorm.data_ptr(), ptr(self.rnorm))


@dataclass
class ValueCache:
    codes: "torch.Tensor"   # noqa: F821  [B, H, T, d*b/8] uint8
    params: "torch.Tensor"  # noqa: F821  [B, H, T, d/g, 2] int16 (fp16 bit patterns)

    def c(self) -> L.VCache:
        return L.VCache(self.codes.data_ptr(), self.params.data_ptr())


def alloc_key_cache(fmt: KeyFormat, B: int, H: int, T: int, device="cuda") -> KeyCache:
    """Planes of a key cache; the first-stage format (qjl_m = 0) has no signs
    and no rnorm plane."""
    import torch
    kf = fmt.c()
    row = lambda p: lib().tq_key_plane_bytes(ctypes.byref(kf), 1, p)
    qjl = kf.qjl_m > 0
    return KeyCache(torch.empty((B, H, T, row(0)), dtype=torch.uint8, device=device),
                    torch.empty((B, H, T, row(1)), dtype=torch.uint8, device=device) if qjl else None,
                    torch.empty((B, H, T), dtype=torch.float32, device=device),
                    torch.empty((B, H, T), dtype=torch.float32, device=device) if qjl else None)


def alloc_value_cache(fmt: ValueFormat, B: int, H: int, T: int, device="cuda") -> ValueCache:
    import torch
    return ValueCache(torch.empty((B, H, T, fmt.d * fmt.bits // 8), dtype=torch.uint8, device=device),
                      torch.empty((B, H, T, fmt.d // fmt.group, 2), dtype=torch.int16, device=device))


# ------------------------------------------------------------------ hot path
def _dtype_code(t) -> int:
    import torch
    return {torch.float32: TQ_F32, torch.bfloat16: TQ_BF16, torch.float16: TQ_F16}[t.dtype]


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _bhtd(x):
    if x.dim() != 4 or x.stride(3) != 1:
        raise ValueError("expected [B, H, T, d] with unit channel stride")
    B, H, T, _ = x.shape
    return B, H, T, x.stride(0), x.stride(1), x.stride(2)


def tq_compress_keys(fmt: KeyFormat, k, out: KeyCache, stream=None) -> None:
    B, H, T, sb, sh, st = _bhtd(k)
    kf = fmt.c()
    check(lib().tq_compress_keys(ctypes.byref(kf), k.data_ptr(), _dtype_code(k), B, H, T, sb, sh, st,
                                 out.c(), _stream(stream)), "tq_compress_keys")


def tq_compress_values(fmt: ValueFormat, v, out: ValueCache, stream=None) -> None:
    B, H, T, sb, sh, st = _bhtd(v)
    vf = fmt.c()
    check(lib().tq_compress_values(ctypes.byref(vf), v.data_ptr(), _dtype_code(v), B, H, T, sb, sh, st,
                                   out.c(), _stream(stream)), "tq_compress_values")


def tq_scores_workspace_bytes(fmt: KeyFormat, B: int, Hq: int) -> int:
    kf = fmt.c()
    return int(lib().tq_scores_workspace_bytes(ctypes.byref(kf), B, Hq))


def tq_scores(fmt: KeyFormat, q, kc: KeyCache, Hkv: int, T: int, out=None, ws=None, stream=None):
    """q [B, Hq, d] contiguous -> scores [B, Hq, T] fp32."""
    import torch
    B, Hq, _ = q.shape
    if out is None:
        out = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    need = tq_scores_workspace_bytes(fmt, B, Hq)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    kf = fmt.c()
    check(lib().tq_scores(ctypes.byref(kf), q.data_ptr(), _dtype_code(q), B, Hq, Hkv, T, kc.c(),
                          out.data_ptr(), ws.data_ptr(), ws.numel(), _stream(stream)), "tq_scores")
    return out


def tq_dequantize_keys(fmt: KeyFormat, kc: KeyCache, B: int, Hkv: int, T: int, out=None, stream=None):
    """Explicit key estimates of a packed cache -> [B, Hkv, T, d] fp32."""
    import torch
    if out is None:
        out = torch.empty((B, Hkv, T, fmt.d), dtype=torch.float32, device=kc.codes.device)
    kf = fmt.c()
    check(lib().tq_dequantize_keys(ctypes.byref(kf), B, Hkv, T, kc.c(), out.data_ptr(), _stream(stream)),
          "tq_dequantize_keys")
    return out


def tq_attend_splits(fmt: KeyFormat, B: int, Hq: int, Hkv: int, T: int) -> int:
    kf = fmt.c()
    return int(lib().tq_attend_splits(ctypes.byref(kf), B, Hq, Hkv, T))


def tq_attend_workspace_bytes(fmt: KeyFormat, B: int, Hq: int, Hkv: int, T: int, n_splits: int = 0) -> int:
    kf = fmt.c()
    return int(lib().tq_attend_workspace_bytes(ctypes.byref(kf), B, Hq, Hkv, T, n_splits))


def tq_attend_decode(kfmt: KeyFormat, vfmt: ValueFormat, q, kc: KeyCache, vc: ValueCache, Hkv: int,
                     T: int, out=None, ws=None, n_splits: int = 0, softmax_scale: float = 0.0,
                     stream=None):
    """q [B, Hq, d] contiguous -> attention output [B, Hq, d] fp32."""
    import torch
    B, Hq, d = q.shape
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if ws is None:
        need = tq_attend_workspace_bytes(kfmt, B, Hq, Hkv, T, n_splits)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    kf, vf = kfmt.c(), vfmt.c()
    check(lib().tq_attend_decode(ctypes.byref(kf), ctypes.byref(vf), q.data_ptr(), _dtype_code(q), B, Hq,
                                 Hkv, T, kc.c(), vc.c(), softmax_scale, n_splits, ws.data_ptr(),
                                 ws.numel(), out.data_ptr(), _stream(stream)), "tq_attend_decode")
    return out


def tq_attend_decode_noalloc(kfmt: KeyFormat, vfmt: ValueFormat, q, kc: KeyCache, vc: ValueCache, Hkv: int,
                             T: int, out, n_splits: int = 0, softmax_scale: float = 0.0, stream=None):
    """tq_attend_decode with the library's static device scratch as its
    workspace: allocates nothing (out [B, Hq, d] fp32 is the caller's)."""
    B, Hq, _ = q.shape
    kf, vf = kfmt.c(), vfmt.c()
    check(lib().tq_attend_decode_noalloc(ctypes.byref(kf), ctypes.byref(vf), q.data_ptr(), _dtype_code(q), B, Hq,
                                         Hkv, T, kc.c(), vc.c(), softmax_scale, n_splits, out.data_ptr(),
                                         _stream(stream)), "tq_attend_decode_noalloc")
    return out


# ------------------------------------------------------------ serving caches
@dataclass
class CacheLayout:
    """A preallocated cache that grows per decode step (tq_cache_layout).
    seq_lens: int32 [B] device tensor.  block_table: None (contiguous planes
    [B, Hkv, capacity, row]) or int32 [B, max_blocks] device tensor into a pool
    of num_blocks blocks of block_size tokens (planes [num_blocks, Hkv,
    block_size, row])."""
    capacity: int
    seq_lens: "torch.Tensor"        # noqa: F821
    block_table: "torch.Tensor" = None  # noqa: F821
    block_size: int = 0
    num_blocks: int = 0

    def c(self) -> L.CacheLayout:
        bt = self.block_table
        return L.CacheLayout(self.capacity, None if self.seq_lens is None else self.seq_lens.data_ptr(),
                             None if bt is None else bt.data_ptr(), self.block_size,
                             0 if bt is None else bt.shape[1], self.num_blocks)


def paged_rows(layout: CacheLayout, B: int, Hkv: int) -> int:
    """Rows each plane of a layout cache holds."""
    if layout.block_table is None:
        return B * Hkv * layout.capacity
    return layout.num_blocks * Hkv * layout.block_size


def alloc_layout_key_cache(fmt: KeyFormat, layout: CacheLayout, B: int, Hkv: int, device="cuda") -> KeyCache:
    """Key planes of a layout cache, flattened to rows."""
    import torch
    kf = fmt.c()
    n = paged_rows(layout, B, Hkv)
    row = lambda p: lib().tq_key_plane_bytes(ctypes.byref(kf), 1, p)
    qjl = kf.qjl_m > 0
    return KeyCache(torch.zeros((n, row(0)), dtype=torch.uint8, device=device),
                    torch.zeros((n, row(1)), dtype=torch.uint8, device=device) if qjl else None,
                    torch.zeros((n,), dtype=torch.float32, device=device),
                    torch.zeros((n,), dtype=torch.float32, device=device) if qjl else None)


def alloc_layout_value_cache(fmt: ValueFormat, layout: CacheLayout, B: int, Hkv: int, device="cuda") -> ValueCache:
    import torch
    n = paged_rows(layout, B, Hkv)
    return ValueCache(torch.zeros((n, fmt.d * fmt.bits // 8), dtype=torch.uint8, device=device),
                      torch.zeros((n, fmt.d // fmt.group, 2), dtype=torch.int16, device=device))


def tq_append_keys(fmt: KeyFormat, k, layout: CacheLayout, pos, cache: KeyCache, stream=None) -> None:
    """k [B, Hkv, n_new, d] -> positions pos[b] .. pos[b] + n_new - 1 of each sequence."""
    B, H, T, sb, sh, st = _bhtd(k)
    kf, lay = fmt.c(), layout.c()
    check(lib().tq_append_keys(ctypes.byref(kf), k.data_ptr(), _dtype_code(k), B, H, T, sb, sh, st,
                               ctypes.byref(lay), pos.data_ptr(), cache.c(), _stream(stream)), "tq_append_keys")


def tq_append_values(fmt: ValueFormat, v, layout: CacheLayout, pos, cache: ValueCache, stream=None) -> None:
    B, H, T, sb, sh, st = _bhtd(v)
    vf, lay = fmt.c(), layout.c()
    check(lib().tq_append_values(ctypes.byref(vf), v.data_ptr(), _dtype_code(v), B, H, T, sb, sh, st,
                                 ctypes.byref(lay), pos.data_ptr(), cache.c(), _stream(stream)), "tq_append_values")


def tq_attend_paged_workspace_bytes(fmt: KeyFormat, B: int, Hq: int, Hkv: int, layout: CacheLayout,
                                    n_splits: int = 0) -> int:
    kf, lay = fmt.c(), layout.c()
    return int(lib().tq_attend_paged_workspace_bytes(ctypes.byref(kf), B, Hq, Hkv, ctypes.byref(lay), n_splits))


def tq_attend_decode_paged(kfmt: KeyFormat, vfmt: ValueFormat, q, kc: KeyCache, vc: ValueCache, Hkv: int,
                           layout: CacheLayout, out=None, ws=None, n_splits: int = 0, softmax_scale: float = 0.0,
                           stream=None):
    """q [B, Hq, d] contiguous over a layout cache -> [B, Hq, d] fp32."""
    import torch
    B, Hq, d = q.shape
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if ws is None:
        need = tq_attend_paged_workspace_bytes(kfmt, B, Hq, Hkv, layout, n_splits)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    kf, vf, lay = kfmt.c(), vfmt.c(), layout.c()
    check(lib().tq_attend_decode_paged(ctypes.byref(kf), ctypes.byref(vf), q.data_ptr(), _dtype_code(q), B, Hq,
                                       Hkv, ctypes.byref(lay), kc.c(), vc.c(), softmax_scale, n_splits,
                                       ws.data_ptr(), ws.numel(), out.data_ptr(), _stream(stream)),
          "tq_attend_decode_paged")
    return out


# ------------------------------------------------- rotated block key formats
@dataclass
class BlockFormat:
    """Rotated 8-bit or 4-bit block key format (tq_block_fmt)."""
    d: int
    bits: int
    rot: Rotation

    def c(self) -> L.BlockFmt:
        return L.BlockFmt(self.d, self.bits, self.rot.handle)


@dataclass
class BlockCache:
    codes: "torch.Tensor"   # noqa: F821  [B, H, T, d*bits/8] uint8
    scales: "torch.Tensor"  # noqa: F821  [B, H, T, d/32] int16 (fp16 bit patterns)

    def c(self) -> L.BCache:
        return L.BCache(self.codes.data_ptr(), self.scales.data_ptr())


def alloc_block_cache(fmt: BlockFormat, B: int, H: int, T: int, device="cuda") -> BlockCache:
    import torch
    return BlockCache(torch.empty((B, H, T, fmt.d * fmt.bits // 8), dtype=torch.uint8, device=device),
                      torch.empty((B, H, T, fmt.d // 32), dtype=torch.int16, device=device))


def tq_compress_keys_block(fmt: BlockFormat, k, out: BlockCache, stream=None) -> None:
    B, H, T, sb, sh, st = _bhtd(k)
    bf = fmt.c()
    check(lib().tq_compress_keys_block(ctypes.byref(bf), k.data_ptr(), _dtype_code(k), B, H, T, sb, sh, st,
                                       out.c(), _stream(stream)), "tq_compress_keys_block")


def tq_attend_block_workspace_bytes(fmt: BlockFormat, B: int, Hq: int, Hkv: int, T: int, n_splits: int = 0) -> int:
    bf = fmt.c()
    return int(lib().tq_attend_block_workspace_bytes(ctypes.byref(bf), B, Hq, Hkv, T, n_splits))


def tq_attend_decode_block(kfmt: BlockFormat, vfmt: ValueFormat, q, kc: BlockCache, vc: ValueCache, Hkv: int,
                           T: int, out=None, ws=None, n_splits: int = 0, softmax_scale: float = 0.0, stream=None):
    """q [B, Hq, d] contiguous over block-format keys -> [B, Hq, d] fp32."""
    import torch
    B, Hq, d = q.shape
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if ws is None:
        need = tq_attend_block_workspace_bytes(kfmt, B, Hq, Hkv, T, n_splits)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    bf, vf = kfmt.c(), vfmt.c()
    check(lib().tq_attend_decode_block(ctypes.byref(bf), ctypes.byref(vf), q.data_ptr(), _dtype_code(q), B, Hq,
                                       Hkv, T, kc.c(), vc.c(), softmax_scale, n_splits, ws.data_ptr(), ws.numel(),
                                       out.data_ptr(), _stream(stream)), "tq_attend_decode_block")
    return out


# ------------------------------------------------------------------ profiling
def tq_profile_enable(on: bool = True) -> None:
    check(lib().tq_profile_enable(1 if on else 0), "tq_profile_enable")


def tq_profile_read(name: str):
    """(total ms, launches) of recorded launches whose kernel name contains `name`."""
    ms, n = ctypes.c_double(), ctypes.c_int64()
    check(lib().tq_profile_read(name.encode(), ctypes.byref(ms), ctypes.byref(n)), "tq_profile_read")
    return ms.value, n.value

"""Seeded synthetic workloads shaped like the pages' KV caches.

This module only draws random tensors with the shapes and statistics of the
workloads; it holds none of the method's arithmetic, and both the GPU path and
the CPU oracle take their inputs from it.

Workloads (the real-model caches they stand in for are not available here):
  tiny            1 x 1 KV head x 512 tokens, d 128, fp32 N(0,1); K 2+1 bits (dense
                  rotation), V 2-bit g32; 4 query heads.
  qwen25-3b-8k    Qwen2.5-3B-shaped cache ("turboquant-pytorch", section "What it
                  does": Qwen2.5-3B, 8K context, 3-bit mode): 36 layers x 2 KV heads x
                  8192 tokens, d 128, bf16, 16 query heads.  Keys per channel
                  N(0, s_c^2) with s_c log-normal(0, 1), 4 outlier channels x20 per
                  head, then one scale per layer so that mean ||k|| = 100 mean ||v||
                  (the K/V norm ratio of 100-180x that the tproger.ru article,
                  section "The K-tensor problem", reports); values N(0,1).
  batched-8b-32k  32 sequences x 8 KV heads x 32768 tokens, d 128, bf16 N(0,1); K 2+1
                  bits with the randomized Hadamard rotation, V 4-bit g32; 32 query heads.
  long-1m         1 sequence x 8 KV heads x 1,048,576 tokens, d 128, bf16 N(0,1); K 3+1
                  bits (dense), V 2-bit g64; 64 query heads.
  asym-d256       16 sequences x 16 KV heads x 65536 tokens, d 256, bf16; keys N(0,1)
                  scaled to a K/V norm ratio of 150, K 7+1 bits (dense), V 4-bit g32;
                  32 query heads (the TQ8-K + TQ4-V split the tproger.ru article
                  recommends).
Queries are N(0,1) in the cache dtype, one decode token per sequence.
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    B: int
    Hkv: int
    Hq: int
    T: int
    d: int
    dtype: str          # "float32" | "bfloat16"
    k_bits: int         # Lloyd-Max bits per coordinate (one QJL bit per row on top)
    rot: str            # "dense" | "hadamard"
    v_bits: int
    group: int
    keys: str           # "iid" | "channel_lognormal" | "scaled"
    kv_ratio: float     # target mean ||k|| / mean ||v|| (0: unscaled)
    seed: int
    qjl: bool = True    # False: the first-stage key format (codes and ||k|| only)
    block_bits: int = 0  # 8 or 4: rotated block key format instead of TurboQuant keys

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def with_T(self, T: int, B: int | None = None, layers: int | None = None) -> "Workload":
        return replace(self, T=T, B=self.B if B is None else B,
                       layers=self.layers if layers is None else layers)

    def key_bytes(self) -> int:
        """packed bytes per key vector: codes + signs + fp32 ||k|| + fp32 ||r||
        (codes + fp32 ||k|| for the first-stage format; codes + an fp16 scale
        per 32 coordinates for a block format)"""
        if self.block_bits:
            return self.d * self.block_bits // 8 + 2 * (self.d // 32)
        return self.d * self.k_bits // 8 + (self.d // 8 + 4 if self.qjl else 0) + 4

    @property
    def qjl_m(self) -> int:
        return self.d if self.qjl else 0

    def value_bytes(self) -> int:
        """packed bytes per value vector: codes + fp16 (scale, zero) per group"""
        return self.d * self.v_bits // 8 + 4 * (self.d // self.group)

    def vectors(self) -> int:
        return self.layers * self.B * self.Hkv * self.T

    def packed_bytes(self) -> int:
        return self.vectors() * (self.key_bytes() + self.value_bytes())

    def rotation_seed(self, layer: int) -> int:
        return self.seed * 1000 + layer


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 1, 4, 512, 128, "float32", 2, "dense", 2, 32, "iid", 0.0, 1),
    "qwen25-3b-8k": Workload("qwen25-3b-8k", 36, 1, 2, 16, 8192, 128, "bfloat16", 2, "dense", 2, 32,
                             "channel_lognormal", 100.0, 2),
    "batched-8b-32k": Workload("batched-8b-32k", 1, 32, 8, 32, 32768, 128, "bfloat16", 2, "hadamard",
                               4, 32, "iid", 0.0, 3),
    "long-1m": Workload("long-1m", 1, 1, 8, 64, 1 << 20, 128, "bfloat16", 3, "dense", 2, 64, "iid",
                        0.0, 4),
    "asym-d256": Workload("asym-d256", 1, 16, 16, 32, 65536, 256, "bfloat16", 7, "dense", 4, 32,
                          "scaled", 150.0, 5),
}


def _seed(*parts) -> int:
    h = hashlib.sha256(repr(parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, *parts):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


def _torch_dtype(w: Workload):
    import torch
    return {"float32": torch.float32, "bfloat16": torch.bfloat16}[w.dtype]


def make_values(w: Workload, layer: int = 0, device="cpu"):
    """V [B, Hkv, T, d] ~ N(0, 1) in the workload dtype."""
    import torch
    g = _gen(device, w.name, w.seed, layer, "v", w.B, w.Hkv, w.T)
    v = torch.empty((w.B, w.Hkv, w.T, w.d), dtype=_torch_dtype(w), device=device)
    for b in range(w.B):        # one sequence at a time keeps the fp32 temporaries small
        v[b] = torch.randn((w.Hkv, w.T, w.d), generator=g, device=device).to(v.dtype)
    return v


def _mean_gaussian_norm(d: int) -> float:
    """E||x|| for x ~ N(0, I_d): sqrt(2) Gamma((d+1)/2) / Gamma(d/2)."""
    return math.sqrt(2.0) * math.exp(math.lgamma((d + 1) / 2) - math.lgamma(d / 2))


def make_keys(w: Workload, layer: int = 0, device="cpu"):
    """K [B, Hkv, T, d] with the workload's key statistics, in the workload dtype."""
    import torch
    g = _gen(device, w.name, w.seed, layer, "k", w.B, w.Hkv, w.T)
    k = torch.empty((w.B, w.Hkv, w.T, w.d), dtype=_torch_dtype(w), device=device)
    if w.keys == "channel_lognormal":
        # per-(head, channel) spread, 4 outlier channels per head, then one scale
        # per layer that puts mean ||k|| at kv_ratio x mean ||v||
        sig = torch.exp(torch.randn((w.Hkv, 1, w.d), generator=g, device=device))
        for h in range(w.Hkv):
            sig[h, 0, torch.randperm(w.d, generator=g, device=device)[:4]] *= 20.0
        x = torch.randn((w.B, w.Hkv, w.T, w.d), generator=g, device=device) * sig
        mean_norm = float(torch.linalg.vector_norm(x, dim=-1).mean())
        k.copy_(x * (w.kv_ratio * _mean_gaussian_norm(w.d) / mean_norm))
        return k
    scale = w.kv_ratio if w.keys == "scaled" else 1.0   # same law as V, so the ratio is the scale
    for b in range(w.B):        # one sequence at a time keeps the fp32 temporaries small
        k[b] = (torch.randn((w.Hkv, w.T, w.d), generator=g, device=device) * scale).to(k.dtype)
    return k


def make_queries(w: Workload, layer: int = 0, device="cpu"):
    """Q [B, Hq, d] ~ N(0, 1) in the workload dtype (one decode token per sequence)."""
    import torch
    g = _gen(device, w.name, w.seed, layer, "q", w.B, w.Hq)
    return torch.randn((w.B, w.Hq, w.d), generator=g, device=device).to(_torch_dtype(w))


def random_packed_cache(w: Workload, layer: int = 0, device="cpu", peaked: bool = False):
    """Uniformly random packed planes of the workload's format (codes, signs,
    value codes as random bytes; norms and value scale/zero drawn in realistic
    ranges).  `peaked` scales ||k|| up by 100 so the softmax is near one-hot.
    Returns a dict of tensors shaped [B, Hkv, T, ...]."""
    import torch
    g = _gen(device, w.name, w.seed, layer, "packed", w.B, w.Hkv, w.T, peaked)
    shp = (w.B, w.Hkv, w.T)
    u8 = lambda n: torch.randint(0, 256, shp + (n,), generator=g, device=device, dtype=torch.int32).to(torch.uint8)
    kn = (w.d ** 0.5) * (1.0 + 0.1 * torch.randn(shp, generator=g, device=device)).abs()
    if peaked:
        kn = kn * 100.0
    rn = 0.3 * (1.0 + 0.2 * torch.randn(shp, generator=g, device=device)).abs()
    ng = w.d // w.group
    levels = (1 << w.v_bits) - 1
    sc = (2 * 2.5 / levels) * (0.5 + torch.rand(shp + (ng,), generator=g, device=device))
    ze = -2.5 * (0.5 + torch.rand(shp + (ng,), generator=g, device=device))
    params = torch.stack([sc.to(torch.float16), ze.to(torch.float16)], dim=-1).view(torch.int16)
    return {
        "codes": u8(w.d * w.k_bits // 8), "signs": u8(w.d // 8),
        "knorm": kn.to(torch.float32), "rnorm": rn.to(torch.float32),
        "vcodes": u8(w.d * w.v_bits // 8), "vparams": params.contiguous(),
    }

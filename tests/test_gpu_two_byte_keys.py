"""Two-byte keys (bf16, fp16) under a dense rotation through the input paths
other than a flat contiguous call: strided (token-major) inputs, and appends
into contiguous and paged serving caches.

These keys take the fp16 form of y = Pi k, each key staged times a power of
two of its own (the staging reads either layout and the append's row map the
same way).  Every case is compared with the oracle's encoding of the same
tokens (codes and signs bit-exact except coordinates within 1e-5 of a
decision boundary, ||k|| relative 1e-6, ||r|| relative 1e-5) and bit for bit
with the flat contiguous compressor's rows."""
from dataclasses import replace

import numpy as np
import pytest

import attention_decode_amd as tq
from attention_decode_amd import workloads as W
import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available()
    return torch


def _keys(torch, w, dtype):
    return W.make_keys(replace(w, dtype="bfloat16")).to(getattr(torch, dtype))


@pytest.mark.parametrize("dtype", ["bfloat16", "float16"])
@pytest.mark.parametrize("name", ["long-1m", "asym-d256"])
def test_strided_keys_match_contiguous_and_oracle(torch_cuda, name, dtype):
    torch = torch_cuda
    w = replace(W.WORKLOADS[name], name="strided", B=2, Hkv=3, T=333, dtype=dtype, rot="dense", seed=51)
    print(f"[strided] {name} d={w.d} bits={w.k_bits} dtype={dtype}", flush=True)
    fm = P.Formats(w, 0)
    k = _keys(torch, w, dtype).cuda()
    v = torch.zeros_like(k)
    kc, _ = P.gpu_compress(fm, k, v)
    # the same tensor stored token-major ([B, T, H, d]) and viewed as [B, H, T, d]
    k2 = k.transpose(1, 2).contiguous().transpose(1, 2)
    kc2, _ = P.gpu_compress(fm, k2, v)
    torch.cuda.synchronize()
    for a, b in [(kc.codes, kc2.codes), (kc.signs, kc2.signs), (kc.knorm, kc2.knorm), (kc.rnorm, kc2.rnorm)]:
        assert torch.equal(a, b)
    st = P.compare_keys(fm, kc2, P.f64(k.cpu()).reshape(-1, w.d))
    print(f"[strided] {name} {dtype}: {st}", flush=True)


def _layout(torch, B, cap, block_size, rng):
    lens = torch.zeros(B, dtype=torch.int32, device="cuda")
    if block_size == 0:
        return tq.CacheLayout(cap, lens), None
    maxb = cap // block_size
    nblocks = B * maxb + 2
    perm = rng.permutation(nblocks)[: B * maxb].reshape(B, maxb).astype(np.int32)
    return tq.CacheLayout(cap, lens, torch.from_numpy(perm).cuda(), block_size, nblocks), perm


def _rows(perm, H, cap, bs, b, h, t):
    if perm is None:
        return (b * H + h) * cap + t
    return (perm[b, t // bs] * H + h) * bs + t % bs


@pytest.mark.parametrize("block_size", [0, 64])
@pytest.mark.parametrize("dtype", ["bfloat16", "float16"])
@pytest.mark.parametrize("name", ["long-1m", "asym-d256"])
def test_appended_keys_match_flat_and_oracle(torch_cuda, name, dtype, block_size):
    torch = torch_cuda
    cap = 192
    w = replace(W.WORKLOADS[name], name="append2", B=2, Hkv=2, T=cap, dtype=dtype, rot="dense", seed=53)
    print(f"[append2] {name} d={w.d} bits={w.k_bits} dtype={dtype} block_size={block_size}", flush=True)
    rng = np.random.default_rng(53)
    fm = P.Formats(w, 0)
    lay, perm = _layout(torch, w.B, cap, block_size, rng)
    k = _keys(torch, w, dtype).cuda()
    fk = tq.alloc_key_cache(fm.kf, w.B, w.Hkv, w.T)
    tq.tq_compress_keys(fm.kf, k, fk)
    lk = tq.alloc_layout_key_cache(fm.kf, lay, w.B, w.Hkv)
    # a prefill chunk, then single tokens, then a ragged chunk per sequence
    fill = [0] * w.B
    for n in (70, 1, 1, 45, 1):
        for b in range(w.B):
            take = min(n + 3 * b, cap - fill[b])
            pos = torch.full((w.B,), cap + 5, dtype=torch.int32, device="cuda")   # other sequences: skipped
            pos[b] = fill[b]
            tq.tq_append_keys(fm.kf, k[:, :, fill[b]:fill[b] + take].contiguous(), lay, pos, lk)
            fill[b] += take
    torch.cuda.synchronize()
    kin = P.f64(k.cpu())
    src, at = [], []
    for b in range(w.B):
        for h in range(w.Hkv):
            t = np.arange(fill[b])
            src.append(kin[b, h, t])
            at.append(_rows(perm, w.Hkv, cap, block_size, b, h, t))
    at = np.concatenate(at)
    st = P.compare_keys(fm, lk, np.concatenate(src), row_index=at)
    print(f"[append2] {name} {dtype} bs={block_size}: fills {fill}, oracle {st}", flush=True)
    idx = torch.from_numpy(at).cuda()
    fr = torch.from_numpy(np.concatenate([(b * w.Hkv + h) * w.T + np.arange(fill[b])
                                          for b in range(w.B) for h in range(w.Hkv)])).cuda()
    assert torch.equal(lk.codes[idx], fk.codes.reshape(-1, fk.codes.shape[-1])[fr])
    assert torch.equal(lk.signs[idx], fk.signs.reshape(-1, fk.signs.shape[-1])[fr])
    assert torch.equal(lk.knorm[idx], fk.knorm.reshape(-1)[fr])
    assert torch.equal(lk.rnorm[idx], fk.rnorm.reshape(-1)[fr])

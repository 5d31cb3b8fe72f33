"""Parity of the next rows of the path at full workload sizes, in the launch
configuration bench.py times (auto split count): a seeded random packed cache
of the full shape is attended on the GPU and the oracle recomputes whole
sampled (sequence, KV head) units.

  * paged layout: batched-8b-32k's cache in a pool of 64-token blocks behind a
    shuffled block table, with ragged sequence lengths;
  * first-stage keys (qjl_m = 0) at long-1m's shape;
  * rotated 8-bit block keys at asym-d256's shape, plus sampled rows of the
    block compressor on the workload's own keys.
"""
from dataclasses import replace

import numpy as np
import pytest

import attention_decode_amd as tq
from attention_decode_amd import workloads as W
import oracle as O
import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available()
    return torch


def _units(w, seed):
    rng = np.random.default_rng(seed)
    units = {(0, 0), (w.B - 1, w.Hkv - 1)}
    if w.B * w.Hkv > 2:
        units.add((int(rng.integers(w.B)), int(rng.integers(w.Hkv))))
    return sorted(units)


def test_fullsize_paged_decode_sampled_units(torch_cuda):
    torch = torch_cuda
    w = W.WORKLOADS["batched-8b-32k"]
    bs = 64
    maxb = w.T // bs
    print(f"[full] paged decode {w.name}: {w.B}x{w.Hkv}x{w.T}, blocks of {bs}", flush=True)
    fm = P.Formats(w, 0)
    pc = W.random_packed_cache(w, 0, device="cuda")
    rng = np.random.default_rng(71)
    nblocks = w.B * maxb
    perm = rng.permutation(nblocks).astype(np.int32).reshape(w.B, maxb)
    lens = rng.integers(w.T // 2, w.T + 1, size=w.B).astype(np.int32)
    lens[0] = w.T
    lay = tq.CacheLayout(maxb * bs, torch.from_numpy(lens).cuda(), torch.from_numpy(perm).cuda(), bs, nblocks)

    def to_pool(x):
        # [B, Hkv, T, *row] -> [nblocks, Hkv, bs, *row] with block i of sequence b at perm[b, i]
        row = x.shape[3:]
        y = x.reshape(w.B, w.Hkv, maxb, bs, *row).transpose(1, 2).reshape(nblocks, w.Hkv, bs, *row)
        out = torch.empty_like(y)
        out[torch.from_numpy(perm.reshape(-1).astype(np.int64)).cuda()] = y
        return out.reshape(nblocks * w.Hkv * bs, *row)

    kc = tq.KeyCache(to_pool(pc["codes"]), to_pool(pc["signs"]), to_pool(pc["knorm"]), to_pool(pc["rnorm"]))
    vc = tq.ValueCache(to_pool(pc["vcodes"]), to_pool(pc["vparams"]))
    q = W.make_queries(w, 0, device="cuda")
    out = tq.tq_attend_decode_paged(fm.kf, fm.vf, q, kc, vc, w.Hkv, lay)
    torch.cuda.synchronize()
    G, worst = w.G, 0.0
    for b, h in _units(w, 72):
        n = int(lens[b])
        okc = O.KeyCache(pc["codes"][b, h, :n].cpu().numpy(), pc["signs"][b, h, :n].cpu().numpy(),
                         pc["knorm"][b, h, :n].cpu().numpy(), pc["rnorm"][b, h, :n].cpu().numpy())
        ovc = O.ValueCache(pc["vcodes"][b, h, :n].cpu().numpy(), pc["vparams"][b, h, :n].cpu().numpy().view(np.uint16))
        qq = q[b, h * G:(h + 1) * G].double().cpu().numpy()
        ref = O.attend(qq, okc, w.k_bits, fm.orot, ovc, w.v_bits, w.group)
        worst = max(worst, P.check_attention(out[b, h * G:(h + 1) * G].double().cpu().numpy(), ref))
    print(f"[full] paged {w.name}: max abs err {worst:.3g}", flush=True)
    del pc, kc, vc
    torch.cuda.empty_cache()


def test_fullsize_first_stage_decode_sampled_units(torch_cuda):
    torch = torch_cuda
    w = replace(W.WORKLOADS["long-1m"], qjl=False)
    print(f"[full] first-stage decode long-1m: {w.B}x{w.Hkv}x{w.T}", flush=True)
    seed = w.rotation_seed(0)
    cb = tq.tq_build_codebook(w.d, w.k_bits)
    rot = tq.tq_make_rotation(seed, w.d, w.rot)
    kf, vf = tq.KeyFormat(w.d, w.k_bits, cb, rot, qjl_m=0), tq.ValueFormat(w.d, w.v_bits, w.group)
    orot = O.rotation(seed, w.d, w.rot, m=0)
    pc = W.random_packed_cache(w, 0, device="cuda")
    kc = tq.KeyCache(pc["codes"], None, pc["knorm"], None)
    vc = tq.ValueCache(pc["vcodes"], pc["vparams"])
    q = W.make_queries(w, 0, device="cuda")
    out = tq.tq_attend_decode(kf, vf, q, kc, vc, w.Hkv, w.T)
    torch.cuda.synchronize()
    G, worst = w.G, 0.0
    for b, h in _units(w, 73)[:2]:
        T = w.T
        okc = O.KeyCache(pc["codes"][b, h].cpu().numpy(), np.zeros((T, 0), np.uint8), pc["knorm"][b, h].cpu().numpy(),
                         np.zeros(T, np.float32))
        ovc = O.ValueCache(pc["vcodes"][b, h].cpu().numpy(), pc["vparams"][b, h].cpu().numpy().view(np.uint16))
        qq = q[b, h * G:(h + 1) * G].double().cpu().numpy()
        ref = O.attend(qq, okc, w.k_bits, orot, ovc, w.v_bits, w.group)
        worst = max(worst, P.check_attention(out[b, h * G:(h + 1) * G].double().cpu().numpy(), ref))
    print(f"[full] first-stage long-1m: max abs err {worst:.3g}", flush=True)
    del pc, kc, vc
    torch.cuda.empty_cache()


def test_fullsize_block_format_sampled(torch_cuda):
    torch = torch_cuda
    w = W.WORKLOADS["asym-d256"]
    print(f"[full] q8_0 {w.name}: {w.B}x{w.Hkv}x{w.T}x{w.d}", flush=True)
    seed = w.rotation_seed(0)
    rot = tq.tq_make_rotation(seed, w.d, w.rot)
    bf, vf = tq.BlockFormat(w.d, 8, rot), tq.ValueFormat(w.d, w.v_bits, w.group)
    orot = O.rotation(seed, w.d, w.rot)
    # compressor on the workload's keys: sampled rows against the oracle
    k = W.make_keys(w, 0, device="cuda")
    kc = tq.alloc_block_cache(bf, w.B, w.Hkv, w.T)
    tq.tq_compress_keys_block(bf, k, kc)
    torch.cuda.synchronize()
    n_total = w.B * w.Hkv * w.T
    rows = np.unique(np.concatenate([np.random.default_rng(74).choice(n_total, 256, replace=False), [0, n_total - 1]]))
    idx = torch.from_numpy(rows).cuda()
    ok = O.compress_keys_block(k.reshape(-1, w.d).index_select(0, idx).double().cpu().numpy(), 8, orot.pi,
                               keep_aux=True)
    g_sc = kc.scales.reshape(-1, w.d // 32).index_select(0, idx).cpu().numpy().view(np.uint16)
    g_cd = kc.codes.reshape(-1, w.d).index_select(0, idx).cpu().numpy().view(np.int8).astype(np.int64)
    assert np.array_equal(g_sc, ok.scales)
    mism = g_cd != ok.codes.view(np.int8).astype(np.int64)
    tie = np.abs(np.abs(ok.quot - np.floor(ok.quot)) - 0.5) < 1e-9
    assert np.all(tie[mism])
    del k
    # decode over a random packed cache of the full shape
    g = torch.Generator(device="cuda")
    g.manual_seed(75)
    shp = (w.B, w.Hkv, w.T)
    codes = torch.empty(shp + (w.d,), dtype=torch.int8, device="cuda")
    for b in range(w.B):            # int16 temporaries one sequence at a time
        codes[b] = torch.randint(-127, 128, shp[1:] + (w.d,), generator=g, device="cuda", dtype=torch.int16)
    scales = (0.02 * (0.5 + torch.rand(shp + (w.d // 32,), generator=g, device="cuda"))).to(torch.float16)
    bc = tq.BlockCache(codes.view(torch.uint8), scales.view(torch.int16))
    pc = W.random_packed_cache(w, 0, device="cuda")
    vc = tq.ValueCache(pc["vcodes"], pc["vparams"])
    q = W.make_queries(w, 0, device="cuda")
    out = tq.tq_attend_decode_block(bf, vf, q, bc, vc, w.Hkv, w.T)
    torch.cuda.synchronize()
    G, worst = w.G, 0.0
    for b, h in _units(w, 76):
        okc = O.BlockKeyCache(bc.codes[b, h].cpu().numpy(), bc.scales[b, h].cpu().numpy().view(np.uint16))
        ovc = O.ValueCache(pc["vcodes"][b, h].cpu().numpy(), pc["vparams"][b, h].cpu().numpy().view(np.uint16))
        qq = q[b, h * G:(h + 1) * G].double().cpu().numpy()
        ref = O.attend_block(qq, okc, 8, orot.pi, ovc, w.v_bits, w.group)
        worst = max(worst, P.check_attention(out[b, h * G:(h + 1) * G].double().cpu().numpy(), ref))
    print(f"[full] q8_0 {w.name}: {int(mism.sum())} tie flips in sampled rows, max abs err {worst:.3g}", flush=True)

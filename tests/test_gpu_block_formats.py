"""GPU parity of the rotated block key formats (8-bit and 4-bit codes, one
fp16 scale per 32 rotated coordinates) against the oracle.

Bars: scales bit-exact and codes bit-exact except where the exact quotient
x / scale lies within 1e-9 of a half-integer (the GPU rotates in fp64 from the
same fp64 Pi, so only ties can differ); attention within 1e-3 absolute on
the oracle's own packed cache, like the TurboQuant path."""
from dataclasses import replace

import numpy as np
import pytest

import attention_decode_amd as tq
from attention_decode_amd import workloads as W
import oracle as O
import parity as P

pytestmark = pytest.mark.gpu

BASE = W.WORKLOADS["tiny"]


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available()
    return torch


@pytest.mark.parametrize("d,bits,rot,dtype,keys", [(128, 8, "dense", "bfloat16", "iid"),
                                                   (128, 4, "hadamard", "float32", "iid"),
                                                   (256, 8, "dense", "bfloat16", "scaled"),
                                                   (256, 4, "dense", "bfloat16", "channel_lognormal")])
def test_block_compress_matches_oracle(torch_cuda, d, bits, rot, dtype, keys):
    torch = torch_cuda
    w = replace(BASE, name="blk", B=2, Hkv=3, T=111, d=d, rot=rot, dtype=dtype, keys=keys,
                kv_ratio=150.0 if keys != "iid" else 0.0, seed=51)
    r = tq.tq_make_rotation(w.rotation_seed(0), d, rot)
    bf = tq.BlockFormat(d, bits, r)
    k = W.make_keys(w)
    kc = tq.alloc_block_cache(bf, w.B, w.Hkv, w.T)
    tq.tq_compress_keys_block(bf, k.cuda(), kc)
    torch.cuda.synchronize()
    orot = O.rotation(w.rotation_seed(0), d, rot)
    ok = O.compress_keys_block(P.f64(k).reshape(-1, d), bits, orot.pi, keep_aux=True)
    g_scales = kc.scales.reshape(-1, d // 32).cpu().numpy().view(np.uint16)
    assert np.array_equal(g_scales, ok.scales)
    g_codes = kc.codes.reshape(-1, d * bits // 8).cpu().numpy()
    if bits == 8:
        gi, oi = g_codes.view(np.int8).astype(np.int64), ok.codes.view(np.int8).astype(np.int64)
    else:
        gi, oi = P.unpack_le(g_codes, d, 4).astype(np.int64), P.unpack_le(ok.codes, d, 4).astype(np.int64)
    mism = gi != oi
    tie = np.abs(np.abs(ok.quot - np.floor(ok.quot)) - 0.5) < 1e-9
    assert np.all(tie[mism]), f"{int(mism.sum())} code mismatches off a tie"
    print(f"[block compress] d={d} b={bits} {rot} {keys}: {int(mism.sum())} tie flips", flush=True)


CASES = [
    # (d, bits, rot, Hkv, Hq, v_bits, group, T, keys)
    (128, 8, "dense", 2, 16, 2, 32, 700, "iid"),          # GQA 8 (two row tiles), 2-bit g32 values
    (128, 4, "hadamard", 2, 8, 4, 32, 333, "iid"),        # 4-bit codes
    (256, 8, "dense", 2, 4, 4, 32, 300, "scaled"),        # the TQ8-K + 4-bit V split, one-hot regime
    (256, 4, "dense", 1, 2, 2, 64, 257, "iid"),           # GQA 2
    (128, 8, "dense", 1, 6, 4, 128, 129, "iid"),          # GQA 6 -> chunks of 2
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "d{}b{}G{}T{}".format(c[0], c[1], c[4] // c[3], c[7]))
def test_block_decode_matches_oracle(torch_cuda, case):
    torch = torch_cuda
    d, bits, rot, Hkv, Hq, vb, g, T, keys = case
    w = replace(BASE, name="blkd", B=2, Hkv=Hkv, Hq=Hq, T=T, d=d, rot=rot, v_bits=vb, group=g, keys=keys,
                kv_ratio=150.0 if keys == "scaled" else 0.0, dtype="bfloat16", seed=52)
    r = tq.tq_make_rotation(w.rotation_seed(0), d, rot)
    bf = tq.BlockFormat(d, bits, r)
    vf = tq.ValueFormat(d, vb, g)
    orot = O.rotation(w.rotation_seed(0), d, rot)
    k, v, q = W.make_keys(w), W.make_values(w), W.make_queries(w)
    ok = O.compress_keys_block(P.f64(k).reshape(-1, d), bits, orot.pi)
    ov = O.compress_values(P.f64(v).reshape(-1, d), vb, g)
    kc = tq.BlockCache(torch.from_numpy(ok.codes).reshape(w.B, Hkv, T, -1).cuda(),
                       torch.from_numpy(ok.scales.view(np.int16)).reshape(w.B, Hkv, T, -1).cuda())
    vc = tq.ValueCache(torch.from_numpy(ov.codes).reshape(w.B, Hkv, T, -1).cuda(),
                       torch.from_numpy(ov.params.view(np.int16)).reshape(w.B, Hkv, T, -1, 2).cuda())
    G = Hq // Hkv
    qn = P.f64(q)
    want = np.zeros((w.B, Hq, d))
    for b in range(w.B):
        for h in range(Hkv):
            rows = (b * Hkv + h) * T + np.arange(T)
            okc = O.BlockKeyCache(ok.codes[rows], ok.scales[rows])
            ovc = O.ValueCache(ov.codes[rows], ov.params[rows])
            want[b, h * G:(h + 1) * G] = O.attend_block(qn[b, h * G:(h + 1) * G], okc, bits, orot.pi, ovc, vb, g)
    qd = q.cuda()
    for splits in (0, 1, 4):
        out = tq.tq_attend_decode_block(bf, vf, qd, kc, vc, Hkv, T, n_splits=splits)
        torch.cuda.synchronize()
        err = P.check_attention(out.double().cpu().numpy(), want)
        print(f"[block decode] {case} splits={splits}: max abs err {err:.3g}", flush=True)

"""GPU parity of the two-round Hadamard rotation (TQ_ROT_HADAMARD2): key
compression (codes, signs and norms under the usual bars) and decode
attention against the oracle, at both head dims of the matrix-core path and
at d = 64 (general kernel)."""
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


@pytest.mark.parametrize("d,bits,keys", [(128, 2, "iid"), (256, 7, "scaled"), (64, 3, "iid"), (128, 4, "channel_lognormal")])
def test_two_round_hadamard_compress(torch_cuda, d, bits, keys):
    torch = torch_cuda
    w = replace(BASE, name="h2", B=2, Hkv=2, T=300, d=d, k_bits=bits, rot="hadamard2", keys=keys,
                kv_ratio=150.0 if keys != "iid" else 0.0, dtype="bfloat16", seed=61)
    fm = P.Formats(w, 0)
    k, v = W.make_keys(w).cuda(), W.make_values(w).cuda()
    kc, vc = P.gpu_compress(fm, k, v)
    torch.cuda.synchronize()
    st = P.compare_keys(fm, kc, P.f64(k).reshape(-1, d))
    print(f"[hadamard2 compress] d={d} b={bits} {keys}: {st}", flush=True)


@pytest.mark.parametrize("d,bits,Hkv,Hq,vb,g,T", [(128, 3, 2, 8, 2, 64, 400), (256, 2, 1, 4, 4, 32, 300),
                                                  (64, 2, 1, 4, 2, 32, 260)])
def test_two_round_hadamard_decode(torch_cuda, d, bits, Hkv, Hq, vb, g, T):
    torch = torch_cuda
    w = replace(BASE, name="h2d", B=2, Hkv=Hkv, Hq=Hq, T=T, d=d, k_bits=bits, rot="hadamard2", v_bits=vb,
                group=g, dtype="bfloat16", seed=62)
    fm = P.Formats(w, 0)
    k, v, q = W.make_keys(w), W.make_values(w), W.make_queries(w)
    ok = O.compress_keys(P.f64(k).reshape(-1, d), bits, fm.orot)
    ov = O.compress_values(P.f64(v).reshape(-1, d), vb, g)
    shape = (w.B, w.Hkv, w.T)
    kc, vc = P.to_device_cache(ok, ov, shape, "cuda")
    qn = P.f64(q)
    osc, oat = P.oracle_units(fm, qn, ok, ov, shape)
    for splits in (0, 3):
        out = tq.tq_attend_decode(fm.kf, fm.vf, q.cuda(), kc, vc, w.Hkv, w.T, n_splits=splits)
        torch.cuda.synchronize()
        err = P.check_attention(out.double().cpu().numpy(), oat)
        print(f"[hadamard2 decode] d={d} b={bits} splits={splits}: {err:.3g}", flush=True)
    sc = tq.tq_scores(fm.kf, q.cuda(), kc, w.Hkv, w.T)
    torch.cuda.synchronize()
    P.check_scores(sc.double().cpu().numpy(), osc, qn, ok.knorm.reshape(shape), w.Hkv)


# Both implementations of the Walsh-Hadamard rotations in the key compressor:
# the randomized butterfly in registers (DPP lane stages) and the +-1 sign
# matrix on the matrix cores, each against the oracle under the flip rule, on
# every head dim, input dtype, one and two rounds, both key tilings (64-key
# workgroups for large launches, 32-key ones for small), ragged tails, and the
# first-stage format (no QJL rows).
HAD_CASES = [
    # (d, bits, rot, dtype, B, Hkv, T, qjl)
    (128, 2, "hadamard", "bfloat16", 2, 8, 777, True),
    (128, 3, "hadamard", "float32", 1, 2, 300, True),
    (64, 4, "hadamard", "bfloat16", 1, 3, 333, True),
    (64, 2, "hadamard2", "float32", 2, 1, 129, True),
    (256, 7, "hadamard", "bfloat16", 2, 2, 300, True),
    (256, 2, "hadamard2", "bfloat16", 1, 2, 515, True),
    (256, 5, "hadamard", "float32", 1, 1, 200, True),
    (128, 2, "hadamard", "bfloat16", 64, 8, 128, True),     # 64-key workgroups (>= 512 of them)
    (256, 7, "hadamard2", "bfloat16", 32, 4, 256, True),    # 64-key workgroups, two residual passes
    (128, 3, "hadamard", "bfloat16", 2, 2, 301, False),     # first stage
]


@pytest.mark.parametrize("kernel", ["butterfly", "matrix"])
@pytest.mark.parametrize("case", HAD_CASES, ids=lambda c: "d{}b{}{}{}B{}H{}T{}{}".format(
    c[0], c[1], c[2], c[3][:4], c[4], c[5], c[6], "" if c[7] else "mse"))
def test_hadamard_kernels_match_oracle(torch_cuda, monkeypatch, kernel, case):
    torch = torch_cuda
    d, bits, rot, dtype, B, Hkv, T, qjl = case
    monkeypatch.setenv("TQ_HADAMARD_KERNEL", kernel)
    w = replace(BASE, name="had", B=B, Hkv=Hkv, T=T, d=d, k_bits=bits, rot=rot, dtype=dtype, seed=67,
                keys="scaled", kv_ratio=150.0, qjl=qjl)
    fm = P.Formats(w, 0)
    kf = tq.KeyFormat(d, bits, fm.cb, fm.rot, qjl_m=w.qjl_m)
    k = W.make_keys(w, device="cuda")
    kc = tq.alloc_key_cache(kf, B, Hkv, T)
    tq.tq_compress_keys(kf, k, kc)
    torch.cuda.synchronize()
    st = P.compare_keys(fm, kc, P.f64(k.cpu()).reshape(-1, d))
    print(f"[hadamard {kernel}] {case}: {st}", flush=True)

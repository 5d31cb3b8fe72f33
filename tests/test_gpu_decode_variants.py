"""Decode parity across the format and shape variants the decode kernels
specialise on: key bits, head dim, GQA ratio (query chunks of 1-8 heads),
value bits and group size, query dtype, and split counts.  Every case runs
the oracle's packed cache through tq_attend_decode and compares with the
oracle's attention (1e-3 absolute) and scores (1e-4 ||q|| ||k||)."""
from dataclasses import replace

import numpy as np
import pytest

import attention_decode_amd as tq
from attention_decode_amd import workloads as W
import oracle as O
import parity as P

pytestmark = pytest.mark.gpu

BASE = W.WORKLOADS["tiny"]

CASES = [
    # (d, k_bits, rot, Hkv, Hq, v_bits, group, T, keys, dtype)
    (128, 2, "dense", 2, 16, 2, 32, 1000, "iid", "bfloat16"),      # GQA 8, 2-bit g32 (two groups per tile)
    (128, 1, "dense", 2, 8, 4, 64, 333, "iid", "float32"),         # 1-bit keys
    (256, 2, "dense", 1, 4, 4, 32, 700, "iid", "bfloat16"),        # d 256
    (256, 1, "hadamard", 2, 2, 2, 64, 129, "iid", "bfloat16"),     # GQA 1
    (128, 2, "hadamard", 1, 6, 4, 128, 517, "iid", "bfloat16"),    # GQA 6
    (128, 2, "dense", 1, 16, 2, 128, 300, "scaled", "bfloat16"),   # GQA 16, one-hot regime
    (128, 3, "dense", 1, 8, 2, 64, 400, "iid", "bfloat16"),        # 3-bit keys (pair table)
    (128, 4, "dense", 2, 8, 4, 32, 450, "iid", "bfloat16"),        # 4-bit keys (pair table)
    (128, 3, "hadamard", 2, 8, 4, 32, 390, "iid", "bfloat16"),     # 3-bit keys, 4-bit values (4 KB table budget)
    (128, 7, "dense", 1, 8, 4, 64, 270, "scaled", "bfloat16"),     # 7-bit keys at d 128 (single-code table, 4 KB budget)
    (128, 5, "hadamard", 1, 4, 2, 64, 290, "iid", "bfloat16"),     # 5-bit keys (largest pair table)
    (128, 6, "dense", 1, 2, 4, 32, 333, "iid", "float32"),         # 6-bit keys (single-code table)
    (256, 7, "dense", 2, 4, 4, 32, 260, "scaled", "bfloat16"),     # 7-bit keys (largest format), d 256
    (256, 3, "dense", 1, 8, 2, 32, 500, "iid", "bfloat16"),        # 3-bit keys, d 256, two-group value tiles
    (256, 5, "dense", 2, 2, 4, 64, 300, "scaled", "bfloat16"),     # GQA 1 at d 256: value operand spread over lanes
    (256, 4, "hadamard", 1, 2, 2, 64, 333, "iid", "bfloat16"),     # GQA 2, 2-bit values g64: spread, four groups
    (64, 2, "dense", 1, 4, 2, 32, 260, "iid", "float32"),          # d 64 (general kernel)
    # the decode plan splits a GQA group into smaller query chunks while the
    # grid has fewer than 256 (unit, tile) pairs, so the short cases above run
    # with small chunks; the cases below keep chunks of 4 or 8 (2 x 8 heads x
    # 17 tiles)
    (128, 2, "dense", 8, 64, 2, 32, 2100, "iid", "bfloat16"),      # bit-plane scores, two row tiles
    (128, 3, "dense", 8, 64, 2, 64, 2100, "iid", "bfloat16"),      # table scores, eight queries per unit
    # d 256 table scores score the QJL signs on int8 tiles of four queries:
    # four heads per unit fill one tile, eight take both
    (256, 7, "dense", 8, 32, 4, 32, 2100, "scaled", "bfloat16"),   # table scores d 256, four queries per unit
    (256, 5, "dense", 8, 64, 2, 64, 2100, "iid", "bfloat16"),      # table scores d 256, eight queries per unit
]


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available()
    return torch


@pytest.mark.parametrize("case", CASES, ids=lambda c: "d{}b{}{}G{}v{}g{}T{}".format(c[0], c[1], c[2][0], c[4] // c[3], c[5], c[6], c[7]))
def test_decode_variant(torch_cuda, case):
    torch = torch_cuda
    d, kb, rot, Hkv, Hq, vb, g, T, keys, dt = case
    w = replace(BASE, name="variant", B=2, Hkv=Hkv, Hq=Hq, T=T, d=d, k_bits=kb, rot=rot, v_bits=vb, group=g,
                keys=keys, kv_ratio=150.0 if keys == "scaled" else 0.0, dtype=dt, seed=11)
    fm = P.Formats(w, 0)
    k, v, q = W.make_keys(w), W.make_values(w), W.make_queries(w)
    ok = O.compress_keys(P.f64(k).reshape(-1, d), kb, fm.orot)
    ov = O.compress_values(P.f64(v).reshape(-1, d), vb, g)
    shape = (w.B, w.Hkv, w.T)
    kc, vc = P.to_device_cache(ok, ov, shape, "cuda")
    qd = q.cuda()
    qn = P.f64(q)
    osc, oat = P.oracle_units(fm, qn, ok, ov, shape)
    for splits in (0, 1, 5):
        out = tq.tq_attend_decode(fm.kf, fm.vf, qd, kc, vc, w.Hkv, w.T, n_splits=splits)
        torch.cuda.synchronize()
        err = P.check_attention(out.double().cpu().numpy(), oat)
        print(f"[variant] {case} splits={splits}: attention max abs err {err:.3g}", flush=True)
    sc = tq.tq_scores(fm.kf, qd, kc, w.Hkv, w.T)
    torch.cuda.synchronize()
    P.check_scores(sc.double().cpu().numpy(), osc, qn, ok.knorm.reshape(shape), w.Hkv)


def test_fp16_queries(torch_cuda):
    torch = torch_cuda
    w = replace(BASE, name="variant16", B=1, Hkv=2, Hq=8, T=200, seed=12)
    fm = P.Formats(w, 0)
    k, v = W.make_keys(w), W.make_values(w)
    q = W.make_queries(w).to(torch.float16)
    ok = O.compress_keys(P.f64(k).reshape(-1, w.d), w.k_bits, fm.orot)
    ov = O.compress_values(P.f64(v).reshape(-1, w.d), w.v_bits, w.group)
    shape = (w.B, w.Hkv, w.T)
    kc, vc = P.to_device_cache(ok, ov, shape, "cuda")
    out = tq.tq_attend_decode(fm.kf, fm.vf, q.cuda(), kc, vc, w.Hkv, w.T)
    torch.cuda.synchronize()
    _, oat = P.oracle_units(fm, P.f64(q), ok, ov, shape)
    P.check_attention(out.double().cpu().numpy(), oat)


@pytest.mark.parametrize("Hq", [32, 64])
def test_fp16_queries_d256_table(torch_cuda, Hq):
    """fp16 queries on the d = 256 table scores (int8 QJL sign digits built
    from the fp16 query): four and eight query heads per KV head, so one and
    both sign tiles; attention and scores against the oracle."""
    torch = torch_cuda
    w = replace(BASE, name="variant16d256", B=2, Hkv=8, Hq=Hq, T=2100, d=256, k_bits=5, rot="dense", v_bits=4,
                group=32, dtype="bfloat16", seed=13)
    fm = P.Formats(w, 0)
    k, v = W.make_keys(w), W.make_values(w)
    q = W.make_queries(w).to(torch.float16)
    ok = O.compress_keys(P.f64(k).reshape(-1, w.d), w.k_bits, fm.orot)
    ov = O.compress_values(P.f64(v).reshape(-1, w.d), w.v_bits, w.group)
    shape = (w.B, w.Hkv, w.T)
    kc, vc = P.to_device_cache(ok, ov, shape, "cuda")
    qn = P.f64(q)
    osc, oat = P.oracle_units(fm, qn, ok, ov, shape)
    out = tq.tq_attend_decode(fm.kf, fm.vf, q.cuda(), kc, vc, w.Hkv, w.T)
    sc = tq.tq_scores(fm.kf, q.cuda(), kc, w.Hkv, w.T)
    torch.cuda.synchronize()
    err = P.check_attention(out.double().cpu().numpy(), oat)
    P.check_scores(sc.double().cpu().numpy(), osc, qn, ok.knorm.reshape(shape), w.Hkv)
    print(f"[fp16 q d256] Hq={Hq}: attention max abs err {err:.3g}", flush=True)

"""libtq vs the fp64 oracle on the GPU, through the C ABI.

Reduced-size cases keep each workload's format, dtype and statistics with a
token count that spans several tiles and ends in a ragged tail; the oracle
checks every output.  Full-size cases run in the launch configuration the
benchmark times and check sampled outputs (compression) or whole sampled
(sequence, KV head) units (decode, on a seeded random packed cache).
"""
import numpy as np
import pytest

import attention_decode_amd as tq
from attention_decode_amd import workloads as W
import oracle as O
import parity as P

pytestmark = pytest.mark.gpu

REDUCED = {
    "tiny": dict(T=512),
    "qwen25-3b-8k": dict(T=1000, layers=1),
    "batched-8b-32k": dict(T=777, B=2),
    "long-1m": dict(T=1500),
    "asym-d256": dict(T=300, B=2),
}


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def _reduced(name):
    return W.WORKLOADS[name].with_T(**REDUCED[name])


@pytest.mark.parametrize("name", list(REDUCED))
def test_compress_matches_oracle(torch_cuda, name):
    torch = torch_cuda
    w = _reduced(name)
    layer = 3 if w.layers > 1 or name == "qwen25-3b-8k" else 0
    print(f"[parity] compress {name} B={w.B} T={w.T} layer={layer}", flush=True)
    fm = P.Formats(w, layer)
    k, v = W.make_keys(w, layer), W.make_values(w, layer)
    kc, vc = P.gpu_compress(fm, k.cuda(), v.cuda())
    torch.cuda.synchronize()
    stats = P.compare_keys(fm, kc, P.f64(k).reshape(-1, w.d))
    vflips = P.compare_values(fm, vc, P.f64(v).reshape(-1, w.d))
    print(f"[parity] {name}: {stats} value flips {vflips}", flush=True)


@pytest.mark.parametrize("name", list(REDUCED))
def test_decode_on_oracle_cache(torch_cuda, name):
    torch = torch_cuda
    w = _reduced(name)
    print(f"[parity] decode {name} B={w.B} T={w.T}", flush=True)
    fm = P.Formats(w, 0)
    k, v, q = W.make_keys(w), W.make_values(w), W.make_queries(w)
    ok = O.compress_keys(P.f64(k).reshape(-1, w.d), w.k_bits, fm.orot)
    ov = O.compress_values(P.f64(v).reshape(-1, w.d), w.v_bits, w.group)
    shape = (w.B, w.Hkv, w.T)
    kc, vc = P.to_device_cache(ok, ov, shape, "cuda")
    qd = q.cuda()
    sc = tq.tq_scores(fm.kf, qd, kc, w.Hkv, w.T)
    out = tq.tq_attend_decode(fm.kf, fm.vf, qd, kc, vc, w.Hkv, w.T)
    torch.cuda.synchronize()
    qn = P.f64(q)
    osc, oat = P.oracle_units(fm, qn, ok, ov, shape)
    r = P.check_scores(sc.double().cpu().numpy(), osc, qn, ok.knorm.reshape(shape), w.Hkv)
    e = P.check_attention(out.double().cpu().numpy(), oat)
    print(f"[parity] {name}: score err {r:.3g} x bound, attention max abs err {e:.3g}", flush=True)


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 16, 33, 64, 100])
def test_split_count_invariance(torch_cuda, splits):
    torch = torch_cuda
    w = _reduced("long-1m")
    fm = P.Formats(w, 0)
    k, v, q = W.make_keys(w, device="cuda"), W.make_values(w, device="cuda"), W.make_queries(w, device="cuda")
    kc, vc = P.gpu_compress(fm, k, v)
    ref = tq.tq_attend_decode(fm.kf, fm.vf, q, kc, vc, w.Hkv, w.T, n_splits=1)
    out = tq.tq_attend_decode(fm.kf, fm.vf, q, kc, vc, w.Hkv, w.T, n_splits=splits)
    torch.cuda.synchronize()
    assert torch.allclose(out, ref, atol=1e-5, rtol=1e-5), (out - ref).abs().max()


def _random_cache(w):
    pc = W.random_packed_cache(w, 0, device="cuda")
    return pc, tq.KeyCache(pc["codes"], pc["signs"], pc["knorm"], pc["rnorm"]), \
        tq.ValueCache(pc["vcodes"], pc["vparams"])


def _oracle_unit(w, fm, pc, q, b, h):
    G = w.G
    okc = O.KeyCache(pc["codes"][b, h].cpu().numpy(), pc["signs"][b, h].cpu().numpy(),
                     pc["knorm"][b, h].cpu().numpy(), pc["rnorm"][b, h].cpu().numpy())
    ovc = O.ValueCache(pc["vcodes"][b, h].cpu().numpy(), pc["vparams"][b, h].cpu().numpy().view(np.uint16))
    qq = q[b, h * G:(h + 1) * G].double().cpu().numpy()
    return O.attend(qq, okc, w.k_bits, fm.orot, ovc, w.v_bits, w.group)


@pytest.mark.parametrize("splits", [257, 300, 1024])
def test_many_splits_merge(torch_cuda, splits):
    """More than 256 splits take the looping log-sum-exp merge: the output
    equals the one-split decode and the oracle on whole units (a long-1m
    shaped cache of 131072 tokens)."""
    torch = torch_cuda
    w = W.WORKLOADS["long-1m"].with_T(131072)
    print(f"[parity] many splits {splits}: {w.B}x{w.Hkv}x{w.T}", flush=True)
    fm = P.Formats(w, 0)
    pc, kc, vc = _random_cache(w)
    q = W.make_queries(w, 0, device="cuda")
    ref = tq.tq_attend_decode(fm.kf, fm.vf, q, kc, vc, w.Hkv, w.T, n_splits=1)
    out = tq.tq_attend_decode(fm.kf, fm.vf, q, kc, vc, w.Hkv, w.T, n_splits=splits)
    torch.cuda.synchronize()
    G = w.G
    errs = []
    for b, h in [(0, 0), (0, w.Hkv - 1)]:
        want = _oracle_unit(w, fm, pc, q, b, h)
        errs.append(P.check_attention(out[b, h * G:(h + 1) * G].double().cpu().numpy(), want))
        errs.append(P.check_attention(ref[b, h * G:(h + 1) * G].double().cpu().numpy(), want))
    # One split sums 32768 tokens per wave in fp32 (softmax sum and value
    # accumulators), many splits a few hundred per partial: the two orders of
    # summation differ by up to about 2^-24 per addition in the long chain
    # (1e-3 relative after 2^14 additions, outputs here are ~0.02), so they
    # are compared at a tenth of the attention bar rather than bit for bit.
    diff = float((out - ref).abs().max())
    print(f"[parity] many splits {splits}: oracle errors (splits, one split) {errs}, |splits - one| {diff:.3g}",
          flush=True)
    assert diff <= 0.1 * P.ATTN_TOL


def test_auto_plan_beyond_256_splits(torch_cuda):
    """The automatic split plan of one long sequence with two KV heads (a
    Qwen2.5-3B-shaped head layout at 64K tokens) picks more than 256 splits;
    the decode still matches the oracle on every unit."""
    torch = torch_cuda
    w = W.WORKLOADS["qwen25-3b-8k"].with_T(65536, layers=1)
    fm = P.Formats(w, 0)
    auto = tq.tq_attend_splits(fm.kf, w.B, w.Hq, w.Hkv, w.T)
    print(f"[parity] auto plan for {w.B}x{w.Hkv}x{w.T}, {w.Hq} query heads: {auto} splits", flush=True)
    assert auto > 256
    pc, kc, vc = _random_cache(w)
    q = W.make_queries(w, 0, device="cuda")
    out = tq.tq_attend_decode(fm.kf, fm.vf, q, kc, vc, w.Hkv, w.T)
    torch.cuda.synchronize()
    G = w.G
    for h in range(w.Hkv):
        want = _oracle_unit(w, fm, pc, q, 0, h)
        P.check_attention(out[0, h * G:(h + 1) * G].double().cpu().numpy(), want)


def test_edge_cases(torch_cuda):
    torch = torch_cuda
    w = W.WORKLOADS["tiny"].with_T(3)
    fm = P.Formats(w, 0)
    # zero key, a key with one nonzero channel, a constant value row
    k = torch.zeros((1, 1, 3, 128), dtype=torch.float32)
    k[0, 0, 1, 5] = 2.0
    k[0, 0, 2] = torch.randn(128)
    v = torch.randn((1, 1, 3, 128), dtype=torch.float32)
    v[0, 0, 0] = 0.75
    kc, vc = P.gpu_compress(fm, k.cuda(), v.cuda())
    torch.cuda.synchronize()
    P.compare_keys(fm, kc, P.f64(k).reshape(-1, 128))
    P.compare_values(fm, vc, P.f64(v).reshape(-1, 128))
    # T = 1: attention returns the single dequantised value
    q = torch.randn((1, 4, 128)).cuda()
    kc1 = tq.KeyCache(kc.codes[:, :, 2:3].clone(), kc.signs[:, :, 2:3].clone(),
                      kc.knorm[:, :, 2:3].clone(), kc.rnorm[:, :, 2:3].clone())
    vc1 = tq.ValueCache(vc.codes[:, :, 0:1].clone(), vc.params[:, :, 0:1].clone())
    out = tq.tq_attend_decode(fm.kf, fm.vf, q, kc1, vc1, 1, 1)
    torch.cuda.synchronize()
    assert torch.all(out.cpu() == 0.75)
    # scores of the three edge keys on the oracle's packed cache (the zero key
    # scores exactly 0), and of a one-key cache (the same key, the same score)
    ok = O.compress_keys(P.f64(k).reshape(-1, 128), w.k_bits, fm.orot)
    ov = O.compress_values(P.f64(v).reshape(-1, 128), w.v_bits, w.group)
    kco, _ = P.to_device_cache(ok, ov, (1, 1, 3), "cuda")
    qn = P.f64(q.cpu())
    osc, _ = P.oracle_units(fm, qn, ok, ov, (1, 1, 3), want_attn=False)
    sc = tq.tq_scores(fm.kf, q, kco, 1, 3)
    torch.cuda.synchronize()
    P.check_scores(sc.double().cpu().numpy(), osc, qn, ok.knorm.reshape(1, 1, 3), 1)
    assert torch.all(sc[:, :, 0] == 0)
    kco1 = tq.KeyCache(kco.codes[:, :, 2:3].clone(), kco.signs[:, :, 2:3].clone(),
                       kco.knorm[:, :, 2:3].clone(), kco.rnorm[:, :, 2:3].clone())
    sc1 = tq.tq_scores(fm.kf, q, kco1, 1, 1)
    torch.cuda.synchronize()
    assert torch.equal(sc1[:, :, 0], sc[:, :, 2])
    # T = 0: zeros, and compression is a no-op
    out0 = torch.full((1, 4, 128), 7.0, device="cuda")
    tq.tq_attend_decode(fm.kf, fm.vf, q, kc1, vc1, 1, 0, out=out0)
    torch.cuda.synchronize()
    assert torch.all(out0 == 0)


def test_strided_layouts_agree(torch_cuda):
    torch = torch_cuda
    w = W.WORKLOADS["batched-8b-32k"].with_T(300, B=2)
    fm = P.Formats(w, 0)
    k = W.make_keys(w, device="cuda")
    v = W.make_values(w, device="cuda")
    kc, vc = P.gpu_compress(fm, k, v)
    # the same tensors stored token-major ([B, T, H, d]) and viewed as [B, H, T, d]
    k2 = k.transpose(1, 2).contiguous().transpose(1, 2)
    v2 = v.transpose(1, 2).contiguous().transpose(1, 2)
    kc2, vc2 = P.gpu_compress(fm, k2, v2)
    torch.cuda.synchronize()
    for a, b in [(kc.codes, kc2.codes), (kc.signs, kc2.signs), (kc.knorm, kc2.knorm),
                 (kc.rnorm, kc2.rnorm), (vc.codes, vc2.codes), (vc.params, vc2.params)]:
        assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["asym-d256", "long-1m"])
def test_compressor_tilings_agree(torch_cuda, name):
    """One large launch (64 keys per workgroup; at d = 256 the residual and
    sign steps in two passes) and small launches of the same keys (32 keys per
    workgroup) pack the same planes, bit for bit; sampled rows of the large
    launch match the oracle."""
    torch = torch_cuda
    w = W.WORKLOADS[name].with_T(4096, B=4 if name == "asym-d256" else 1)
    assert w.B * w.Hkv * w.T >= 64 * 512          # the large launch takes the 64-key tiling
    fm = P.Formats(w, 0)
    k = W.make_keys(w, device="cuda")
    v = W.make_values(w, device="cuda")
    kc, _ = P.gpu_compress(fm, k, v)
    parts = []
    for b in range(w.B):
        for h in range(w.Hkv):
            one = tq.alloc_key_cache(fm.kf, 1, 1, 256, device="cuda")
            tq.tq_compress_keys(fm.kf, k[b:b + 1, h:h + 1, :256], one)
            parts.append(one)
    torch.cuda.synchronize()
    for i, one in enumerate(parts):
        b, h = divmod(i, w.Hkv)
        for big, small in [(kc.codes, one.codes), (kc.signs, one.signs), (kc.knorm, one.knorm), (kc.rnorm, one.rnorm)]:
            assert torch.equal(big[b, h, :256], small[0, 0]), f"unit ({b}, {h})"
    rows = np.random.default_rng(5).choice(w.B * w.Hkv * w.T, 48, replace=False)
    kn = P.f64(k.cpu()).reshape(-1, w.d)
    P.compare_keys(fm, kc, kn[rows], row_index=rows)


def test_deterministic(torch_cuda):
    torch = torch_cuda
    w = _reduced("asym-d256")
    fm = P.Formats(w, 0)
    k, v, q = W.make_keys(w, device="cuda"), W.make_values(w, device="cuda"), W.make_queries(w, device="cuda")
    a = P.gpu_compress(fm, k, v)
    b = P.gpu_compress(fm, k, v)
    o1 = tq.tq_attend_decode(fm.kf, fm.vf, q, a[0], a[1], w.Hkv, w.T)
    o2 = tq.tq_attend_decode(fm.kf, fm.vf, q, a[0], a[1], w.Hkv, w.T)
    torch.cuda.synchronize()
    assert torch.equal(a[0].codes, b[0].codes) and torch.equal(a[0].signs, b[0].signs)
    assert torch.equal(a[1].codes, b[1].codes) and torch.equal(a[1].params, b[1].params)
    assert torch.equal(o1, o2)

"""Parity at the full workload sizes, in the launch configuration bench.py
times (auto split count, whole tensors in one call).

Compression: every row is produced by the GPU; one whole (sequence, KV head)
slice and a seeded sample of rows (plus the first and last) are re-encoded by
the oracle and compared under the flip rule.  Decode: a seeded random packed
cache of the full shape (uniform codes
and signs, realistic norms and value scales; flat and one-hot softmax
regimes) is attended on the GPU; the oracle recomputes whole sampled
(sequence, KV head) units over all T tokens.
"""
import numpy as np
import pytest

import attention_decode_amd as tq
from attention_decode_amd import workloads as W
import oracle as O
import parity as P

pytestmark = pytest.mark.gpu

NAMES = ["tiny", "qwen25-3b-8k", "batched-8b-32k", "long-1m", "asym-d256"]


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available()
    return torch


def _sample_rows(n_total, k, seed):
    rng = np.random.default_rng(seed)
    rows = rng.choice(n_total, size=min(k, n_total), replace=False)
    return np.unique(np.concatenate([rows, [0, n_total - 1]]))


@pytest.mark.parametrize("name", NAMES)
def test_fullsize_compression(torch_cuda, name):
    """Whole-tensor compression in the benchmark's launch configuration: one
    whole (sequence, KV head) slice (the last one, all T tokens) and a seeded
    sample of rows from everywhere else are re-encoded by the oracle and
    compared under the flip rule; the flip budget is checked on the slice's
    T x 2d coordinates."""
    torch = torch_cuda
    w = W.WORKLOADS[name]
    layer = w.layers - 1
    w1 = w.with_T(w.T, layers=1)
    print(f"[full] compress {name} layer {layer}: {w.B}x{w.Hkv}x{w.T}x{w.d}", flush=True)
    fm = P.Formats(w, layer)
    k = W.make_keys(w, layer, device="cuda")
    v = W.make_values(w, layer, device="cuda")
    kc, vc = P.gpu_compress(fm, k, v)
    torch.cuda.synchronize()
    b, h = w.B - 1, w.Hkv - 1
    base = (b * w.Hkv + h) * w.T
    tot = {"code_flips": 0, "sign_flips": 0, "flipped_keys": 0, "coords": 0}
    vflips = 0
    step = 65536
    for lo in range(0, w.T, step):
        hi = min(lo + step, w.T)
        rows = base + np.arange(lo, hi)
        st = P.compare_keys(fm, kc, k[b, h, lo:hi].double().cpu().numpy(), row_index=rows)
        vflips += P.compare_values(fm, vc, v[b, h, lo:hi].double().cpu().numpy(), row_index=rows)
        for key in tot:
            tot[key] += st[key]
    assert tot["code_flips"] + tot["sign_flips"] <= P.FLIP_FRAC * tot["coords"]
    n_total = w1.B * w1.Hkv * w1.T
    rows = _sample_rows(n_total, 384, sum(map(ord, name)))
    idx = torch.from_numpy(rows).cuda()
    krows = k.reshape(-1, w.d).index_select(0, idx).double().cpu().numpy()
    vrows = v.reshape(-1, w.d).index_select(0, idx).double().cpu().numpy()
    sampled = P.compare_keys(fm, kc, krows, row_index=rows)
    vflips += P.compare_values(fm, vc, vrows, row_index=rows)
    print(f"[full] {name}: slice ({b}, {h}) of {w.T} keys {tot}; {rows.size} sampled rows {sampled}; "
          f"value flips {vflips}", flush=True)
    del k, v, kc, vc
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", NAMES)
@pytest.mark.parametrize("peaked", [False, True])
def test_fullsize_decode_sampled_units(torch_cuda, name, peaked):
    torch = torch_cuda
    w = W.WORKLOADS[name].with_T(W.WORKLOADS[name].T, layers=1)
    print(f"[full] decode {name} peaked={peaked}: {w.B}x{w.Hkv}x{w.T}", flush=True)
    fm = P.Formats(w, 0)
    pc = W.random_packed_cache(w, 0, device="cuda", peaked=peaked)
    kc = tq.KeyCache(pc["codes"], pc["signs"], pc["knorm"], pc["rnorm"])
    vc = tq.ValueCache(pc["vcodes"], pc["vparams"])
    q = W.make_queries(w, 0, device="cuda")
    out = tq.tq_attend_decode(fm.kf, fm.vf, q, kc, vc, w.Hkv, w.T)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    units = {(0, 0), (w.B - 1, w.Hkv - 1)}
    if w.B * w.Hkv > 2:
        units.add((int(rng.integers(w.B)), int(rng.integers(w.Hkv))))
    G = w.G
    worst = worst_rel = 0.0
    for b, h in sorted(units):
        okc = O.KeyCache(pc["codes"][b, h].cpu().numpy(), pc["signs"][b, h].cpu().numpy(),
                         pc["knorm"][b, h].cpu().numpy(), pc["rnorm"][b, h].cpu().numpy())
        ovc = O.ValueCache(pc["vcodes"][b, h].cpu().numpy(),
                           pc["vparams"][b, h].cpu().numpy().view(np.uint16))
        qq = q[b, h * G:(h + 1) * G].double().cpu().numpy()
        ref = O.attend(qq, okc, w.k_bits, fm.orot, ovc, w.v_bits, w.group)
        got = out[b, h * G:(h + 1) * G].double().cpu().numpy()
        worst = max(worst, P.check_attention(got, ref))
        worst_rel = max(worst_rel, P.attention_rel_err(got, ref))
    print(f"[full] {name} peaked={peaked}: units {sorted(units)} max abs err {worst:.3g}, "
          f"relative to the row's largest output {worst_rel:.3g}", flush=True)
    del pc, kc, vc
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", NAMES)
def test_fullsize_scores_sampled_unit(torch_cuda, name):
    torch = torch_cuda
    w = W.WORKLOADS[name].with_T(W.WORKLOADS[name].T, layers=1)
    fm = P.Formats(w, 0)
    pc = W.random_packed_cache(w, 0, device="cuda")
    kc = tq.KeyCache(pc["codes"], pc["signs"], pc["knorm"], pc["rnorm"])
    q = W.make_queries(w, 0, device="cuda")
    sc = tq.tq_scores(fm.kf, q, kc, w.Hkv, w.T)
    torch.cuda.synchronize()
    b, h, G = w.B - 1, w.Hkv - 1, w.G
    okc = O.KeyCache(pc["codes"][b, h].cpu().numpy(), pc["signs"][b, h].cpu().numpy(),
                     pc["knorm"][b, h].cpu().numpy(), pc["rnorm"][b, h].cpu().numpy())
    qq = q[b, h * G:(h + 1) * G].double().cpu().numpy()
    ref = O.scores(qq, okc, w.k_bits, fm.orot)
    got = sc[b, h * G:(h + 1) * G].double().cpu().numpy()
    r = P.check_scores(got[None], ref[None], qq[None], okc.knorm[None, None], 1)
    print(f"[full] scores {name}: {r:.3g} x bound", flush=True)

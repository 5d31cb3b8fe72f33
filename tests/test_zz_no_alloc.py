"""The allocation-free decode entry point, tq_attend_decode_noalloc, through
the C ABI: its workspace is the library's static device scratch.

Each call is checked against tq_attend_decode (the workspace entry point) on
the same inputs, bit for bit (the same kernels and split plan), and against
the oracle's attention within the 1e-3 bar.  Calls run back to back on one
GPU, the second on a smaller input than the first, then a third on the first
input with another split count, so the scratch holds the previous call's
contents each time.  A shape whose workspace exceeds the scratch is refused
before anything is launched."""
import pytest

import attention_decode_amd as tq
from attention_decode_amd import _lib as L
from attention_decode_amd import workloads as W
import oracle as O
import parity as P

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 16 << 20


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available()
    return torch


def _case(w):
    """Formats, the oracle's packed cache on the device, queries, and the
    oracle's attention of every (sequence, KV head) unit."""
    fm = P.Formats(w, 0)
    k, v, q = W.make_keys(w), W.make_values(w), W.make_queries(w)
    ok = O.compress_keys(P.f64(k).reshape(-1, w.d), w.k_bits, fm.orot)
    ov = O.compress_values(P.f64(v).reshape(-1, w.d), w.v_bits, w.group)
    shape = (w.B, w.Hkv, w.T)
    kc, vc = P.to_device_cache(ok, ov, shape, "cuda")
    _, want = P.oracle_units(fm, P.f64(q), ok, ov, shape)
    return fm, kc, vc, q.cuda(), want


def _run(torch, w, case, n_splits):
    fm, kc, vc, q, want = case
    assert tq.tq_attend_workspace_bytes(fm.kf, w.B, w.Hq, w.Hkv, w.T, n_splits) <= SCRATCH_BYTES
    out = torch.full((w.B, w.Hq, w.d), float("nan"), dtype=torch.float32, device="cuda")
    tq.tq_attend_decode_noalloc(fm.kf, fm.vf, q, kc, vc, w.Hkv, w.T, out, n_splits=n_splits)
    ref = tq.tq_attend_decode(fm.kf, fm.vf, q, kc, vc, w.Hkv, w.T, n_splits=n_splits)
    torch.cuda.synchronize()
    assert torch.equal(out, ref), float((out - ref).abs().max())
    err = P.check_attention(out.double().cpu().numpy(), want)
    print(f"[noalloc] {w.name} B={w.B} Hkv={w.Hkv} T={w.T} d={w.d} splits={n_splits}: "
          f"equal to tq_attend_decode, oracle max abs err {err:.3g}", flush=True)


def test_noalloc_matches_workspace_entry_point(torch_cuda):
    torch = torch_cuda
    big = W.WORKLOADS["asym-d256"].with_T(1000, B=2)           # d 256, 7+1-bit keys, 2 splits or more
    small = W.WORKLOADS["qwen25-3b-8k"].with_T(300, layers=1)  # d 128, 2+1-bit keys, a smaller input
    cb, cs = _case(big), _case(small)
    _run(torch, big, cb, 0)
    _run(torch, small, cs, 0)
    _run(torch, big, cb, 3)


def test_noalloc_refuses_shapes_beyond_the_scratch(torch_cuda):
    torch = torch_cuda
    w = W.WORKLOADS["batched-8b-32k"].with_T(512, B=256)
    fm = P.Formats(w, 0)
    need = tq.tq_attend_workspace_bytes(fm.kf, w.B, w.Hq, w.Hkv, w.T, 0)
    assert need > SCRATCH_BYTES
    # real planes of the full shape (zeros), so that even a launch would stay in bounds
    shp = (w.B, w.Hkv, w.T)
    kc = tq.KeyCache(torch.zeros(shp + (w.d * w.k_bits // 8,), dtype=torch.uint8, device="cuda"),
                     torch.zeros(shp + (w.d // 8,), dtype=torch.uint8, device="cuda"),
                     torch.zeros(shp, dtype=torch.float32, device="cuda"),
                     torch.zeros(shp, dtype=torch.float32, device="cuda"))
    vc = tq.ValueCache(torch.zeros(shp + (w.d * w.v_bits // 8,), dtype=torch.uint8, device="cuda"),
                       torch.zeros(shp + (w.d // w.group, 2), dtype=torch.int16, device="cuda"))
    q = W.make_queries(w, 0, device="cuda")
    out = torch.full((w.B, w.Hq, w.d), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(L.TQError) as ei:
        tq.tq_attend_decode_noalloc(fm.kf, fm.vf, q, kc, vc, w.Hkv, w.T, out)
    torch.cuda.synchronize()
    assert ei.value.status == L.TQ_ENOMEM
    assert "static scratch" in str(ei.value)
    assert torch.all(out == 7.0)          # nothing was launched
    print(f"[noalloc] refused {need} B > {SCRATCH_BYTES} B: {ei.value}", flush=True)

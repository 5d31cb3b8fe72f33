"""Launch failures on the GPU path map to TQ_EHIP.  The failure is forced from
the host (TQ_TEST_HOOK=launch: each entry point reports a launch failure
after its argument checks and launches nothing), so no kernel faults: the
test checks the status, the message, and that no output was touched."""
import pytest

import attention_decode_amd as tq
from attention_decode_amd import _lib as L
from attention_decode_amd import workloads as W
import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available()
    return torch


def test_forced_launch_failure_reports_ehip(torch_cuda, monkeypatch):
    torch = torch_cuda
    w = W.WORKLOADS["tiny"].with_T(64)
    fm = P.Formats(w, 0)
    k, v, q = W.make_keys(w, device="cuda"), W.make_values(w, device="cuda"), W.make_queries(w, device="cuda")
    kc = tq.alloc_key_cache(fm.kf, w.B, w.Hkv, w.T)
    vc = tq.alloc_value_cache(fm.vf, w.B, w.Hkv, w.T)
    for t in (kc.codes, kc.signs, vc.codes):
        t.fill_(0xAB)
    for t in (kc.knorm, kc.rnorm):
        t.fill_(3.0)
    vc.params.fill_(0x1234)
    out = torch.full((w.B, w.Hq, w.d), 5.0, device="cuda")
    sc = torch.full((w.B, w.Hq, w.T), 5.0, device="cuda")
    torch.cuda.synchronize()
    monkeypatch.setenv("TQ_TEST_HOOK", "launch")
    calls = [
        ("tq_compress_keys", lambda: tq.tq_compress_keys(fm.kf, k, kc)),
        ("tq_compress_values", lambda: tq.tq_compress_values(fm.vf, v, vc)),
        ("tq_scores", lambda: tq.tq_scores(fm.kf, q, kc, w.Hkv, w.T, out=sc)),
        ("tq_attend_decode", lambda: tq.tq_attend_decode(fm.kf, fm.vf, q, kc, vc, w.Hkv, w.T, out=out)),
        ("tq_attend_decode_noalloc", lambda: tq.tq_attend_decode_noalloc(fm.kf, fm.vf, q, kc, vc, w.Hkv, w.T, out)),
    ]
    for name, call in calls:
        with pytest.raises(L.TQError) as ei:
            call()
        assert ei.value.status == L.TQ_EHIP, name
        assert name in str(ei.value)
    torch.cuda.synchronize()
    assert torch.all(kc.codes == 0xAB) and torch.all(kc.knorm == 3.0) and torch.all(vc.codes == 0xAB)
    assert torch.all(out == 5.0) and torch.all(sc == 5.0)
    # the same calls run once the hook is gone
    monkeypatch.delenv("TQ_TEST_HOOK")
    tq.tq_compress_keys(fm.kf, k, kc)
    tq.tq_attend_decode(fm.kf, fm.vf, q, kc, vc, w.Hkv, w.T, out=out)
    torch.cuda.synchronize()
    assert not torch.all(kc.codes == 0xAB)

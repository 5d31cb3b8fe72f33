"""Decode launches replayed from a captured HIP graph give the eager results.

The per-layer decode (q-prep, split-K attention, split merge), or tq_scores,
is captured once for several layers and replayed three times; before each replay the queries
are rewritten in place and the eager launches run on the same inputs, so each
replay must reproduce the eager outputs bit for bit (same kernels, same launch
configuration, no state kept between calls)."""
import numpy as np
import pytest

import attention_decode_amd as tq
from attention_decode_amd import workloads as W

pytestmark = pytest.mark.gpu

LAYERS = 3


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available()
    return torch


def _layers(torch, kind):
    w = W.Workload("graph", LAYERS, 2, 2, 16, 777, 128, "bfloat16", 2, "dense", 2, 32, "iid", 0.0, 61)
    out = []
    for l in range(LAYERS):
        rot = tq.tq_make_rotation(w.rotation_seed(l), w.d, w.rot)
        vf = tq.ValueFormat(w.d, w.v_bits, w.group)
        pc = W.random_packed_cache(w, l, device="cuda")
        vc = tq.ValueCache(pc["vcodes"], pc["vparams"])
        q = W.make_queries(w, l, device="cuda")
        o = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
        if kind == "q8_0":
            bf = tq.BlockFormat(w.d, 8, rot)
            g = torch.Generator(device="cuda")
            g.manual_seed(100 + l)
            codes = torch.randint(-127, 128, (w.B, w.Hkv, w.T, w.d), generator=g, device="cuda",
                                  dtype=torch.int16).to(torch.int8).view(torch.uint8)
            scales = (0.02 * (0.5 + torch.rand((w.B, w.Hkv, w.T, w.d // 32), generator=g, device="cuda"))).half()
            kc = tq.BlockCache(codes, scales.view(torch.int16))
            ws = torch.empty(tq.tq_attend_block_workspace_bytes(bf, w.B, w.Hq, w.Hkv, w.T), dtype=torch.uint8,
                             device="cuda")
            call = (lambda bf=bf, vf=vf, q=q, kc=kc, vc=vc, o=o, ws=ws:
                    tq.tq_attend_decode_block(bf, vf, q, kc, vc, w.Hkv, w.T, out=o, ws=ws))
        else:
            cb = tq.tq_build_codebook(w.d, w.k_bits)
            kf = tq.KeyFormat(w.d, w.k_bits, cb, rot)
            kc = tq.KeyCache(pc["codes"], pc["signs"], pc["knorm"], pc["rnorm"])
            if kind == "scores":
                o = torch.empty((w.B, w.Hq, w.T), dtype=torch.float32, device="cuda")
                ws = torch.empty(tq.tq_scores_workspace_bytes(kf, w.B, w.Hq), dtype=torch.uint8, device="cuda")
                call = (lambda kf=kf, q=q, kc=kc, o=o, ws=ws:
                        tq.tq_scores(kf, q, kc, w.Hkv, w.T, out=o, ws=ws))
            elif kind == "flat":
                ws = torch.empty(tq.tq_attend_workspace_bytes(kf, w.B, w.Hq, w.Hkv, w.T), dtype=torch.uint8,
                                 device="cuda")
                call = (lambda kf=kf, vf=vf, q=q, kc=kc, vc=vc, o=o, ws=ws:
                        tq.tq_attend_decode(kf, vf, q, kc, vc, w.Hkv, w.T, out=o, ws=ws))
            else:
                # the same planes as a contiguous layout cache with ragged lengths
                lens = torch.tensor([w.T, w.T - 300], dtype=torch.int32, device="cuda")
                lay = tq.CacheLayout(w.T, lens)
                flat = lambda x: x.reshape(w.B * w.Hkv * w.T, *x.shape[3:])
                kc = tq.KeyCache(flat(pc["codes"]), flat(pc["signs"]), flat(pc["knorm"]), flat(pc["rnorm"]))
                vc = tq.ValueCache(flat(pc["vcodes"]), flat(pc["vparams"]))
                ws = torch.empty(tq.tq_attend_paged_workspace_bytes(kf, w.B, w.Hq, w.Hkv, lay), dtype=torch.uint8,
                                 device="cuda")
                call = (lambda kf=kf, vf=vf, q=q, kc=kc, vc=vc, o=o, ws=ws, lay=lay:
                        tq.tq_attend_decode_paged(kf, vf, q, kc, vc, w.Hkv, lay, out=o, ws=ws))
        out.append((q, o, call, (rot, vf, pc, kc, vc, ws)))
    return w, out


@pytest.mark.parametrize("kind", ["flat", "layout", "q8_0", "scores"])
def test_graph_replay_matches_eager(torch_cuda, kind):
    torch = torch_cuda
    w, layers = _layers(torch, kind)
    print(f"[graph] {kind}: {LAYERS} layers, B={w.B} Hq={w.Hq} T={w.T}", flush=True)
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for _, _, call, _ in layers:
            call()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _, _, call, _ in layers:
            call()
    torch.cuda.synchronize()
    g = torch.Generator(device="cuda")
    for rep in range(3):
        g.manual_seed(1000 + rep)
        for q, _, _, _ in layers:
            q.copy_(torch.randn(q.shape, generator=g, device="cuda").to(q.dtype))
        for _, o, call, _ in layers:          # eager launches on the new queries
            call()
        torch.cuda.synchronize()
        want = [o.clone() for _, o, _, _ in layers]
        for _, o, _, _ in layers:
            o.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for l, (_, o, _, _) in enumerate(layers):
            assert torch.equal(o, want[l]), f"replay {rep}, layer {l}"
            assert torch.isfinite(o).all()
        print(f"[graph] {kind}: replay {rep} matches eager", flush=True)

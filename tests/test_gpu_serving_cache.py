"""GPU parity of the serving-style cache: appends into a preallocated cache
(contiguous with a capacity, or a pool of blocks behind a block table) and
decode attention over ragged sequence lengths through the block table.

Appended rows are compared with the oracle's encoding of the same tokens
(codes and signs bit-exact except coordinates within 1e-5 of a decision
boundary, norms, value planes) and with the flat compressor's rows (bit for
bit: the same per-key arithmetic); the paged decode must match the oracle's
attention over each sequence's first seq_lens[b] tokens (1e-3 absolute)."""
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


def _layout(torch, B, cap, block_size, rng, extra_blocks=3):
    """Contiguous (block_size 0) or paged layout with shuffled physical blocks."""
    lens = torch.zeros(B, dtype=torch.int32, device="cuda")
    if block_size == 0:
        return tq.CacheLayout(cap, lens), None
    maxb = cap // block_size
    nblocks = B * maxb + extra_blocks
    perm = rng.permutation(nblocks)[: B * maxb].reshape(B, maxb).astype(np.int32)
    bt = torch.from_numpy(perm).cuda()
    return tq.CacheLayout(cap, lens, bt, block_size, nblocks), perm


def _rows(perm, B, H, cap, bs, b, h, t):
    """Host copy of the layout's row formula."""
    if perm is None:
        return (b * H + h) * cap + t
    return (perm[b, t // bs] * H + h) * bs + t % bs


@pytest.mark.parametrize("block_size,m", [(0, None), (32, None), (64, 0), (256, None)])
def test_append_matches_oracle(torch_cuda, block_size, m):
    """Prefill chunks and single-token steps appended at per-sequence positions
    give the oracle's encoding of those tokens (under the flip rule), and
    exactly the rows the flat compressor writes for the same tokens."""
    torch = torch_cuda
    d, bits = 128, 3
    w = replace(BASE, name="append", B=3, Hkv=2, T=256, d=d, k_bits=bits, v_bits=2, group=32, seed=41)
    rng = np.random.default_rng(41)
    cap = 256
    lay, perm = _layout(torch, w.B, cap, block_size, rng)
    cb = tq.tq_build_codebook(d, bits)
    rot = tq.tq_make_rotation(w.rotation_seed(0), d, w.rot)
    qm = d if m is None else m
    kf = tq.KeyFormat(d, bits, cb, rot, qjl_m=qm)
    vf = tq.ValueFormat(d, w.v_bits, w.group)
    k, v = W.make_keys(w).cuda(), W.make_values(w).cuda()
    # flat reference rows
    fk = tq.alloc_key_cache(kf, w.B, w.Hkv, w.T)
    fv = tq.alloc_value_cache(vf, w.B, w.Hkv, w.T)
    tq.tq_compress_keys(kf, k, fk)
    tq.tq_compress_values(vf, v, fv)
    lk = tq.alloc_layout_key_cache(kf, lay, w.B, w.Hkv)
    lv = tq.alloc_layout_value_cache(vf, lay, w.B, w.Hkv)
    # sequence b receives tokens [0, fill[b]) of its row of k: a prefill chunk,
    # then single tokens; positions differ per sequence
    fill = [0] * w.B
    steps = [(0, 100), (1, 1), (1, 1), (2, 37), (1, 1)]
    for who, n in steps:
        for b in range(w.B):
            take = n + b * (who == 2)          # ragged: later sequences take more per chunk
            lo = fill[b]
            pos = torch.full((w.B,), cap + 5, dtype=torch.int32, device="cuda")   # others: past capacity, skipped
            pos[b] = lo
            chunk_k = k[:, :, lo:lo + take].contiguous()
            chunk_v = v[:, :, lo:lo + take].contiguous()
            tq.tq_append_keys(kf, chunk_k, lay, pos, lk)
            tq.tq_append_values(vf, chunk_v, lay, pos, lv)
            fill[b] += take
    torch.cuda.synchronize()
    # against the oracle: every appended row, encoded by the oracle from the
    # same input tokens
    fm = P.Formats(w, 0)
    kin, vin = P.f64(k.cpu()), P.f64(v.cpu())
    src_k, src_v, at = [], [], []
    for b in range(w.B):
        for h in range(w.Hkv):
            t = np.arange(fill[b])
            src_k.append(kin[b, h, t])
            src_v.append(vin[b, h, t])
            at.append(_rows(perm, w.B, w.Hkv, cap, block_size, b, h, t))
    at = np.concatenate(at)
    kstats = P.compare_keys(fm, lk, np.concatenate(src_k), row_index=at)
    vflips = P.compare_values(fm, lv, np.concatenate(src_v), row_index=at)
    print(f"[append] block_size={block_size} m={qm}: oracle {kstats}, value flips {vflips}", flush=True)
    # against the flat compressor: bit for bit
    for b in range(w.B):
        for h in range(w.Hkv):
            t = np.arange(fill[b])
            rows = _rows(perm, w.B, w.Hkv, cap, block_size, b, h, t)
            fr = (b * w.Hkv + h) * w.T + t
            assert torch.equal(lk.codes[rows], fk.codes.reshape(-1, fk.codes.shape[-1])[fr])
            assert torch.equal(lk.knorm[rows], fk.knorm.reshape(-1)[fr])
            if qm:
                assert torch.equal(lk.signs[rows], fk.signs.reshape(-1, fk.signs.shape[-1])[fr])
                assert torch.equal(lk.rnorm[rows], fk.rnorm.reshape(-1)[fr])
            assert torch.equal(lv.codes[rows], fv.codes.reshape(-1, fv.codes.shape[-1])[fr])
            assert torch.equal(lv.params[rows], fv.params.reshape(-1, *fv.params.shape[-2:])[fr])
    # rows never appended stay untouched (zero)
    written = np.zeros(lk.codes.shape[0], bool)
    for b in range(w.B):
        for h in range(w.Hkv):
            written[_rows(perm, w.B, w.Hkv, cap, block_size, b, h, np.arange(fill[b]))] = True
    assert int(lk.codes[torch.from_numpy(~written).cuda()].abs().sum()) == 0
    print(f"[append] block_size={block_size} m={qm}: fills {fill}", flush=True)


CASES = [
    # (d, k_bits, qjl, Hkv, Hq, v_bits, group, block_size, lens)
    (128, 2, True, 2, 16, 2, 32, 32, [0, 1, 31, 200]),        # bit-plane scores, GQA 8
    (128, 3, True, 2, 8, 2, 64, 64, [129, 63, 64, 256]),       # table scores
    (128, 3, False, 1, 4, 4, 32, 32, [97, 33]),                # first-stage keys
    (256, 7, True, 1, 2, 4, 32, 128, [255, 1]),                # largest format
    (128, 2, True, 2, 4, 4, 32, 0, [5, 256, 77]),              # contiguous layout
    (64, 3, True, 1, 4, 2, 32, 32, [300, 17]),                 # d 64 (general kernel)
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "d{}b{}{}bs{}".format(c[0], c[1], "" if c[2] else "mse", c[7]))
def test_paged_decode_matches_oracle(torch_cuda, case):
    torch = torch_cuda
    d, kb, qjl, Hkv, Hq, vb, g, bs, lens = case
    B = len(lens)
    cap = 320 if bs in (0, 32, 64) else 384
    if bs:
        cap = (cap // bs) * bs
    T = max(lens)
    w = replace(BASE, name="paged", B=B, Hkv=Hkv, Hq=Hq, T=T, d=d, k_bits=kb, v_bits=vb, group=g, seed=42,
                dtype="bfloat16")
    rng = np.random.default_rng(42 + bs)
    lay, perm = _layout(torch, B, cap, bs, rng)
    lay.seq_lens.copy_(torch.tensor(lens, dtype=torch.int32))
    m = d if qjl else 0
    cb = tq.tq_build_codebook(d, kb)
    rot = tq.tq_make_rotation(w.rotation_seed(0), d, w.rot)
    kf = tq.KeyFormat(d, kb, cb, rot, qjl_m=m)
    vf = tq.ValueFormat(d, vb, g)
    orot = O.rotation(w.rotation_seed(0), d, w.rot, m=m)
    k, v, q = W.make_keys(w), W.make_values(w), W.make_queries(w)
    ok = O.compress_keys(P.f64(k).reshape(-1, d), kb, orot)
    ov = O.compress_values(P.f64(v).reshape(-1, d), vb, g)
    # scatter the oracle's packed rows into the layout's planes
    lk = tq.alloc_layout_key_cache(kf, lay, B, Hkv)
    lv = tq.alloc_layout_value_cache(vf, lay, B, Hkv)
    src_rows, dst_rows = [], []
    for b in range(B):
        for h in range(Hkv):
            t = np.arange(lens[b])
            src_rows.append((b * Hkv + h) * T + t)
            dst_rows.append(_rows(perm, B, Hkv, cap, bs, b, h, t))
    sr, dr = np.concatenate(src_rows), torch.from_numpy(np.concatenate(dst_rows)).cuda()
    lk.codes[dr] = torch.from_numpy(ok.codes[sr]).cuda()
    lk.knorm[dr] = torch.from_numpy(ok.knorm[sr]).cuda()
    if qjl:
        lk.signs[dr] = torch.from_numpy(ok.signs[sr]).cuda()
        lk.rnorm[dr] = torch.from_numpy(ok.rnorm[sr]).cuda()
    lv.codes[dr] = torch.from_numpy(ov.codes[sr]).cuda()
    lv.params[dr] = torch.from_numpy(ov.params.view(np.int16)[sr]).cuda()
    # oracle attention of each sequence over its own tokens
    G = Hq // Hkv
    qn = P.f64(q)
    want = np.zeros((B, Hq, d))
    for b in range(B):
        for h in range(Hkv):
            if lens[b] == 0:
                continue
            rows = (b * Hkv + h) * T + np.arange(lens[b])
            okc = O.KeyCache(ok.codes[rows], ok.signs[rows], ok.knorm[rows], ok.rnorm[rows])
            ovc = O.ValueCache(ov.codes[rows], ov.params[rows])
            want[b, h * G:(h + 1) * G] = O.attend(qn[b, h * G:(h + 1) * G], okc, kb, orot, ovc, vb, g)
    qd = q.cuda()
    for splits in (0, 1, 5):
        out = tq.tq_attend_decode_paged(kf, vf, qd, lk, lv, Hkv, lay, n_splits=splits)
        torch.cuda.synchronize()
        err = P.check_attention(out.double().cpu().numpy(), want)
        print(f"[paged] {case} splits={splits}: max abs err {err:.3g}", flush=True)


def test_out_of_pool_blocks_are_skipped(torch_cuda):
    """A block id outside [0, num_blocks) drops that block's tokens (no access);
    the sequence attends its remaining tokens, as the oracle over those does."""
    torch = torch_cuda
    d, kb, Hkv, Hq, bs = 128, 2, 1, 4, 32
    lens = [128, 96]
    B, T, cap = 2, 128, 128
    w = replace(BASE, name="oob", B=B, Hkv=Hkv, Hq=Hq, T=T, seed=43)
    rng = np.random.default_rng(43)
    lay, perm = _layout(torch, B, cap, bs, rng, extra_blocks=0)
    lay.seq_lens.copy_(torch.tensor(lens, dtype=torch.int32))
    cb = tq.tq_build_codebook(d, kb)
    rot = tq.tq_make_rotation(w.rotation_seed(0), d, w.rot)
    kf, vf = tq.KeyFormat(d, kb, cb, rot), tq.ValueFormat(d, 2, 32)
    orot = O.rotation(w.rotation_seed(0), d, w.rot)
    k, v, q = W.make_keys(w), W.make_values(w), W.make_queries(w)
    ok = O.compress_keys(P.f64(k).reshape(-1, d), kb, orot)
    ov = O.compress_values(P.f64(v).reshape(-1, d), 2, 32)
    lk = tq.alloc_layout_key_cache(kf, lay, B, Hkv)
    lv = tq.alloc_layout_value_cache(vf, lay, B, Hkv)
    sr = np.concatenate([(b * Hkv) * T + np.arange(lens[b]) for b in range(B)])
    dr = np.concatenate([_rows(perm, B, Hkv, cap, bs, b, 0, np.arange(lens[b])) for b in range(B)])
    drt = torch.from_numpy(dr).cuda()
    lk.codes[drt] = torch.from_numpy(ok.codes[sr]).cuda()
    lk.signs[drt] = torch.from_numpy(ok.signs[sr]).cuda()
    lk.knorm[drt] = torch.from_numpy(ok.knorm[sr]).cuda()
    lk.rnorm[drt] = torch.from_numpy(ok.rnorm[sr]).cuda()
    lv.codes[drt] = torch.from_numpy(ov.codes[sr]).cuda()
    lv.params[drt] = torch.from_numpy(ov.params.view(np.int16)[sr]).cuda()
    # sequence 0: block 1 points outside the pool, block 2 is negative
    bt = lay.block_table.cpu()
    bt[0, 1] = lay.num_blocks + 7
    bt[0, 2] = -3
    lay.block_table.copy_(bt)
    out = tq.tq_attend_decode_paged(kf, vf, q.cuda(), lk, lv, Hkv, lay, n_splits=3)
    torch.cuda.synchronize()
    qn = P.f64(q)
    keep = [np.r_[0:32, 96:128], np.arange(96)]
    want = np.zeros((B, Hq, d))
    for b in range(B):
        rows = b * Hkv * T + keep[b]
        okc = O.KeyCache(ok.codes[rows], ok.signs[rows], ok.knorm[rows], ok.rnorm[rows])
        ovc = O.ValueCache(ov.codes[rows], ov.params[rows])
        want[b] = O.attend(qn[b], okc, kb, orot, ovc, 2, 32)
    P.check_attention(out.double().cpu().numpy(), want)

"""Key compression against the oracle at every code width the compressor
takes (1 to 7 Lloyd-Max bits) and every head dimension (64, 128, 256), dense
rotation with the QJL sign row, bf16 and fp32 inputs: the register codes
(up to 2 bits) and the code-cell table (from 3 bits) on each kernel shape.
Each case spans several 64-key workgroups and ends in a ragged one.

Bars (the same as every compression test): codes bit-exact except
coordinates within 1e-5 of a decision boundary, where the flipped key's
residual norm and signs must match the oracle's encoding with the other
code; ||k|| relative 1e-6; ||r|| relative 1e-5; signs exact except where
|S r| < 1e-5 ||r||."""
from dataclasses import replace

import pytest

from attention_decode_amd import workloads as W
import parity as P

pytestmark = pytest.mark.gpu

BASE = W.WORKLOADS["tiny"]


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available()
    return torch


@pytest.mark.parametrize("dtype", ["bfloat16", "float32"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 7])
def test_compress_every_width(torch_cuda, bits, d, dtype):
    torch = torch_cuda
    w = replace(BASE, name="sweep", B=1, Hkv=3, T=111, d=d, k_bits=bits, rot="dense", dtype=dtype,
                keys="iid", kv_ratio=0.0, seed=71 + bits)
    print(f"[sweep] d={d} bits={bits} dtype={dtype} keys={w.B * w.Hkv * w.T}", flush=True)
    fm = P.Formats(w, 0)
    k, v = W.make_keys(w), W.make_values(w)
    kc, _ = P.gpu_compress(fm, k.cuda(), v.cuda())
    torch.cuda.synchronize()
    stats = P.compare_keys(fm, kc, P.f64(k).reshape(-1, w.d))
    print(f"[sweep] d={d} bits={bits} dtype={dtype}: {stats}", flush=True)

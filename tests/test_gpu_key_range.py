"""Key compression of 2-byte keys (bf16, fp16) across the supported key range,
against the oracle.

Under a dense rotation these keys take the fp16 form of y = Pi k: each key is
staged times a power of two of its own, chosen from its norm, and Pi is two
fp16 terms.  The cases put that scaling at its edges: norms near both ends of
the supported range (2^-60, 2^64) for bf16, fp16 inputs whose elements are
fp16 subnormals, keys whose one nonzero element carries the whole norm (the
largest staged element), zero keys, and keys whose elements span a wide
dynamic range (tiny elements round on fp16's subnormal grid after scaling).
Each case has more than 512 64-key workgroups, so both key tilings run, and
ends in a ragged workgroup.

Bars (the same as every compression test): codes bit-exact except
coordinates within 1e-5 of a decision boundary, where the flipped key's
residual norm and signs must match the oracle's encoding with the other
code; ||k|| relative 1e-6; ||r|| relative 1e-5; signs exact except where
|S r| < 1e-5."""
from dataclasses import replace

import numpy as np
import pytest

from attention_decode_amd import workloads as W
import parity as P

pytestmark = pytest.mark.gpu

T_KEYS = 33_001          # > 512 workgroups of 64 keys, ragged last workgroup


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available()
    return torch


def _keys(torch, d, dtype, seed):
    """[T_KEYS, d] keys in `dtype`: five blocks of rows at different scales,
    then one-hot, zero and wide-range rows."""
    g = torch.Generator().manual_seed(seed)
    base = torch.randn((T_KEYS, d), generator=g, dtype=torch.float64)
    if dtype == "bfloat16":
        scales = [2.0 ** -55, 2.0 ** -20, 1.0, 2.0 ** 30, 2.0 ** 58]
        peak = 2.0 ** 62            # one-hot element: ||k|| = 2^62
        tdt = torch.bfloat16
    else:
        scales = [2.0 ** -12, 2.0 ** -6, 1.0, 2.0 ** 6, 2.0 ** 12]   # 2^-12: mostly fp16 subnormals
        peak = 60000.0              # near fp16's largest finite value
        tdt = torch.float16
    k = base.clone()
    n = T_KEYS // 8
    for i, s in enumerate(scales):
        k[i * n:(i + 1) * n] *= s
    r0 = 5 * n
    # one-hot rows: the whole norm on one element, at a different channel per row
    for i in range(64):
        k[r0 + i] = 0.0
        k[r0 + i, (7 * i) % d] = peak if i % 2 == 0 else -peak
    # zero rows
    k[r0 + 64:r0 + 96] = 0.0
    # wide dynamic range: one element 2^20 times the rest
    wide = k[r0 + 96:r0 + 96 + n]
    wide[:, 3] *= 2.0 ** 20 if dtype == "bfloat16" else 2.0 ** 10
    return k.to(tdt)


@pytest.mark.parametrize("dtype", ["bfloat16", "float16"])
@pytest.mark.parametrize("name", ["qwen25-3b-8k", "long-1m", "asym-d256"])
def test_two_byte_keys_across_the_range(torch_cuda, name, dtype):
    torch = torch_cuda
    w0 = W.WORKLOADS[name]
    w = replace(w0, name="range", B=1, Hkv=1, T=T_KEYS, dtype=dtype, rot="dense")
    print(f"[range] {name} d={w.d} bits={w.k_bits} dtype={dtype} keys={T_KEYS}", flush=True)
    fm = P.Formats(w, 0)
    k = _keys(torch, w.d, dtype, seed=1234 + w.d + w.k_bits)
    kf = k.reshape(1, 1, T_KEYS, w.d)
    v = torch.zeros((1, 1, T_KEYS, w.d), dtype=k.dtype)
    kc, _ = P.gpu_compress(fm, kf.cuda(), v.cuda())
    torch.cuda.synchronize()
    rows = P.f64(k)
    assert np.all(np.isfinite(rows))
    st = P.compare_keys_chunked(fm, kc, rows, np.arange(T_KEYS))
    print(f"[range] {name} {dtype}: {st}", flush=True)

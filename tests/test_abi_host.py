"""CPU checks of the C ABI: the library loads, exports every entry point the
header declares, builds its host tables like the oracle does (independent
implementations), sizes its planes, and rejects bad arguments before touching
a device."""
import ctypes
import os
import re

import numpy as np
import pytest

import attention_decode_amd as tq
from attention_decode_amd import _lib as L
import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "tq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = L.lib()
    names = _declared()
    assert len(names) >= 19
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.SIGNATURES), set(names) ^ set(L.SIGNATURES)


@pytest.mark.parametrize("d,bits", [(3, 2), (4, 1), (64, 4), (128, 2), (128, 3), (256, 7), (256, 8)])
def test_host_codebook_matches_oracle(d, bits):
    c, t = tq.tq_codebook_host(d, bits)
    oc, ot = O.codebook(d, bits)
    assert np.abs(c - oc).max() < 1e-12
    assert np.abs(t - ot).max() < 1e-12
    assert np.array_equal(c, -c[::-1])


@pytest.mark.parametrize("d,kind", [(64, "dense"), (128, "dense"), (256, "dense"),
                                    (128, "hadamard"), (256, "hadamard"), (128, "hadamard2"),
                                    (256, "hadamard2")])
def test_host_rotation_matches_oracle(d, kind):
    seed = 4242 + d
    pi, s = tq.tq_rotation_host(seed, d, kind)
    ro = O.rotation(seed, d, kind)
    assert np.abs(pi - ro.pi).max() < 1e-12
    assert np.array_equal(s, ro.s)
    assert np.abs(pi.T @ pi - np.eye(d)).max() < 1e-12


def _kf(**kw):
    f = dict(d=128, mse_bits=2, qjl_m=128, cb=None, rot=None)
    f.update(kw)
    return L.KeyFmt(f["d"], f["mse_bits"], f["qjl_m"], f["cb"], f["rot"])


def test_errors_before_any_device_call():
    lib = L.lib()
    h = ctypes.c_void_p()
    assert lib.tq_build_codebook(2, 2, ctypes.byref(h)) == L.TQ_EINVAL
    assert lib.tq_build_codebook(128, 0, ctypes.byref(h)) == L.TQ_EINVAL
    assert lib.tq_build_codebook(128, 9, ctypes.byref(h)) == L.TQ_EINVAL
    assert b"bits" in lib.tq_last_error()
    assert lib.tq_make_rotation(1, 100, 0, ctypes.byref(h)) == L.TQ_EUNSUPPORTED
    assert lib.tq_make_rotation(1, 128, 7, ctypes.byref(h)) == L.TQ_EINVAL
    buf = np.zeros(96 * 96)
    dp = buf.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    assert lib.tq_rotation_host(1, 96, L.TQ_ROT_HADAMARD, dp, dp) == L.TQ_EUNSUPPORTED
    kc, vc = L.KCache(), L.VCache()
    assert lib.tq_compress_keys(None, None, 1, 1, 1, 8, 0, 0, 128, kc, None) == L.TQ_EINVAL
    kf = _kf()
    assert lib.tq_compress_keys(ctypes.byref(kf), None, 1, 1, 1, 8, 0, 0, 128, kc, None) == L.TQ_EINVAL
    assert b"codebook" in lib.tq_last_error()
    vf = L.ValFmt(128, 3, 32)
    assert lib.tq_compress_values(ctypes.byref(vf), None, 1, 1, 1, 8, 0, 0, 128, vc, None) == L.TQ_EUNSUPPORTED
    vf = L.ValFmt(128, 2, 48)
    assert lib.tq_compress_values(ctypes.byref(vf), None, 1, 1, 1, 8, 0, 0, 128, vc, None) == L.TQ_EUNSUPPORTED
    vf = L.ValFmt(64, 2, 128)
    assert lib.tq_compress_values(ctypes.byref(vf), None, 1, 1, 1, 8, 0, 0, 64, vc, None) == L.TQ_EINVAL
    vf = L.ValFmt(128, 2, 32)
    assert lib.tq_compress_values(ctypes.byref(vf), None, 1, 1, 1, 8, 0, 0, 128, vc, None) == L.TQ_EINVAL
    # misaligned input pointer and stride
    assert lib.tq_compress_values(ctypes.byref(vf), ctypes.c_void_p(0x1008), 1, 1, 1, 8, 0, 0, 128, vc,
                                  None) == L.TQ_EALIGN
    assert lib.tq_compress_values(ctypes.byref(vf), ctypes.c_void_p(0x1000), 1, 1, 1, 8, 0, 0, 132, vc,
                                  None) == L.TQ_EALIGN
    # an enum argument outside its enumerators (a C caller may pass any int)
    vf = L.ValFmt(128, 2, 32)
    assert lib.tq_compress_values(ctypes.byref(vf), ctypes.c_void_p(0x1000), 9, 1, 1, 8, 0, 0, 128, vc,
                                  None) == L.TQ_EINVAL
    assert b"dtype" in lib.tq_last_error()
    assert lib.tq_rotation_host(1, 64, -1, dp, dp) == L.TQ_EINVAL
    # T = 0 is a no-op that needs no planes
    assert lib.tq_compress_values(ctypes.byref(vf), None, 1, 1, 1, 0, 0, 0, 128, vc, None) == L.TQ_OK
    ms, n = ctypes.c_double(), ctypes.c_int64()
    assert lib.tq_profile_read(None, ctypes.byref(ms), ctypes.byref(n)) == L.TQ_EINVAL


def test_plane_sizes():
    lib = L.lib()
    kf = _kf(mse_bits=3)
    assert lib.tq_key_plane_bytes(ctypes.byref(kf), 10, 0) == 10 * 48
    assert lib.tq_key_plane_bytes(ctypes.byref(kf), 10, 1) == 10 * 16
    assert lib.tq_key_plane_bytes(ctypes.byref(kf), 10, 2) == 40
    assert lib.tq_key_plane_bytes(ctypes.byref(kf), 10, 3) == 40
    assert lib.tq_key_plane_bytes(ctypes.byref(kf), 10, 4) == 0
    kf7 = _kf(d=256, mse_bits=7, qjl_m=256)
    assert lib.tq_key_plane_bytes(ctypes.byref(kf7), 1, 0) == 224
    vf = L.ValFmt(128, 2, 32)
    assert lib.tq_val_plane_bytes(ctypes.byref(vf), 3, 0) == 96
    assert lib.tq_val_plane_bytes(ctypes.byref(vf), 3, 1) == 3 * 16
    # per-vector totals agree with the oracle's size accounting
    for d, b, g, vb in [(128, 2, 32, 2), (128, 3, 64, 2), (256, 7, 32, 4)]:
        kf = _kf(d=d, mse_bits=b, qjl_m=d)
        vf = L.ValFmt(d, vb, g)
        kb = sum(lib.tq_key_plane_bytes(ctypes.byref(kf), 1, p) for p in range(4))
        vbb = sum(lib.tq_val_plane_bytes(ctypes.byref(vf), 1, p) for p in range(2))
        assert kb == O.key_bytes_per_vector(d, b, d)
        assert vbb == O.value_bytes_per_vector(d, vb, g)


def test_first_stage_format_sizes_and_checks():
    """qjl_m = 0: no signs and no rnorm plane; qjl_m other than 0 or d is refused."""
    lib = L.lib()
    for d, b in [(64, 3), (128, 2), (256, 7)]:
        kf = _kf(d=d, mse_bits=b, qjl_m=0)
        sizes = [lib.tq_key_plane_bytes(ctypes.byref(kf), 5, p) for p in range(4)]
        assert sizes == [5 * d * b // 8, 0, 20, 0]
        assert sum(sizes) == 5 * O.key_bytes_per_vector(d, b, 0)
    kc = L.KCache()
    kf = _kf(qjl_m=64)
    assert lib.tq_compress_keys(ctypes.byref(kf), None, 1, 1, 1, 8, 0, 0, 128, kc, None) == L.TQ_EINVAL
    # the format check runs first: no codebook handle
    assert lib.tq_dequantize_keys(ctypes.byref(_kf(qjl_m=0)), 1, 1, 8, kc, None, None) == L.TQ_EINVAL
    assert b"codebook" in lib.tq_last_error()
    assert lib.tq_dequantize_keys(None, 1, 1, 8, kc, None, None) == L.TQ_EINVAL


def test_split_policy_and_workspace():
    lib = L.lib()
    kf = _kf()
    # one long sequence with 8 KV heads spreads over many splits
    s = lib.tq_attend_splits(ctypes.byref(kf), 1, 64, 8, 1 << 20)
    assert 64 <= s <= 1024
    # never more splits than tiles: 128 keys on the matrix-core path (d 128 and
    # 256, any key bits), 256 on the general path (d 64 here)
    assert lib.tq_attend_splits(ctypes.byref(kf), 1, 4, 1, 300) == 3
    kf3 = _kf(mse_bits=3)
    assert lib.tq_attend_splits(ctypes.byref(kf3), 1, 4, 1, 300) == 3
    kf64 = _kf(d=64, mse_bits=3, qjl_m=64)
    assert lib.tq_attend_splits(ctypes.byref(kf64), 1, 4, 1, 300) == 2
    assert lib.tq_attend_splits(ctypes.byref(kf), 1, 4, 1, 0) == 1
    assert lib.tq_attend_splits(ctypes.byref(kf), 1, 5, 2, 100) == 0      # Hq % Hkv != 0
    ws = lib.tq_attend_workspace_bytes(ctypes.byref(kf), 2, 8, 2, 1000, 3)
    assert ws >= 2 * 8 * ((128 + 128) + 3 * 2 + 3 * 128) * 4
    # tq_scores: the prepared queries, plus (matrix-core path) the score
    # operands of every unit and the per-query scales, independent of Hkv
    rows = 2 * 8
    steps2 = 2 * (128 * 2 // 128) + 2 * (128 // 128)     # 2-bit codes and signs, per k-block quarter
    need2 = rows * (128 + 128) * 4 + rows * steps2 * 1024 + rows * 16
    assert lib.tq_scores_workspace_bytes(ctypes.byref(kf), 2, 8) >= need2
    need3 = rows * (128 + 128) * 4 + rows * 2 * (128 // 32) * 1024 + rows * 16
    assert lib.tq_scores_workspace_bytes(ctypes.byref(kf3), 2, 8) >= need3
    assert lib.tq_scores_workspace_bytes(None, 2, 8) == 0
    assert lib.tq_scores_workspace_bytes(ctypes.byref(kf), 0, 8) == 0


# ------------------------------------------------------ forced failure paths
def _status(fn, *args):
    try:
        fn(*args)
    except L.TQError as e:
        return e.status, str(e)
    return L.TQ_OK, ""


def test_forced_nonconvergence(monkeypatch):
    """The Lloyd-Max iteration cap (TQ_TEST_HOOK=codebook_iters=N) gives
    TQ_ENOTCONV with the residual in the message, and no handle."""
    monkeypatch.setenv("TQ_TEST_HOOK", "codebook_iters=0")
    st, msg = _status(tq.tq_codebook_host, 128, 3)
    assert st == L.TQ_ENOTCONV and "residual" in msg
    h = ctypes.c_void_p()
    assert L.lib().tq_build_codebook(128, 3, ctypes.byref(h)) == L.TQ_ENOTCONV
    assert h.value is None
    # a few sweeps are not enough either at 7 bits
    monkeypatch.setenv("TQ_TEST_HOOK", "codebook_iters=3")
    assert _status(tq.tq_codebook_host, 256, 7)[0] == L.TQ_ENOTCONV
    # without the hook the same tables converge
    monkeypatch.delenv("TQ_TEST_HOOK")
    c, t = tq.tq_codebook_host(256, 7)
    assert np.abs(c - O.codebook(256, 7)[0]).max() < 1e-12


def test_forced_handle_allocation_failure(monkeypatch):
    """A failed host allocation in handle creation (TQ_TEST_HOOK=host_alloc)
    gives TQ_ENOMEM and no handle; host-only calls are unaffected."""
    monkeypatch.setenv("TQ_TEST_HOOK", "host_alloc")
    lib = L.lib()
    h = ctypes.c_void_p()
    assert lib.tq_build_codebook(128, 2, ctypes.byref(h)) == L.TQ_ENOMEM
    assert h.value is None and b"allocation" in lib.tq_last_error()
    assert lib.tq_make_rotation(7, 128, L.TQ_ROT_DENSE, ctypes.byref(h)) == L.TQ_ENOMEM
    assert h.value is None and b"allocation" in lib.tq_last_error()
    c, _ = tq.tq_codebook_host(128, 2)
    assert c.shape == (4,)


def _gpu_visible():
    import torch
    return torch.cuda.is_available()


def test_device_errors_map_to_ehip():
    """Without a GPU the device uploads of handle creation fail in the HIP
    runtime: TQ_EHIP with the runtime's message, and no handle."""
    if _gpu_visible():
        pytest.skip("a GPU is visible: the uploads succeed")
    lib = L.lib()
    h = ctypes.c_void_p()
    assert lib.tq_build_codebook(128, 2, ctypes.byref(h)) == L.TQ_EHIP
    assert h.value is None and b"device" in lib.tq_last_error()
    assert lib.tq_make_rotation(7, 128, L.TQ_ROT_DENSE, ctypes.byref(h)) == L.TQ_EHIP
    assert h.value is None

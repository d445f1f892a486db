"""HTS_DEBUG=1: the debug checks pass every valid call unchanged and turn a corrupt tile index, a
buffer shorter than the call needs, or host memory in place of device memory into an error
status before anything is launched.  (Without the checks these calls would read or write out of
bounds; they are made here only with the checks on, which refuse them on the host or in the
index-check kernel, whose own reads stay inside the index.)"""
import ctypes
import os

import numpy as np
import pytest
import torch

import tile_gemm_amd as hts
import workloads as wl
from helpers import DEV, say

pytestmark = pytest.mark.gpu


def _hip():
    try:
        return ctypes.CDLL("libamdhip64.so")
    except OSError:
        return ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))


class DeviceBuffer:
    """Exactly `nbytes` of device memory from hipMalloc (its allocation range is its size)."""

    def __init__(self, nbytes):
        self.hip = _hip()
        self.ptr = ctypes.c_void_p()
        assert self.hip.hipMalloc(ctypes.byref(self.ptr), ctypes.c_size_t(nbytes)) == 0
        assert self.hip.hipMemset(self.ptr, 0, ctypes.c_size_t(nbytes)) == 0
        self.nbytes = nbytes

    def free(self):
        torch.cuda.synchronize()
        self.hip.hipFree(self.ptr)


def _case(N=1024, K=2048, M=600, seed=3):
    g = np.random.default_rng(seed)
    W = hts.tensor_from_bits(wl.gaussian_bits((N, K), 0.02, "bf16", g), "bf16", DEV)
    X = hts.tensor_from_bits(wl.gaussian_bits((M, K), 1.0, "bf16", g), "bf16", DEV)
    m = (g.random((N // 128) * (K // 128)) < 0.5).astype(np.uint8)
    return W, X, m


@pytest.fixture
def debug(monkeypatch):
    monkeypatch.setenv("HTS_DEBUG", "1")
    yield
    monkeypatch.delenv("HTS_DEBUG", raising=False)


def test_valid_calls_are_unchanged(monkeypatch):
    W, X, m = _case()
    results = {}
    for mode in ("0", "1"):
        monkeypatch.setenv("HTS_DEBUG", mode)
        pw = hts.pack(W, m, 128, 128)
        Wu = hts.unpack(pw)
        out = [pw.values.clone(), pw.meta.clone()]
        for M in (1, 40, 600):
            out.append(hts.gemm(X[:M], pw, out_dtype=torch.float32))
        out.append(hts.dense_gemm(X, W, out_dtype=torch.float32))
        out.append(Wu)
        torch.cuda.synchronize()
        results[mode] = out
    for a, b in zip(results["0"], results["1"]):
        assert torch.equal(a, b)


def test_corrupt_index_is_refused(debug):
    W, X, m = _case()
    pw = hts.pack(W, m, 128, 128)
    Y = torch.empty((X.shape[0], W.shape[0]), dtype=torch.float32, device=DEV)
    for what, t, col, delta in (("type", 3, 2, 7), ("val_off", 5, 0, 8), ("reserved", 0, 3, 1)):
        bad = pw.index.clone()
        bad[t, col] += delta
        say(f"[debug] corrupt {what} of record {t}")
        with pytest.raises(hts.HTSError) as e:
            hts.hts_gemm(pw.desc, bad, pw.values, pw.meta, X, Y)
        assert e.value.status == 5 and f"first: record {t}" in str(e.value), str(e.value)
        with pytest.raises(hts.HTSError) as e:
            hts.hts_unpack(pw.desc, bad, pw.values, pw.meta, torch.empty_like(W))
        assert e.value.status == 5
    # the intact index still runs, with the same result as without the checks (same path: no
    # workspace, so no split over K)
    hts.hts_gemm(pw.desc, pw.index, pw.values, pw.meta, X, Y)
    torch.cuda.synchronize()
    os.environ["HTS_DEBUG"] = "0"
    Y0 = torch.empty_like(Y)
    hts.hts_gemm(pw.desc, pw.index, pw.values, pw.meta, X, Y0)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y0)


def _raw_gemm(pw, M, X_ptr, ldx, Y_ptr, ldy, values_ptr=None):
    L = hts.lib()
    return L.hts_gemm(ctypes.byref(pw.desc), pw.index.data_ptr(), values_ptr or pw.values.data_ptr(),
                      pw.meta.data_ptr(), M, X_ptr, ldx, Y_ptr, ldy, hts.HTS_F32, None, 0,
                      torch.cuda.current_stream().cuda_stream)


def test_short_buffers_are_refused(debug):
    N, K, M = 4096, 4096, 1024
    W, X, m = _case(N, K, M)
    pw = hts.pack(W, m, 128, 128)
    torch.cuda.synchronize()
    need_y, need_x = M * N * 4, M * K * 2
    Yshort, Xshort = DeviceBuffer(need_y // 2), DeviceBuffer(need_x // 2)
    Vshort = DeviceBuffer(int(pw.sizes["values_bytes"]) // 2)
    Yfull = torch.empty((M, N), dtype=torch.float32, device=DEV)
    try:
        say("[debug] Y half the size the call needs")
        assert _raw_gemm(pw, M, X.data_ptr(), K, Yshort.ptr.value, N) == 3
        assert "Y needs" in hts.lib().hts_last_error().decode()
        say("[debug] X half the size")
        assert _raw_gemm(pw, M, Xshort.ptr.value, K, Yfull.data_ptr(), N) == 3
        assert "X needs" in hts.lib().hts_last_error().decode()
        say("[debug] values half the size")
        assert _raw_gemm(pw, M, X.data_ptr(), K, Yfull.data_ptr(), N, Vshort.ptr.value) == 3
        assert "values needs" in hts.lib().hts_last_error().decode()
        # the exact sizes pass, with the result of the same call without the checks
        assert _raw_gemm(pw, M, X.data_ptr(), K, Yfull.data_ptr(), N) == 0
        torch.cuda.synchronize()
        os.environ["HTS_DEBUG"] = "0"
        Y0 = torch.empty_like(Yfull)
        assert _raw_gemm(pw, M, X.data_ptr(), K, Y0.data_ptr(), N) == 0
        torch.cuda.synchronize()
        assert torch.equal(Yfull, Y0)
    finally:
        for b in (Yshort, Xshort, Vshort):
            b.free()


def test_host_memory_is_refused(debug):
    W, X, m = _case()
    pw = hts.pack(W, m, 128, 128)
    Xh = X.cpu()   # pageable host memory
    Y = torch.empty((X.shape[0], W.shape[0]), dtype=torch.float32, device=DEV)
    say("[debug] X in host memory")
    assert _raw_gemm(pw, X.shape[0], Xh.data_ptr(), X.shape[1], Y.data_ptr(), W.shape[0]) == 1
    assert "not device memory" in hts.lib().hts_last_error().decode()
    # the error left no stale runtime state: the next call runs
    Y2 = hts.gemm(X, pw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.isfinite(Y2).all()

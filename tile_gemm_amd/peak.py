"""Binding of libhts_peak.so: measured roofline denominators (streaming read bandwidth and
register-operand matrix-core throughput) used beside the published MI355X peaks.  Argument
marshalling and event timing only; the work runs in the library's kernels."""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhts_peak.so")
KINDS = {"bf16_dense": 0, "bf16_sparse24": 1, "fp8_dense": 2, "fp8_sparse24": 3, "fp8_dense_k128": 4}
_SIGS = {
    "hts_peak_stream_read": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int,
                                            ctypes.c_void_p]),
    "hts_peak_mfma": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]),
    "hts_peak_mfma_flops_per_instruction": (ctypes.c_double, [ctypes.c_int]),
    "hts_peak_onchip": (ctypes.c_int, [ctypes.c_int, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_void_p]),
}
ONCHIP = {"l2_to_lds": 0, "l2_to_vgpr": 1, "lds_read": 2}
EXPORTED = tuple(_SIGS)
_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m tile_gemm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def _time(fn, reps: int) -> float:
    """Best of `reps` event-timed runs (seconds), after one untimed run."""
    fn()
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3
        best = t if best is None else min(best, t)
    return best


def stream_read_gbs(nbytes: int = 2 << 30, reps: int = 5, device: str = "cuda:0") -> float:
    """Bandwidth (GB/s) of one streaming read of `nbytes` (far beyond the 256 MB Infinity Cache)."""
    src = torch.ones(nbytes // 4, dtype=torch.int32, device=device)
    sink = torch.zeros(1, dtype=torch.int32, device=device)
    stream = torch.cuda.current_stream().cuda_stream
    best = None
    for blocks in (1024, 2048, 4096):
        t = _time(lambda: _check(lib().hts_peak_stream_read(src.data_ptr(), nbytes, sink.data_ptr(), blocks, stream)),
                  reps)
        best = t if best is None else min(best, t)
    del src
    return nbytes / best / 1e9


def mfma_tflops(kind: str, iters: int = 256, reps: int = 5, device: str = "cuda:0") -> float:
    """Algorithmic TFLOP/s of one matrix-core instruction kind with register operands, all CUs busy
    (8 workgroups of 4 waves per CU)."""
    k = KINDS[kind]
    blocks = 256 * 8
    out = torch.empty(blocks * 256, dtype=torch.float32, device=device)
    stream = torch.cuda.current_stream().cuda_stream
    t = _time(lambda: _check(lib().hts_peak_mfma(k, iters, blocks, out.data_ptr(), stream)), reps)
    per = lib().hts_peak_mfma_flops_per_instruction(k)
    return blocks * 4 * iters * 8 * per / t / 1e12


def onchip_gbs(mode: str, iters: int = 64, reps: int = 5, device: str = "cuda:0") -> float:
    """Chip-wide GB/s of one on-chip path (`ONCHIP`), 4 workgroups of 4 waves per CU, sources in L2."""
    m = ONCHIP[mode]
    nbytes, blocks = 2 << 20, 256 * 4
    src = torch.ones(nbytes // 4, dtype=torch.int32, device=device)
    sink = torch.zeros(1, dtype=torch.int32, device=device)
    stream = torch.cuda.current_stream().cuda_stream
    t = _time(lambda: _check(lib().hts_peak_onchip(m, src.data_ptr(), nbytes, iters, blocks, sink.data_ptr(), stream)),
              reps)
    return blocks * iters * 65536 / t / 1e9


def _check(status: int) -> None:
    if status != 0:
        raise RuntimeError(f"libhts_peak call failed with status {status}")

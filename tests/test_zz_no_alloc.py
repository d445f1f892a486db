"""hts_gemm_noalloc: the hybrid product with its workspace in the library's static device scratch.

Called through the C ABI and compared bit for bit with hts_gemm given a workspace of
hts_gemm_workspace() bytes (same kernels, same split, same summation order), on two calls in a
row, the second with a smaller input: split products (fp32 parts in the scratch), the unpacked
weight of 32-wide tiles, and a streaming-range call that needs no scratch.
"""
import numpy as np
import pytest
import torch

import oracle
import tile_gemm_amd as hts
import workloads as wl
from helpers import DEV, say

pytestmark = pytest.mark.gpu
TOL = 5e-3


def _layer(N, K, bn, bk, seed):
    g = np.random.default_rng(seed)
    W = wl.gaussian_bits((N, K), 0.02, "bf16", g)
    m = (g.random((N // bn) * (K // bk)) < 0.5).astype(np.uint8)
    return W, m, g


def _with_workspace(pw, X, M):
    Y = torch.empty((M, pw.desc.N), dtype=torch.float32, device=DEV)
    nb = hts.hts_gemm_workspace(pw.desc, M)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=DEV)
    hts.hts_gemm(pw.desc, pw.index, pw.values, pw.meta, X, Y, workspace=ws if nb else None)
    return Y, nb


def _noalloc(pw, X, M):
    Y = torch.full((M, pw.desc.N), float("nan"), dtype=torch.float32, device=DEV)
    hts.hts_gemm_noalloc(pw.desc, pw.index, pw.values, pw.meta, X, Y)
    return Y


@pytest.mark.parametrize("case", ["split", "unpacked_32", "streaming"])
def test_noalloc_equals_gemm_with_workspace(case):
    N, K, bn, bk, Ms = {"split": (11008, 4096, 128, 128, (128, 64)),
                        "unpacked_32": (1024, 2048, 32, 32, (300, 100)),
                        "streaming": (1024, 2048, 128, 128, (16, 3))}[case]
    W, m, g = _layer(N, K, bn, bk, {"split": 1, "unpacked_32": 2, "streaming": 3}[case])
    pw = hts.pack(hts.tensor_from_bits(W, "bf16", DEV), m, bn, bk)
    Xall = wl.gaussian_bits((max(Ms), K), 1.0, "bf16", g)
    for M in Ms:            # two calls in a row, the second smaller: the scratch keeps the first's data
        say(f"[noalloc] {case} N={N} K={K} tile={bn}x{bk} M={M}")
        X = hts.tensor_from_bits(np.ascontiguousarray(Xall[:M]), "bf16", DEV)
        Yr, nb = _with_workspace(pw, X, M)
        if case != "streaming":
            assert nb > 0, "this case is meant to use the scratch"
        Yn = _noalloc(pw, X, M)
        torch.cuda.synchronize()
        assert torch.equal(Yn, Yr), f"{case} M={M}: differs from hts_gemm"
        ok, rel = oracle.within_tolerance(Yn.cpu().numpy(), oracle.hybrid_ref(Xall[:M], W, "bf16", m, bn, bk), TOL)
        say(f"    max err / max|ref| = {rel:.3e}")
        assert ok


def test_noalloc_rejects_more_than_its_scratch():
    # 32-wide tiles of the 7B up-projection above the streaming range: the unpacked weight (90 MB)
    # exceeds the 64 MiB scratch; nothing is launched
    desc = hts.make_desc(11008, 4096, 32, 32, torch.bfloat16)
    assert hts.hts_gemm_workspace(desc, 64) > (64 << 20)
    X = torch.zeros((64, 4096), dtype=torch.bfloat16, device=DEV)
    Y = torch.zeros((64, 11008), dtype=torch.float32, device=DEV)
    dummy = torch.zeros(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(hts.HTSError) as e:
        hts.hts_gemm_noalloc(desc, dummy, dummy, dummy, X, Y)
    assert e.value.status == 6

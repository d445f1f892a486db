"""Products captured in a HIP graph and replayed: the streaming kernel with X rows staged through
LDS, the split product (tiled kernel writing parts into a workspace, then the fixed-order sum)
and the unsplit tiled kernel.

Each graph is replayed several times with eager work in between: other products into the same
workspace, and torch kernels on the same stream. Every replay must equal the eager result bit
for bit, since the kernels and their summation order are the same.
"""
import numpy as np
import pytest
import torch

import tile_gemm_amd as hts
import workloads as wl
from helpers import DEV, say

pytestmark = pytest.mark.gpu


def _layer(N, K, dtype, seed):
    g = np.random.default_rng(seed)
    W = wl.gaussian_bits((N, K), 0.02, dtype, g)
    m = (g.random((N // 128) * (K // 128)) < 0.4).astype(np.uint8)
    return g, hts.pack(hts.tensor_from_bits(W, dtype, DEV), m, 128, 128)


@pytest.mark.parametrize("M", [1, 16, 64, 300])
def test_graph_replays_equal_eager(M):
    N, K = 1024, 2048
    g, pw = _layer(N, K, "bf16", 2000 + M)
    X = hts.tensor_from_bits(wl.gaussian_bits((M, K), 1.0, "bf16", g), "bf16", DEV)
    X2 = hts.tensor_from_bits(wl.gaussian_bits((M, K), 1.0, "bf16", g), "bf16", DEV)
    nbytes = hts.hts_gemm_workspace(pw.desc, M)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=DEV)
    say(f"[graph] M={M} workspace={nbytes}")
    Y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    hts.gemm(X, pw, out=Y, workspace=ws)
    torch.cuda.synchronize()
    eager = Y.clone()
    other = hts.gemm(X2, pw, out_dtype=torch.float32, workspace=ws)   # eager result of a second input
    torch.cuda.synchronize()
    other_ref = other.clone()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        hts.gemm(X, pw, out=Y, workspace=ws)          # warm-up on the capture stream
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        hts.gemm(X, pw, out=Y, workspace=ws)
    torch.cuda.synchronize()
    for r in range(4):
        Y.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, eager), f"replay {r} differs from the eager product"
        # eager work between replays: another product through the same workspace, torch kernels
        other.zero_()
        hts.gemm(X2, pw, out=other, workspace=ws)
        junk = (X2.float() * 2.0).sum()
        torch.cuda.synchronize()
        assert torch.equal(other, other_ref)
        assert torch.isfinite(junk)

"""GPU parity of hts_gemm_silu_mul: Y = silu(G) * (X . mask(W)^T), the hybrid product with the
gated-MLP step in its output stage, against the oracle's gated step on the unrounded product.

Every product path is covered: the streaming kernel (one and two groups of X rows, 8-bit weights,
32-wide tiles), the tiled kernel unsplit and split (the gate is then applied by the sum of the
parts), and the unpack + dense path of 32-wide tiles above the streaming range.  Also: f32 and
16-bit outputs, G given in place of Y, strided G, and repeat calls equal bit for bit.
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
TD = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def _case(M, dtype, bn, bk, seed, out="bf16"):
    g = np.random.default_rng(seed)
    N, K = 512, 1536
    W = wl.gaussian_bits((N, K), 1.0 if dtype == "fp8" else 0.02, dtype, g)
    X = wl.gaussian_bits((M, K), 1.0, dtype, g)
    m = (g.random((N // bn) * (K // bk)) < 0.5).astype(np.uint8)
    if out == "f32":
        Gh = g.standard_normal((M, N), dtype=np.float32) * 2.0
        G = torch.from_numpy(Gh).to(DEV)
        G_bits = Gh
    else:
        G_bits = wl.gaussian_bits((M, N), 2.0, out, g)
        G = hts.tensor_from_bits(G_bits, out, DEV)
    pw = hts.pack(hts.tensor_from_bits(W, dtype, DEV), m, bn, bk)
    Xt = hts.tensor_from_bits(X, dtype, DEV)
    ref = oracle.gated_ref(G_bits, oracle.hybrid_ref(X, W, dtype, m, bn, bk), out)
    return pw, Xt, G, ref


def _got(Y, out):
    return Y.cpu().numpy().astype(np.float64) if out == "f32" else oracle.widen_f64(hts.bits_from_tensor(Y), out)


CASES = [(1, "bf16", 128, 128, "bf16"), (16, "bf16", 128, 128, "bf16"), (24, "f16", 128, 128, "f16"),
         (100, "bf16", 128, 128, "bf16"), (300, "bf16", 128, 128, "f32"), (40, "f16", 64, 64, "f16"),
         (8, "bf16", 32, 32, "bf16"), (40, "bf16", 32, 32, "bf16"), (1, "fp8", 128, 128, "bf16"),
         (300, "fp8", 128, 128, "f32"), (300, "bf16", 64, 64, "f32"), (130, "f16", 64, 128, "f16")]


@pytest.mark.parametrize("M,dtype,bn,bk,out", CASES, ids=lambda v: str(v))
def test_gated_product(M, dtype, bn, bk, out):
    say(f"[gated] M={M} {dtype} tile={bn}x{bk} out={out}")
    pw, Xt, G, ref = _case(M, dtype, bn, bk, 7000 + M + bn, out)
    Y = hts.gemm_silu_mul(Xt, pw, G)
    Y2 = hts.gemm_silu_mul(Xt, pw, G)
    torch.cuda.synchronize()
    ok, rel = oracle.within_tolerance(_got(Y, out), ref, TOL)
    say(f"    max err / max|ref| = {rel:.3e}")
    assert ok, f"relative error {rel:.3e}"
    assert torch.equal(Y, Y2)


@pytest.mark.parametrize("M", [16, 100, 300])
def test_gated_in_place_and_strided(M):
    # G passed as the output (each element read, then written, by one thread), and a strided G
    pw, Xt, G, ref = _case(M, "bf16", 128, 128, 7100 + M)
    Gs = torch.zeros((M, pw.N + 64), dtype=torch.bfloat16, device=DEV)
    Gs[:, :pw.N] = G
    Y = hts.gemm_silu_mul(Xt, pw, Gs[:, :pw.N])
    Gi = G.clone()
    hts.gemm_silu_mul(Xt, pw, Gi, out=Gi)
    torch.cuda.synchronize()
    for what, got in (("strided G", Y), ("in place", Gi)):
        ok, rel = oracle.within_tolerance(_got(got, "bf16"), ref, TOL)
        assert ok, f"{what}: {rel:.3e}"
    assert torch.equal(Y, Gi)

"""The tiled kernel's 128 x 192 blocks (taken when they need fewer rounds of workgroups than
128 x 128 ones, e.g. the 7B up-projection at M = 2048), forced with HTS_PREFILL_BLOCK_M=192 on
small layers: ragged M (blocks ending inside, at and past M), products split over K into the
workspace and unsplit, edge maps, both sparse-tile paths, 16-bit outputs, 8-bit data, the gated
output stage and the dense product.  Acceptance as everywhere: max|Y - Y_ref| <= 5e-3 * max|Y_ref|."""
import numpy as np
import pytest
import torch

import oracle
import tile_gemm_amd as hts
import workloads as wl
from helpers import DEV, say

pytestmark = pytest.mark.gpu
TOL = 5e-3
TD = {"bf16": torch.bfloat16, "f16": torch.float16}


@pytest.fixture
def block192(monkeypatch):
    monkeypatch.setenv("HTS_PREFILL_BLOCK_M", "192")


def _check(Y, Y_ref, what):
    ok, rel = oracle.within_tolerance(Y, Y_ref, TOL)
    say(f"    {what}: max err / max|ref| = {rel:.3e}")
    assert ok, f"{what}: relative error {rel:.3e} > {TOL}"


def _layer(dtype, kind, seed, N=384, K=1024, Mmax=600):
    g = np.random.default_rng(seed)
    T = (N // 128) * (K // 128)
    m = {"random": g.random(T) < 0.5, "all_dense": np.zeros(T, bool), "all_sparse": np.ones(T, bool)}[kind]
    m = m.astype(np.uint8)
    W = wl.gaussian_bits((N, K), 1.0 if dtype == "fp8" else 0.02, dtype, g)
    X = wl.gaussian_bits((Mmax, K), 1.0, dtype, g)
    return W, X, m


@pytest.mark.parametrize("sparse_path", ["smfmac", "decompress"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_block192_ragged_m(dtype, sparse_path, block192, monkeypatch):
    monkeypatch.setenv("HTS_SPARSE_PATH", sparse_path)
    W, X, m = _layer(dtype, "random", 19200 + (dtype == "f16"))
    Y_ref = oracle.hybrid_ref(X, W, dtype, m, 128, 128)
    pw = hts.pack(hts.tensor_from_bits(W, dtype, DEV), m, 128, 128)
    Xt = hts.tensor_from_bits(X, dtype, DEV)
    for M in (65, 191, 192, 193, 385, 600):
        say(f"[block192] {dtype} {sparse_path} M={M}")
        Y = hts.gemm(Xt[:M], pw, out_dtype=torch.float32)            # split over K when it pays
        Yu = torch.empty_like(Y)
        hts.hts_gemm(pw.desc, pw.index, pw.values, pw.meta, Xt[:M], Yu)  # no workspace: unsplit
        Yh = hts.gemm(Xt[:M], pw)                                     # 16-bit output
        torch.cuda.synchronize()
        _check(Y.cpu().numpy(), Y_ref[:M], f"M={M}")
        _check(Yu.cpu().numpy(), Y_ref[:M], f"M={M} unsplit")
        _check(oracle.widen_f64(hts.bits_from_tensor(Yh), dtype), Y_ref[:M], f"M={M} {dtype} out")


def test_block192_fp8(block192):
    # 8-bit data: one 16x16x128 product per 16 x 16 block and slice, SMFMAC 16x16x128 for 2:4 groups
    W, X, m = _layer("fp8", "random", 19250)
    Y_ref = oracle.hybrid_ref(X, W, "fp8", m, 128, 128)
    pw = hts.pack(hts.tensor_from_bits(W, "fp8", DEV), m, 128, 128)
    Xt = hts.tensor_from_bits(X, "fp8", DEV)
    Wt = hts.tensor_from_bits(W, "fp8", DEV)
    for M in (65, 193, 600):
        say(f"[block192] fp8 M={M}")
        Y = hts.gemm(Xt[:M], pw, out_dtype=torch.float32)
        Yu = torch.empty_like(Y)
        hts.hts_gemm(pw.desc, pw.index, pw.values, pw.meta, Xt[:M], Yu)
        Yd = hts.dense_gemm(Xt[:M], Wt, out_dtype=torch.float32)
        torch.cuda.synchronize()
        _check(Y.cpu().numpy(), Y_ref[:M], f"fp8 M={M}")
        _check(Yu.cpu().numpy(), Y_ref[:M], f"fp8 M={M} unsplit")
        _check(Yd.cpu().numpy(), oracle.gemm_ref(X[:M], W, "fp8"), f"fp8 dense M={M}")


@pytest.mark.parametrize("kind", ["all_dense", "all_sparse"])
def test_block192_edge_maps(kind, block192):
    W, X, m = _layer("bf16", kind, 19210 + len(kind))
    pw = hts.pack(hts.tensor_from_bits(W, "bf16", DEV), m, 128, 128)
    Xt = hts.tensor_from_bits(X, "bf16", DEV)
    say(f"[block192] {kind} M=600")
    Y = hts.gemm(Xt, pw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _check(Y.cpu().numpy(), oracle.hybrid_ref(X, W, "bf16", m, 128, 128), kind)
    if kind == "all_dense":   # p = 0: the hybrid product equals the same-library dense product
        Yd = hts.dense_gemm(Xt, hts.tensor_from_bits(W, "bf16", DEV), out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(Y, Yd)


@pytest.mark.parametrize("M", [100, 193, 600])
def test_block192_dense_product(M, block192):
    g = np.random.default_rng(19220 + M)
    W = wl.gaussian_bits((256, 1536), 0.02, "f16", g)
    X = wl.gaussian_bits((M, 1536), 1.0, "f16", g)
    say(f"[block192] dense M={M}")
    Y = hts.dense_gemm(hts.tensor_from_bits(X, "f16", DEV), hts.tensor_from_bits(W, "f16", DEV),
                       out_dtype=torch.float32)
    torch.cuda.synchronize()
    _check(Y.cpu().numpy(), oracle.gemm_ref(X, W, "f16"), f"dense M={M}")


@pytest.mark.parametrize("M", [150, 450])
def test_block192_gated(M, block192):
    g = np.random.default_rng(19230 + M)
    W, X, m = _layer("bf16", "random", 19240 + M, N=512, K=1536, Mmax=M)
    G_bits = wl.gaussian_bits((M, 512), 2.0, "bf16", g)
    pw = hts.pack(hts.tensor_from_bits(W, "bf16", DEV), m, 128, 128)
    say(f"[block192] gated M={M}")
    Y = hts.gemm_silu_mul(hts.tensor_from_bits(X, "bf16", DEV), pw, hts.tensor_from_bits(G_bits, "bf16", DEV))
    torch.cuda.synchronize()
    ref = oracle.gated_ref(G_bits, oracle.hybrid_ref(X, W, "bf16", m, 128, 128), "bf16")
    _check(oracle.widen_f64(hts.bits_from_tensor(Y), "bf16"), ref, f"gated M={M}")

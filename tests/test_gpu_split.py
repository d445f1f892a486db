"""GPU parity of split products: with at most 256 output blocks the tiled kernel splits the slices
of every tile row over several workgroups and sums their fp32 parts in a fixed order.

The checks cover:
- split counts chosen by the library and forced (HTS_PREFILL_SPLIT);
- ragged M, and parts that cross the dense / 2:4 boundary of the ordered tile list;
- parts that start past the first 64 list entries (86 tile columns of the 7B down-projection);
- 8-bit weights, 64x64 tiles, the dense product, and the unpack path of 32-wide tiles;
- a workspace too small for the parts, which runs the product unsplit;
- every chunk size of the dense-first ordered tile list (HTS_PREFILL_CHUNK).

Results must be within 5e-3 * max|Y_ref| of the oracle and identical from call to call.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import tile_gemm_amd as hts
import workloads as wl
from helpers import DEV, say

pytestmark = pytest.mark.gpu
TOL = 5e-3


def _check(Y, Y_ref, what):
    ok, rel = oracle.within_tolerance(Y, Y_ref, TOL)
    say(f"    {what}: max err / max|ref| = {rel:.3e}")
    assert ok, f"{what}: relative error {rel:.3e} > {TOL}"


def _layer(N, K, dtype, p, seed, bn=128, bk=128, w_sigma=None):
    g = np.random.default_rng(seed)
    W = wl.gaussian_bits((N, K), (1.0 if dtype == "fp8" else 0.02) if w_sigma is None else w_sigma, dtype, g)
    T = (N // bn) * (K // bk)
    m = (g.random(T) < p).astype(np.uint8)
    return W, m, g


@pytest.mark.parametrize("split", ["auto", "2", "3", "5", "7", "16"])
@pytest.mark.parametrize("M", [33, 100, 130])
def test_split_forced_counts(split, M, monkeypatch):
    if split != "auto":
        monkeypatch.setenv("HTS_PREFILL_SPLIT", split)
    N, K = 384, 2048
    W, m, g = _layer(N, K, "bf16", 0.5, zlib.crc32(f"split{M}".encode()))
    X = wl.gaussian_bits((M, K), 1.0, "bf16", g)
    say(f"[split-forced] split={split} M={M}")
    pw = hts.pack(hts.tensor_from_bits(W, "bf16", DEV), m, 128, 128)
    Xt = hts.tensor_from_bits(X, "bf16", DEV)
    Y = hts.gemm(Xt, pw, out_dtype=torch.float32)
    Y2 = hts.gemm(Xt, pw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _check(Y.cpu().numpy(), oracle.hybrid_ref(X, W, "bf16", m, 128, 128), f"split={split} M={M}")
    assert torch.equal(Y, Y2)


@pytest.mark.parametrize("kind", ["all_dense", "all_sparse", "one_sparse", "mixed"])
def test_split_list_boundaries(kind, monkeypatch):
    # 16 tile columns, 32 slices over 3 parts: the dense / 2:4 boundary of the ordered list falls
    # inside a part (or nowhere)
    monkeypatch.setenv("HTS_PREFILL_SPLIT", "3")
    N, K, M = 256, 2048, 70
    W, _, g = _layer(N, K, "f16", 0.0, zlib.crc32(kind.encode()))
    T = (N // 128) * (K // 128)
    m = {"all_dense": np.zeros(T, np.uint8), "all_sparse": np.ones(T, np.uint8),
         "one_sparse": (np.arange(T) == 5).astype(np.uint8),
         "mixed": (g.random(T) < 0.4).astype(np.uint8)}[kind]
    X = wl.gaussian_bits((M, K), 1.0, "f16", g)
    say(f"[split-boundary] {kind}")
    pw = hts.pack(hts.tensor_from_bits(W, "f16", DEV), m, 128, 128)
    for od in (torch.float32, torch.float16):
        Y = hts.gemm(hts.tensor_from_bits(X, "f16", DEV), pw, out_dtype=od)
        torch.cuda.synchronize()
        _check(Y.float().cpu().numpy(), oracle.hybrid_ref(X, W, "f16", m, 128, 128), f"{kind} out={od}")


@pytest.mark.parametrize("M", [33, 128, 256])
def test_split_7b_down_projection(M):
    # 4096 x 11008: 86 tile columns, 172 slices; at 32 < M <= 256 the 32-64 blocks split 8 ways and
    # later parts start past list entry 64
    c = wl.config("7b_block")
    L = next(x for x in c.layers if x.name == "down")
    W = wl.weight_bits(c, L)
    T = (L.N // 128) * (L.K // 128)
    m = wl.exact_map(T, T // 2, wl.rng(c.cfg_id, L.layer_id, wl.TAG_MAP, (99,)))
    X = wl.activation_bits(c, L, M)
    say(f"[split-down] M={M} workspace={hts.hts_gemm_workspace(hts.make_desc(L.N, L.K, 128, 128, torch.bfloat16), M)}")
    pw = hts.pack(hts.tensor_from_bits(W, "bf16", DEV), m, 128, 128)
    Y = hts.gemm(hts.tensor_from_bits(np.ascontiguousarray(X), "bf16", DEV), pw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = np.arange(M)
    _check(Y.cpu().numpy()[rows], oracle.gemm_ref(X[rows], oracle.masked_weights(W, "bf16", m, 128, 128), "bf16"),
           f"down M={M}")


@pytest.mark.parametrize("M", [33, 64, 200])
def test_split_7b_up_projection(M):
    c = wl.config("7b_up")
    L = c.layers[0]
    W = wl.weight_bits(c, L)
    m = wl.tile_map(c, L)
    X = wl.activation_bits(c, L, 2048)[:M]
    desc = hts.make_desc(L.N, L.K, 128, 128, torch.bfloat16)
    nbytes = hts.hts_gemm_workspace(desc, M)
    say(f"[split-7b-up] M={M} workspace={nbytes}")
    assert nbytes > 0
    pw = hts.pack(hts.tensor_from_bits(W, "bf16", DEV), m, 128, 128)
    Xt = hts.tensor_from_bits(np.ascontiguousarray(X), "bf16", DEV)
    Y = hts.gemm(Xt, pw, out_dtype=torch.float32)
    # a workspace 256 bytes short of the parts: the product runs unsplit
    small = torch.empty(nbytes - 256, dtype=torch.uint8, device=DEV)
    Yu = hts.gemm(Xt, pw, out_dtype=torch.float32, workspace=small)
    torch.cuda.synchronize()
    rows = np.arange(M)
    Y_ref = oracle.gemm_ref(X[rows], oracle.masked_weights(W, "bf16", m, 128, 128), "bf16")
    _check(Y.cpu().numpy()[rows], Y_ref, f"split M={M}")
    _check(Yu.cpu().numpy()[rows], Y_ref, f"unsplit M={M}")


@pytest.mark.parametrize("M", [33, 100])
def test_split_fp8(M):
    N, K = 512, 1024
    W, m, g = _layer(N, K, "fp8", 0.5, 900 + M)
    X = wl.gaussian_bits((M, K), 1.0, "fp8", g)
    say(f"[split-fp8] M={M}")
    pw = hts.pack(hts.tensor_from_bits(W, "fp8", DEV), m, 128, 128)
    Y = hts.gemm(hts.tensor_from_bits(X, "fp8", DEV), pw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _check(Y.cpu().numpy(), oracle.hybrid_ref(X, W, "fp8", m, 128, 128), f"fp8 M={M}")


@pytest.mark.parametrize("M", [17, 150])
def test_split_64_tiles(M):
    N, K = 320, 1536
    W, m, g = _layer(N, K, "bf16", 0.5, 1000 + M, bn=64, bk=64)
    X = wl.gaussian_bits((M, K), 1.0, "bf16", g)
    say(f"[split-64] M={M}")
    pw = hts.pack(hts.tensor_from_bits(W, "bf16", DEV), m, 64, 64)
    Y = hts.gemm(hts.tensor_from_bits(X, "bf16", DEV), pw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _check(Y.cpu().numpy(), oracle.hybrid_ref(X, W, "bf16", m, 64, 64), f"64x64 M={M}")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("M", [17, 96, 300])
def test_split_dense_product(dtype, M):
    N, K = 640, 2048
    g = np.random.default_rng(1100 + M)
    W = wl.gaussian_bits((N, K), 1.0 if dtype == "fp8" else 0.02, dtype, g)
    X = wl.gaussian_bits((M, K), 1.0, dtype, g)
    nbytes = hts.hts_dense_gemm_workspace(torch.float8_e4m3fn if dtype == "fp8" else torch.bfloat16, M, N, K)
    say(f"[split-dense] {dtype} M={M} workspace={nbytes}")
    Y = hts.dense_gemm(hts.tensor_from_bits(X, dtype, DEV), hts.tensor_from_bits(W, dtype, DEV),
                       out_dtype=torch.float32)
    torch.cuda.synchronize()
    _check(Y.cpu().numpy(), oracle.gemm_ref(X, W, dtype), f"dense {dtype} M={M}")


def test_split_small_tiles_workspace():
    # 32x32 tiles above M = 16: the unpacked weight, then the parts of the split dense product
    N, K, M = 256, 1024, 40
    W, m, g = _layer(N, K, "bf16", 0.5, 1200, bn=32, bk=32)
    X = wl.gaussian_bits((M, K), 1.0, "bf16", g)
    desc = hts.make_desc(N, K, 32, 32, torch.bfloat16)
    nbytes = hts.hts_gemm_workspace(desc, M)
    say(f"[split-small-tiles] workspace={nbytes} (unpacked weight {N * K * 2})")
    assert nbytes > N * K * 2
    pw = hts.pack(hts.tensor_from_bits(W, "bf16", DEV), m, 32, 32)
    Xt = hts.tensor_from_bits(X, "bf16", DEV)
    Y = hts.gemm(Xt, pw, out_dtype=torch.float32)
    Yu = hts.gemm(Xt, pw, out_dtype=torch.float32,
                  workspace=torch.empty(N * K * 2, dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    Y_ref = oracle.hybrid_ref(X, W, "bf16", m, 32, 32)
    _check(Y.cpu().numpy(), Y_ref, "32x32 split")
    _check(Yu.cpu().numpy(), Y_ref, "32x32 unsplit")


@pytest.mark.parametrize("chunk", ["4", "8", "16", "32", "64"])
@pytest.mark.parametrize("M", [100, 300])
def test_chunked_list_orders(chunk, M, monkeypatch):
    # the ordered list is dense-first inside chunks of tile columns; every chunk size gives the
    # same product within tolerance, split parts starting or ending inside a chunk (M=100: 3
    # blocks, 8 parts) or unsplit (M=300, forced), with a last chunk that is only partly filled
    # (K/bk = 44 tile columns)
    monkeypatch.setenv("HTS_PREFILL_CHUNK", chunk)
    if M == 300:
        monkeypatch.setenv("HTS_PREFILL_SPLIT", "1")
    N, K = 384, 44 * 128
    W, m, g = _layer(N, K, "bf16", 0.5, zlib.crc32(f"chunk{chunk}-{M}".encode()))
    X = wl.gaussian_bits((M, K), 1.0, "bf16", g)
    say(f"[chunk] chunk={chunk} M={M}")
    pw = hts.pack(hts.tensor_from_bits(W, "bf16", DEV), m, 128, 128)
    Y = hts.gemm(hts.tensor_from_bits(X, "bf16", DEV), pw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _check(Y.cpu().numpy(), oracle.hybrid_ref(X, W, "bf16", m, 128, 128), f"chunk={chunk} M={M}")


@pytest.mark.parametrize("chunk", ["4", "8", "64"])
def test_chunked_list_64_tiles(chunk, monkeypatch):
    # bk = 64: one 64-wide slice per tile column, the default chunk is 8 tile columns
    monkeypatch.setenv("HTS_PREFILL_CHUNK", chunk)
    N, K, M = 256, 70 * 64, 200
    W, m, g = _layer(N, K, "f16", 0.4, 1300 + int(chunk), bn=64, bk=64)
    X = wl.gaussian_bits((M, K), 1.0, "f16", g)
    say(f"[chunk-64] chunk={chunk}")
    pw = hts.pack(hts.tensor_from_bits(W, "f16", DEV), m, 64, 64)
    Y = hts.gemm(hts.tensor_from_bits(X, "f16", DEV), pw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _check(Y.cpu().numpy(), oracle.hybrid_ref(X, W, "f16", m, 64, 64), f"64x64 chunk={chunk}")

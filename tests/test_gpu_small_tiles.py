"""GPU parity of tiles of 32 rows or 32 columns (the tile-size ablation of the PATCH page):
pack / unpack bit for bit, and the product within 5e-3 * max|Y_ref| on the streaming kernel
(M <= 16; 32-wide tiles expand their 2:4 groups in registers) and, above it, through the
workspace path (unpack, then the same-library dense product).
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
TILES = [(32, 32), (32, 64), (32, 128), (64, 32), (128, 32)]


def _check(Y, Y_ref, what):
    ok, rel = oracle.within_tolerance(Y, Y_ref, TOL)
    say(f"    {what}: max err / max|ref| = {rel:.3e}")
    assert ok, f"{what}: relative error {rel:.3e} > {TOL}"


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_small_tile_pack_unpack(tile, dtype):
    bn, bk = tile
    N, K = 4 * bn * (128 // bn), 3 * 128
    g = np.random.default_rng(zlib.crc32(f"st{tile}{dtype}".encode()))
    choices = np.array([0.0, -0.0, 0.5, -0.5, 1.0, -1.0, 2.0, 3.0], np.float32)
    W = wl.to_bits(choices[g.integers(0, len(choices), (N, K))], dtype)
    W[g.random((N, K)) < 0.02] = np.uint16(0x0001)
    T = (N // bn) * (K // bk)
    say(f"[small-pack] tile={bn}x{bk} {dtype}")
    for m in ((g.random(T) < 0.5).astype(np.uint8), np.ones(T, np.uint8), (np.arange(T) % 3 == 1).astype(np.uint8)):
        vals, meta, idx = oracle.pack(W, dtype, m, bn, bk)
        pw = hts.pack(hts.tensor_from_bits(W, dtype, DEV), m, bn, bk)
        torch.cuda.synchronize()
        assert np.array_equal(hts.bits_from_tensor(pw.values)[: vals.size], vals)
        assert np.array_equal(pw.meta.cpu().numpy().view(np.uint32)[: meta.size], meta)
        assert np.array_equal(pw.index.cpu().numpy().view(np.uint32), idx)
        assert np.array_equal(hts.bits_from_tensor(hts.unpack(pw)), oracle.masked_weights(W, dtype, m, bn, bk))


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("M", [1, 5, 16, 17, 100, 600])
def test_small_tile_gemm(tile, M):
    bn, bk = tile
    N, K = 384, 512
    dtype = "bf16" if (M + bn) % 2 else "f16"
    g = np.random.default_rng(zlib.crc32(f"stg{tile}{M}".encode()))
    W = wl.gaussian_bits((N, K), 0.02, dtype, g)
    X = wl.gaussian_bits((M, K), 1.0, dtype, g)
    T = (N // bn) * (K // bk)
    m = (g.random(T) < 0.5).astype(np.uint8)
    say(f"[small-gemm] tile={bn}x{bk} M={M} {dtype}")
    Y_ref = oracle.hybrid_ref(X, W, dtype, m, bn, bk)
    pw = hts.pack(hts.tensor_from_bits(W, dtype, DEV), m, bn, bk)
    Y = hts.gemm(hts.tensor_from_bits(X, dtype, DEV), pw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _check(Y.cpu().numpy(), Y_ref, f"tile={bn}x{bk} M={M}")


@pytest.mark.parametrize("env", [{}, {"HTS_DECODE_PP": "2"}, {"HTS_DECODE_KSPLIT": "4"}, {"HTS_DECODE_KSPLIT": "16"},
                                 {"HTS_DECODE_PP": "2", "HTS_DECODE_KSPLIT": "4"}])
def test_small_tile_streaming_launch_shapes(env, monkeypatch):
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    N, K, M = 512, 1024, 16
    g = np.random.default_rng(77)
    W = wl.gaussian_bits((N, K), 0.02, "bf16", g)
    X = wl.gaussian_bits((M, K), 1.0, "bf16", g)
    m = (g.random((N // 32) * (K // 32)) < 0.5).astype(np.uint8)
    say(f"[small-shapes] {env}")
    pw = hts.pack(hts.tensor_from_bits(W, "bf16", DEV), m, 32, 32)
    Y = hts.gemm(hts.tensor_from_bits(X, "bf16", DEV), pw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _check(Y.cpu().numpy(), oracle.hybrid_ref(X, W, "bf16", m, 32, 32), f"{env}")


def test_small_tile_explicit_workspace_reused():
    N, K = 256, 384
    g = np.random.default_rng(5)
    W = wl.gaussian_bits((N, K), 0.02, "bf16", g)
    m = (g.random((N // 32) * (K // 32)) < 0.5).astype(np.uint8)
    pw = hts.pack(hts.tensor_from_bits(W, "bf16", DEV), m, 32, 32)
    ws = torch.empty(hts.hts_gemm_workspace(pw.desc, 300), dtype=torch.uint8, device=DEV)
    for M in (300, 40):
        X = wl.gaussian_bits((M, K), 1.0, "bf16", g)
        Y = hts.gemm(hts.tensor_from_bits(X, "bf16", DEV), pw, out_dtype=torch.float32, workspace=ws)
        torch.cuda.synchronize()
        _check(Y.cpu().numpy(), oracle.hybrid_ref(X, W, "bf16", m, 32, 32), f"workspace M={M}")


@pytest.mark.parametrize("M", [1, 16, 2048])
def test_small_tiles_7b_up_shape(M):
    # the 7B up-projection weight with a 32x32 map at the same 25% of tiles 2:4 (sampled rows)
    c = wl.config("7b_up")
    L = c.layers[0]
    W = wl.weight_bits(c, L)
    T = (L.N // 32) * (L.K // 32)
    m = wl.exact_map(T, int(round(0.25 * T)), wl.rng(c.cfg_id, L.layer_id, wl.TAG_MAP, (32,)))
    X = wl.activation_bits(c, L, max(c.Ms))[:M]
    say(f"[small-7b] M={M}")
    pw = hts.pack(hts.tensor_from_bits(W, "bf16", DEV), m, 32, 32)
    Y = hts.gemm(hts.tensor_from_bits(np.ascontiguousarray(X), "bf16", DEV), pw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = np.arange(M)
    _check(Y.cpu().numpy()[rows], oracle.gemm_ref(X[rows], oracle.masked_weights(W, "bf16", m, 32, 32), "bf16"),
           f"7b 32x32 M={M}")

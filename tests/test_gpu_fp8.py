"""GPU parity of the 8-bit (OCP E4M3) variant against the CPU oracle: pack, masked pack and
unpack bit for bit; the hybrid and dense products within 5e-3 * max|Y_ref| across the streaming
(M <= 16) and the tiled kernel, every launch shape of the streaming kernel, edge maps, strides.
(The full-size 7B-shaped 8-bit layer runs in the named-layer tests of test_gpu_pack / test_gpu_gemm.)
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import tile_gemm_amd as hts
import workloads as wl
from helpers import DEV, say, weight, activations, oracle_map, oracle_packed

pytestmark = pytest.mark.gpu
TOL = 5e-3
FP8_TIES = np.array([0.0, -0.0, 0.5, -0.5, 1.0, -1.0, 2.0, 3.0, 448.0, 2.0 ** -9], np.float32)


def _t(bits):
    return hts.tensor_from_bits(bits, "fp8", DEV)


def _check(Y, Y_ref, what):
    ok, rel = oracle.within_tolerance(Y, Y_ref, TOL)
    say(f"    {what}: max err / max|ref| = {rel:.3e}")
    assert ok, f"{what}: relative error {rel:.3e} > {TOL}"


EDGE = {
    "all_dense": lambda T: np.zeros(T, np.uint8),
    "all_sparse": lambda T: np.ones(T, np.uint8),
    "alternate": lambda T: (np.arange(T) % 2).astype(np.uint8),
    "one_sparse": lambda T: (np.arange(T) == 3).astype(np.uint8),
}


@pytest.mark.parametrize("kind", list(EDGE))
@pytest.mark.parametrize("scaled", [False, True])
def test_fp8_pack_edge_maps_and_ties(kind, scaled):
    N, K = 3 * 128, 5 * 128
    g = np.random.default_rng(zlib.crc32(f"fp8{kind}{scaled}".encode()))
    W = wl.to_bits(FP8_TIES[g.integers(0, len(FP8_TIES), (N, K))], "fp8")
    m = EDGE[kind](15)
    cs = np.abs(g.standard_normal(K)).astype(np.float32).round(1) if scaled else None
    say(f"[fp8-pack] {kind} scaled={scaled}")
    vals, meta, idx = oracle.pack(W, "fp8", m, 128, 128, cs)
    pw = hts.pack(_t(W), m, 128, 128, None if cs is None else torch.from_numpy(cs).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(hts.bits_from_tensor(pw.values)[: vals.size], vals)
    assert np.array_equal(pw.meta.cpu().numpy().view(np.uint32)[: meta.size], meta)
    assert np.array_equal(pw.index.cpu().numpy().view(np.uint32), idx)
    assert np.array_equal(hts.bits_from_tensor(hts.unpack(pw)), oracle.masked_weights(W, "fp8", m, 128, 128, cs))


def test_fp8_pack_masked_malformed_and_strided():
    N, K = 256, 512
    g = np.random.default_rng(31)
    W = wl.gaussian_bits((N, K), 1.0, "fp8", g)
    m = (g.random(8) < 0.6).astype(np.uint8)
    for mask in ((g.random((N, K)) < 0.5).astype(np.uint8) * 7, wl.pair_mask(N, K, g)):
        vals, meta, idx, bad = oracle.pack_masked(W, "fp8", m, mask, 128, 128)
        big = torch.zeros((N, K + 32), dtype=torch.uint8, device=DEV)
        big[:, :K] = torch.from_numpy(mask).to(DEV)
        pw, malformed = hts.pack_masked(_t(W), m, big[:, :K], 128, 128)
        torch.cuda.synchronize()
        assert np.array_equal(hts.bits_from_tensor(pw.values)[: vals.size], vals)
        assert np.array_equal(pw.meta.cpu().numpy().view(np.uint32)[: meta.size], meta)
        assert int(malformed.item()) == bad
        assert np.array_equal(hts.bits_from_tensor(hts.unpack(pw)), oracle.masked_weights_from_mask(W, m, mask, 128, 128))


@pytest.mark.parametrize("M", [1, 2, 5, 15, 16, 17, 31, 64, 127, 128, 129, 300])
def test_fp8_gemm_ragged_m(M):
    N, K = 3 * 128, 4 * 128
    g = np.random.default_rng(500 + M)
    W = wl.gaussian_bits((N, K), 1.0, "fp8", g)
    X = wl.gaussian_bits((M, K), 1.0, "fp8", g)
    m = (g.random(12) < 0.5).astype(np.uint8)
    say(f"[fp8-gemm-ragged] M={M}")
    Y_ref = oracle.hybrid_ref(X, W, "fp8", m, 128, 128)
    pw = hts.pack(_t(W), m, 128, 128)
    for od in (torch.float32, torch.bfloat16, torch.float16):
        Y = hts.gemm(_t(X), pw, out_dtype=od)
        torch.cuda.synchronize()
        _check(Y.float().cpu().numpy(), Y_ref, f"M={M} out={od}")


@pytest.mark.parametrize("kind", list(EDGE))
@pytest.mark.parametrize("M", [1, 16, 256])
def test_fp8_gemm_edge_maps(kind, M):
    N, K = 512, 768
    g = np.random.default_rng(zlib.crc32(f"fp8gemm{kind}{M}".encode()))
    W = wl.gaussian_bits((N, K), 1.0, "fp8", g)
    X = wl.gaussian_bits((M, K), 1.0, "fp8", g)
    m = EDGE[kind](24)
    say(f"[fp8-gemm-edge] {kind} M={M}")
    pw = hts.pack(_t(W), m, 128, 128)
    Y = hts.gemm(_t(X), pw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _check(Y.cpu().numpy(), oracle.hybrid_ref(X, W, "fp8", m, 128, 128), kind)
    if kind == "all_dense":   # p = 0: the hybrid product equals the same-library dense product
        Yd = hts.dense_gemm(_t(X), _t(W), out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(Y, Yd)


@pytest.mark.parametrize("M", [1, 5, 16, 200, 2048])
def test_fp8_dense_gemm(M):
    N, K = 1024, 1536
    g = np.random.default_rng(700 + M)
    W = wl.gaussian_bits((N, K), 1.0, "fp8", g)
    X = wl.gaussian_bits((M, K), 1.0, "fp8", g)
    say(f"[fp8-dense] M={M}")
    rows = np.arange(M)
    Y = hts.dense_gemm(_t(X), _t(W), out_dtype=torch.float32)
    torch.cuda.synchronize()
    _check(Y.cpu().numpy()[rows], oracle.gemm_ref(X[rows], W, "fp8"), "dense")


def test_fp8_strided_x_and_y():
    N, K, M = 256, 512, 40
    g = np.random.default_rng(8)
    W = wl.gaussian_bits((N, K), 1.0, "fp8", g)
    Xbig = wl.gaussian_bits((M, K + 32), 1.0, "fp8", g)
    m = np.array([1, 0, 1, 1, 0, 0, 1, 0], np.uint8)
    Y_ref = oracle.hybrid_ref(np.ascontiguousarray(Xbig[:, :K]), W, "fp8", m, 128, 128)
    pw = hts.pack(_t(W), m, 128, 128)
    for Mx in (M, 9):   # tiled and streaming kernels
        Ybig = torch.full((Mx, N + 32), 7.0, dtype=torch.float32, device=DEV)
        hts.gemm(_t(Xbig)[:Mx, :K], pw, out=Ybig[:, :N])
        torch.cuda.synchronize()
        _check(Ybig[:, :N].cpu().numpy(), Y_ref[:Mx], f"strided M={Mx}")
        assert torch.all(Ybig[:, N:] == 7.0)


@pytest.mark.parametrize("env", [{}, {"HTS_DECODE_PP": "2"}, {"HTS_DECODE_KSPLIT": "4"},
                                 {"HTS_DECODE_KSPLIT": "16"}, {"HTS_DECODE_NT": "4"},
                                 {"HTS_DECODE_PP": "2", "HTS_DECODE_KSPLIT": "4"},
                                 {"HTS_DECODE_XT_MIN_M": "17"},
                                 {"HTS_DECODE_NT": "4", "HTS_DECODE_PP": "2", "HTS_DECODE_XT_MIN_M": "1"}])
@pytest.mark.parametrize("M", [16, 32])
def test_fp8_streaming_launch_shapes(env, M, monkeypatch):
    # every launch shape of the 8-bit streaming kernel, X loaded in the operand layout or as whole
    # rows through LDS, on the 7B-shaped layer; M = 32: two groups of 16 X rows per weight fragment
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    c = wl.config("7b_up_fp8")
    L = c.layers[0]
    say(f"[fp8-shapes] {env} M={M}")
    vals, meta, idx, Wm = oracle_packed(c.cfg_id, L.name)
    pw = hts.pack(_t(weight(c.cfg_id, L.name)), oracle_map(c.cfg_id, L.name), 128, 128)
    X = activations(c.cfg_id, L.name)[:M]
    Y = hts.gemm(_t(np.ascontiguousarray(X)), pw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _check(Y.cpu().numpy(), oracle.gemm_ref(X, Wm, "fp8"), f"{env}")


@pytest.mark.parametrize("M", [1, 2048])
def test_fp8_deterministic(M):
    c = wl.config("7b_up_fp8")
    L = c.layers[0]
    pw = hts.pack(_t(weight(c.cfg_id, L.name)), oracle_map(c.cfg_id, L.name), 128, 128)
    X = _t(np.ascontiguousarray(activations(c.cfg_id, L.name)[:M]))
    Y1 = hts.gemm(X, pw, out_dtype=torch.float32)
    Y2 = hts.gemm(X, pw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2)

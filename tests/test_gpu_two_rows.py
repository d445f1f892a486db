"""The tiled kernel on 64-row tiles: each 128-row block covers two 64-row tile rows, walks K in
tile-column order and feeds each wave's row to the matrix cores by its own tile's type.  Cases:
an odd number of tile rows (the last block has one row), maps whose two rows differ slice by
slice (alternating and checkerboard types, one row all 2:4), both block heights (64 and 128 X
rows; a forced 192 runs as 128), products split over K with parts that start past the first 64
tile columns, both sparse-tile paths, 64 x 64 and 64 x 128 tiles, 16-bit outputs, and the
one-row form (HTS_PREFILL_TWO_ROWS=0) on the same inputs.  Acceptance as everywhere:
max|Y - Y_ref| <= 5e-3 * max|Y_ref|."""
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


def _map(kind, rows, cols, g):
    if kind == "random":
        m = g.random((rows, cols)) < 0.5
    elif kind == "all_dense":
        m = np.zeros((rows, cols), bool)
    elif kind == "all_sparse":
        m = np.ones((rows, cols), bool)
    elif kind == "alternate_rows":          # even tile rows dense, odd rows 2:4
        m = np.zeros((rows, cols), bool)
        m[1::2] = True
    elif kind == "checker":                 # the two rows of a block differ in every column
        m = (np.add.outer(np.arange(rows), np.arange(cols)) % 2).astype(bool)
    else:
        raise ValueError(kind)
    return m.astype(np.uint8).ravel()


def _layer(dtype, bn, bk, N, K, kind, seed, Mmax):
    g = np.random.default_rng(seed)
    m = _map(kind, N // bn, K // bk, g)
    W = wl.gaussian_bits((N, K), 0.02, dtype, g)
    X = wl.gaussian_bits((Mmax, K), 1.0, dtype, g)
    return W, X, m


def _run_all(Xt, pw, M, Y_ref, dtype, what):
    Y = hts.gemm(Xt[:M], pw, out_dtype=torch.float32)             # split over K when it pays
    Yu = torch.empty_like(Y)
    hts.hts_gemm(pw.desc, pw.index, pw.values, pw.meta, Xt[:M], Yu)   # no workspace: unsplit
    Yh = hts.gemm(Xt[:M], pw)                                      # 16-bit output
    torch.cuda.synchronize()
    _check(Y.cpu().numpy(), Y_ref[:M], f"{what} M={M}")
    _check(Yu.cpu().numpy(), Y_ref[:M], f"{what} M={M} unsplit")
    _check(oracle.widen_f64(hts.bits_from_tensor(Yh), dtype), Y_ref[:M], f"{what} M={M} {dtype} out")


@pytest.mark.parametrize("sparse_path", ["smfmac", "decompress"])
@pytest.mark.parametrize("tile", [(64, 64), (64, 128)])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_two_rows_ragged(dtype, tile, sparse_path, monkeypatch):
    monkeypatch.setenv("HTS_SPARSE_PATH", sparse_path)
    bn, bk = tile
    N, K = 5 * 64, 1024                  # five tile rows: the third block has one
    W, X, m = _layer(dtype, bn, bk, N, K, "random", 6400 + bk + (dtype == "f16"), 600)
    Y_ref = oracle.hybrid_ref(X, W, dtype, m, bn, bk)
    pw = hts.pack(hts.tensor_from_bits(W, dtype, DEV), m, bn, bk)
    Xt = hts.tensor_from_bits(X, dtype, DEV)
    for M in (17, 64, 65, 129, 193, 600):
        say(f"[two-rows] {dtype} {bn}x{bk} {sparse_path} M={M}")
        _run_all(Xt, pw, M, Y_ref, dtype, f"{bn}x{bk}")


@pytest.mark.parametrize("kind", ["all_dense", "all_sparse", "alternate_rows", "checker"])
@pytest.mark.parametrize("tile", [(64, 64), (64, 128)])
def test_two_rows_edge_maps(kind, tile):
    bn, bk = tile
    N, K = 7 * 64, 768
    W, X, m = _layer("bf16", bn, bk, N, K, kind, 6500 + bk, 300)
    Y_ref = oracle.hybrid_ref(X, W, "bf16", m, bn, bk)
    pw = hts.pack(hts.tensor_from_bits(W, "bf16", DEV), m, bn, bk)
    Xt = hts.tensor_from_bits(X, "bf16", DEV)
    for M in (40, 300):
        say(f"[two-rows-map] {kind} {bn}x{bk} M={M}")
        _run_all(Xt, pw, M, Y_ref, "bf16", f"{kind} {bn}x{bk}")


@pytest.mark.parametrize("block_m", ["64", "128", "192"])
def test_two_rows_block_heights(block_m, monkeypatch):
    monkeypatch.setenv("HTS_PREFILL_BLOCK_M", block_m)
    N, K = 6 * 64, 1024
    W, X, m = _layer("f16", 64, 64, N, K, "random", 6600 + int(block_m), 450)
    Y_ref = oracle.hybrid_ref(X, W, "f16", m, 64, 64)
    pw = hts.pack(hts.tensor_from_bits(W, "f16", DEV), m, 64, 64)
    Xt = hts.tensor_from_bits(X, "f16", DEV)
    for M in (33, 191, 193, 450):
        say(f"[two-rows-bm] block_m={block_m} M={M}")
        _run_all(Xt, pw, M, Y_ref, "f16", f"block_m={block_m}")


@pytest.mark.parametrize("split", ["2", "3", "5", "8"])
def test_two_rows_split_past_64_columns(split, monkeypatch):
    # 70 tile columns of 64: parts from the second one on start past list entry 64
    monkeypatch.setenv("HTS_PREFILL_SPLIT", split)
    N, K, M = 3 * 64, 70 * 64, 200
    W, X, m = _layer("bf16", 64, 64, N, K, "random", 6700 + int(split), M)
    Y_ref = oracle.hybrid_ref(X, W, "bf16", m, 64, 64)
    pw = hts.pack(hts.tensor_from_bits(W, "bf16", DEV), m, 64, 64)
    Xt = hts.tensor_from_bits(X, "bf16", DEV)
    say(f"[two-rows-split] parts={split}")
    Y = hts.gemm(Xt, pw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _check(Y.cpu().numpy(), Y_ref, f"parts={split}")


@pytest.mark.parametrize("two", ["0", "1"])
def test_two_rows_and_one_row_forms(two, monkeypatch):
    # the one-row form (64-row blocks) stays available and both meet the bar on the same inputs
    monkeypatch.setenv("HTS_PREFILL_TWO_ROWS", two)
    N, K = 9 * 64, 2048
    W, X, m = _layer("bf16", 64, 64, N, K, "random", 6800, 700)
    Y_ref = oracle.hybrid_ref(X, W, "bf16", m, 64, 64)
    pw = hts.pack(hts.tensor_from_bits(W, "bf16", DEV), m, 64, 64)
    Xt = hts.tensor_from_bits(X, "bf16", DEV)
    for M in (100, 700):
        say(f"[two-rows-form] two={two} M={M}")
        _run_all(Xt, pw, M, Y_ref, "bf16", f"two={two}")


@pytest.mark.parametrize("bk,dtype", [(64, "bf16"), (128, "f16")])
def test_two_rows_at_the_column_limit(bk, dtype):
    # 256 tile columns, the most a tile row of the tiled kernel holds: both rows' list registers
    # shift through all four 64-entry blocks; three tile rows, so the second block has one
    N, K, Mmax = 3 * 64, bk * 256, 300
    W, X, m = _layer(dtype, 64, bk, N, K, "random", 6900 + bk, Mmax)
    Y_ref = oracle.hybrid_ref(X, W, dtype, m, 64, bk)
    pw = hts.pack(hts.tensor_from_bits(W, dtype, DEV), m, 64, bk)
    Xt = hts.tensor_from_bits(X, dtype, DEV)
    for M in (48, Mmax):
        say(f"[two-rows-limit] Tk=256 bk={bk} {dtype} M={M}")
        _run_all(Xt, pw, M, Y_ref, dtype, f"Tk=256 bk={bk}")


@pytest.mark.parametrize("M", [64, 300])
def test_two_rows_gated_unsplit_and_split(M):
    # the gated output stage: applied in the kernel's epilogue (no workspace: unsplit) and in the
    # sum of the parts (workspace given: split when it pays)
    N, K = 5 * 64, 1024
    W, X, m = _layer("bf16", 64, 64, N, K, "random", 7300 + M, M)
    g = np.random.default_rng(7400 + M)
    G_bits = wl.gaussian_bits((M, N), 2.0, "bf16", g)
    ref = oracle.gated_ref(G_bits, oracle.hybrid_ref(X, W, "bf16", m, 64, 64), "bf16")
    pw = hts.pack(hts.tensor_from_bits(W, "bf16", DEV), m, 64, 64)
    Xt = hts.tensor_from_bits(X, "bf16", DEV)
    G = hts.tensor_from_bits(G_bits, "bf16", DEV)
    say(f"[two-rows-gated] M={M}")
    Ys = hts.gemm_silu_mul(Xt, pw, G)                                # workspace allocated: split
    Yu = torch.empty_like(G)
    hts.hts_gemm_silu_mul(pw.desc, pw.index, pw.values, pw.meta, Xt, G, Yu)   # unsplit
    torch.cuda.synchronize()
    for what, Y in (("split", Ys), ("unsplit", Yu)):
        _check(oracle.widen_f64(hts.bits_from_tensor(Y), "bf16"), ref, f"gated {what} M={M}")

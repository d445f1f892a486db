"""GPU parity of pack / unpack and of the Wanda-derived maps against the CPU oracle.

Pack output must equal the oracle bit for bit (values, codes, tile index);
unpack(pack(W)) must equal the oracle's mask(W) bit for bit.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import tile_gemm_amd as hts
import workloads as wl
from helpers import DEV, activations, calib_scale, layer_id, named_layers, oracle_map, oracle_packed, say, weight

pytestmark = pytest.mark.gpu


def _gpu_pack(W_bits, dtype, tmap, bn, bk, cs=None):
    Wt = hts.tensor_from_bits(W_bits, dtype, DEV)
    cst = None if cs is None else torch.from_numpy(np.asarray(cs, np.float32)).to(DEV)
    pw = hts.pack(Wt, tmap, bn, bk, cst)
    torch.cuda.synchronize()
    return pw


def _check_packed(pw, vals, meta, idx):
    gv = hts.bits_from_tensor(pw.values)[: vals.size]
    assert np.array_equal(gv, vals), f"values differ at {np.nonzero(gv != vals)[0][:8]}"
    gm = pw.meta.cpu().numpy().view(np.uint32)[: meta.size]
    assert np.array_equal(gm, meta), f"codes differ at {np.nonzero(gm != meta)[0][:8]}"
    gi = pw.index.cpu().numpy().view(np.uint32)
    assert np.array_equal(gi, idx)


@pytest.mark.parametrize("cl", named_layers(), ids=layer_id)
def test_pack_and_unpack_named_layers(cl):
    c, L = cl
    say(f"[pack] {c.name}/{L.name} N={L.N} K={L.K} {L.dtype} tile={L.bn}x{L.bk}")
    W = weight(c.cfg_id, L.name)
    m = oracle_map(c.cfg_id, L.name)
    cs = calib_scale(c.cfg_id, L.name)[1] if L.map_kind == "wanda" else None
    vals, meta, idx, Wm = oracle_packed(c.cfg_id, L.name)
    pw = _gpu_pack(W, L.dtype, m, L.bn, L.bk, cs)
    _check_packed(pw, vals, meta, idx)
    Wu = hts.unpack(pw)
    torch.cuda.synchronize()
    assert np.array_equal(hts.bits_from_tensor(Wu), Wm)


EDGE_MAPS = {
    "all_dense": lambda Tn, Tk: np.zeros((Tn, Tk), np.uint8),
    "all_sparse": lambda Tn, Tk: np.ones((Tn, Tk), np.uint8),
    "checkerboard": lambda Tn, Tk: (np.add.outer(np.arange(Tn), np.arange(Tk)) % 2).astype(np.uint8),
    "one_sparse": lambda Tn, Tk: np.eye(Tn, Tk, 1, dtype=np.uint8) * (np.arange(Tn)[:, None] == 1),
    "sparse_rows": lambda Tn, Tk: np.repeat((np.arange(Tn) % 2)[:, None], Tk, 1).astype(np.uint8),
    "sparse_cols": lambda Tn, Tk: np.repeat((np.arange(Tk) % 3 == 0)[None, :], Tn, 0).astype(np.uint8),
}


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("tile", [(128, 128), (64, 64), (64, 128), (128, 64)])
@pytest.mark.parametrize("kind", list(EDGE_MAPS))
def test_pack_edge_maps_and_ties(dtype, tile, kind):
    bn, bk = tile
    N, K = 3 * bn, 5 * bk
    g = np.random.default_rng(zlib.crc32(f"{dtype}{tile}{kind}".encode()))
    # tie-heavy weights: small integers, signed zeros, subnormals
    choices = np.array([0.0, -0.0, 0.5, -0.5, 1.0, -1.0, 2.0, 3.0], np.float32)
    W = wl.to_bits(choices[g.integers(0, len(choices), (N, K))], dtype)
    W[g.random((N, K)) < 0.02] = np.uint16(0x0001)
    W[g.random((N, K)) < 0.02] = np.uint16(0x8003)
    m = EDGE_MAPS[kind](N // bn, K // bk).ravel()
    say(f"[pack-edge] {kind} {dtype} tile={bn}x{bk}")
    for cs in (None, np.abs(g.standard_normal(K)).astype(np.float32).round(1)):
        vals, meta, idx = oracle.pack(W, dtype, m, bn, bk, cs)
        pw = _gpu_pack(W, dtype, m, bn, bk, cs)
        _check_packed(pw, vals, meta, idx)
        Wu = hts.unpack(pw)
        torch.cuda.synchronize()
        assert np.array_equal(hts.bits_from_tensor(Wu), oracle.masked_weights(W, dtype, m, bn, bk, cs))


def test_pack_row_stride():
    # W as a column slice of a wider matrix (ldw > K)
    g = np.random.default_rng(5)
    N, K, ldw = 256, 256, 384
    big = wl.gaussian_bits((N, ldw), 0.02, "bf16", g)
    m = (g.random(16) < 0.5).astype(np.uint8)
    vals, meta, idx = oracle.pack(np.ascontiguousarray(big[:, :K]), "bf16", m, 64, 64)
    Wt = hts.tensor_from_bits(big, "bf16", DEV)[:, :K]
    pw = hts.pack(Wt, m, 64, 64)
    torch.cuda.synchronize()
    _check_packed(pw, vals, meta, idx)


WANDA_LAYERS = [(c, L) for c, L in named_layers() if L.map_kind == "wanda"]


@pytest.mark.parametrize("cl", WANDA_LAYERS, ids=layer_id)
def test_wanda_scale_cost_and_map(cl):
    c, L = cl
    say(f"[wanda] {c.name}/{L.name}")
    Xc, cs = calib_scale(c.cfg_id, L.name)
    Xt = hts.tensor_from_bits(Xc, L.dtype, DEV)
    gcs = hts.col_norms(Xt)
    torch.cuda.synchronize()
    assert np.array_equal(gcs.cpu().numpy().view(np.uint32), cs.view(np.uint32))
    W = weight(c.cfg_id, L.name)
    Wt = hts.tensor_from_bits(W, L.dtype, DEV)
    desc = hts.make_desc(L.N, L.K, L.bn, L.bk, L.dtype)
    cost = torch.empty(L.T, dtype=torch.float64, device=DEV)
    hts.hts_wanda_tile_cost(desc, Wt, gcs, cost)
    ocost = oracle.wanda_tile_cost(W, L.dtype, cs, L.bn, L.bk)
    gcost = cost.cpu().numpy()
    # same summation order on both sides: equal bits
    assert np.array_equal(gcost.view(np.uint64), ocost.view(np.uint64))
    gmap = hts.wanda_tile_map(Wt, gcs, L.bn, L.bk, L.n_sparse_target)
    torch.cuda.synchronize()
    assert np.array_equal(gmap.cpu().numpy(), oracle_map(c.cfg_id, L.name))
    assert int(gmap.sum().item()) == L.n_sparse_target


def test_wanda_map_ties_and_extremes():
    cost = np.array([3.0, 1.0, 1.0, 2.0, 0.5, 1.0, 7.0], np.float64)
    ct = torch.from_numpy(cost).to(DEV)
    for n_s in range(len(cost) + 1):
        m = torch.empty(len(cost), dtype=torch.uint8, device=DEV)
        hts.hts_wanda_map(ct, n_s, m)
        torch.cuda.synchronize()
        assert np.array_equal(m.cpu().numpy(), oracle.wanda_tile_map(cost, n_s))

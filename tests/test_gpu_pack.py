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


# ---------------------------------------------------------------------------
# packing from a given element mask (frozen 2:4 patterns)
# ---------------------------------------------------------------------------

def _check_masked(W, dtype, tmap, mask_np, bn, bk, ldm_pad=0):
    N, K = W.shape
    vals, meta, idx, bad = oracle.pack_masked(W, dtype, tmap, mask_np, bn, bk)
    Wt = hts.tensor_from_bits(W, dtype, DEV)
    big = torch.zeros((N, K + ldm_pad), dtype=torch.uint8, device=DEV)
    big[:, :K] = torch.from_numpy(np.ascontiguousarray(mask_np)).to(DEV)
    pw, malformed = hts.pack_masked(Wt, tmap, big[:, :K], bn, bk)
    torch.cuda.synchronize()
    _check_packed(pw, vals, meta, idx)
    assert int(malformed.item()) == bad
    back = hts.bits_from_tensor(hts.unpack(pw))
    assert np.array_equal(back, oracle.masked_weights_from_mask(W, tmap, mask_np, bn, bk))
    return pw


@pytest.mark.parametrize("name", ["tiny/tiny", "7b_up/up_proj", "13b/sq_5120", "sweep/sweep_p0.5", "7b_up_fp8/up_proj_fp8"])
def test_pack_masked_named_layers(name):
    cname, lname = name.split("/")
    c = wl.config(cname)
    L = next(l for l in c.layers if l.name == lname)
    say(f"[pack-masked] {cname}/{lname}")
    W = weight(c.cfg_id, L.name)
    _check_masked(W, L.dtype, oracle_map(c.cfg_id, L.name), wl.layer_pair_mask(c, L), L.bn, L.bk)


@pytest.mark.parametrize("dtype,tile", [("bf16", (128, 128)), ("f16", (64, 64)), ("bf16", (128, 64))])
def test_pack_masked_malformed_and_strided(dtype, tile):
    bn, bk = tile
    N, K = 2 * bn, 4 * bk
    g = np.random.default_rng(zlib.crc32(f"{dtype}{tile}".encode()))
    W = wl.gaussian_bits((N, K), 0.02, dtype, g)
    tmap = (g.random((N // bn) * (K // bk)) < 0.6).astype(np.uint8)
    say(f"[pack-masked] malformed {dtype} tile={tile}")
    mask = (g.random((N, K)) < 0.5).astype(np.uint8) * g.integers(1, 255, size=(N, K)).astype(np.uint8)
    _check_masked(W, dtype, tmap, mask, bn, bk, ldm_pad=48)
    _check_masked(W, dtype, tmap, wl.pair_mask(N, K, g), bn, bk, ldm_pad=16)


def test_pack_masked_with_magnitude_mask_equals_pack():
    c = wl.config("7b_up")
    L = c.layers[0]
    W = weight(c.cfg_id, L.name)
    tmap = oracle_map(c.cfg_id, L.name)
    pw = _gpu_pack(W, L.dtype, tmap, L.bn, L.bk)
    Wall = oracle.masked_weights(W, L.dtype, np.ones_like(tmap), L.bn, L.bk)
    mask = np.zeros(W.shape, np.uint8)
    # the magnitude keep pattern, from a pack with every tile 2:4 (zero weights resolved by the codes)
    pall = _gpu_pack(W, L.dtype, np.ones_like(tmap), L.bn, L.bk)
    words = pall.meta.cpu().numpy().view(np.uint32)
    Tk = L.K // L.bk
    codes = words.reshape(L.N // L.bn, Tk, L.bn, L.bk // 32)           # tiles in order, rows, words
    nib = (codes[..., None] >> (4 * np.arange(8, dtype=np.uint32))) & 0xF
    nib = nib.reshape(L.N // L.bn, Tk, L.bn, L.bk // 4).transpose(0, 2, 1, 3).reshape(L.N, L.K // 4)
    rows = np.arange(L.N)[:, None]
    gbase = 4 * np.arange(L.K // 4)[None, :]
    mask[rows, gbase + (nib & 3)] = 1
    mask[rows, gbase + (nib >> 2)] = 1
    assert np.array_equal(np.where(mask == 1, W, 0), Wall)
    Wt = hts.tensor_from_bits(W, L.dtype, DEV)
    pm, malformed = hts.pack_masked(Wt, tmap, torch.from_numpy(mask).to(DEV), L.bn, L.bk)
    torch.cuda.synchronize()
    assert int(malformed.item()) == 0
    assert torch.equal(pm.values, pw.values) and torch.equal(pm.meta, pw.meta)


def test_wanda_global_maps_of_a_block():
    # one sparse-tile budget shared by the seven projections of the 7B block (rho = 0.3 overall)
    c = wl.config("7b_block")
    Ws, css, ocosts = [], [], []
    for L in c.layers:
        Xc, cs = calib_scale(c.cfg_id, L.name)
        W = weight(c.cfg_id, L.name)
        Ws.append(hts.tensor_from_bits(W, L.dtype, DEV))
        css.append(torch.from_numpy(cs).to(DEV))
        ocosts.append(oracle.wanda_tile_cost(W, L.dtype, cs, L.bn, L.bk))
    T = sum(L.T for L in c.layers)
    n_s = int(round(2 * 0.3 * T))
    say(f"[wanda-global] {len(Ws)} layers, {T} tiles, {n_s} sparse")
    gm = hts.wanda_global_maps(Ws, css, 128, 128, n_s)
    torch.cuda.synchronize()
    om = oracle.wanda_global_maps(ocosts, n_s)
    for L, a, b in zip(c.layers, gm, om):
        assert np.array_equal(a.cpu().numpy(), b), L.name
    assert sum(int(m.sum().item()) for m in gm) == n_s

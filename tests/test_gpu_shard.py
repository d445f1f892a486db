"""Column-parallel (N) sharding of the 7B up-projection, checked on one GPU.

An 8-way split gives each GPU a contiguous range of 10 or 11 of the 86 tile rows (N = 1280 or
1408, K = 4096). Because tiles are stored in row-major tile order, a shard is a pure subset of
the tile list:
- its packed values and codes are a contiguous slice of the whole layer's buffers;
- its index is the layer's index shifted by the slice's start.

An output block accumulates over its own tile row only. So the shard's product, run unsplit,
reproduces the whole product's columns bit for bit, with no exchange between GPUs. The library
may split a narrow share's product over K (fewer output blocks), which changes only the fp32
rounding order. Both forms are checked against the oracle on sampled rows.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import tile_gemm_amd as hts
import workloads as wl
from helpers import DEV, say, weight, oracle_map, activations

pytestmark = pytest.mark.gpu
TOL = 5e-3
CFG = wl.config("7b_up")
LAYER = CFG.layers[0]
ROWS = [11] * 6 + [10] * 2           # tile rows per GPU, 86 in all
BOUNDS = np.concatenate([[0], np.cumsum(ROWS)]).tolist()
SHARDS = [(BOUNDS[i], BOUNDS[i + 1]) for i in (0, 6, 7)]   # the first, the first 10-row one, the last


@functools.lru_cache(maxsize=1)
def _full():
    W = weight(CFG.cfg_id, LAYER.name)
    m = oracle_map(CFG.cfg_id, LAYER.name)
    pw = hts.pack(hts.tensor_from_bits(W, "bf16", DEV), m, 128, 128)
    torch.cuda.synchronize()
    return W, m, pw


@functools.lru_cache(maxsize=4)
def _full_product(M):
    _, _, pw = _full()
    X = hts.tensor_from_bits(np.ascontiguousarray(activations(CFG.cfg_id, LAYER.name)[:M]), "bf16", DEV)
    Y = hts.gemm(X, pw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    return X, Y


def _shard(r0, r1):
    W, m, _ = _full()
    Tk = LAYER.K // 128
    Ws = np.ascontiguousarray(W[128 * r0:128 * r1])
    ms = np.ascontiguousarray(m.reshape(-1, Tk)[r0:r1].ravel())
    return Ws, ms


@pytest.mark.parametrize("shard", SHARDS)
def test_shard_pack_is_a_slice_of_the_layer(shard):
    r0, r1 = shard
    Ws, ms = _shard(r0, r1)
    _, m, pw_full = _full()
    say(f"[shard-pack] tile rows {r0}..{r1 - 1}")
    pw = hts.pack(hts.tensor_from_bits(Ws, "bf16", DEV), ms, 128, 128)
    torch.cuda.synchronize()
    Tk = LAYER.K // 128
    idx_full = pw_full.index.cpu().numpy().view(np.uint32)
    idx = pw.index.cpu().numpy().view(np.uint32)
    t0, t1 = r0 * Tk, r1 * Tk
    v0, c0 = int(idx_full[t0, 0]), int(idx_full[t0, 1])
    v1 = int(idx_full[t1, 0]) if t1 < idx_full.shape[0] else pw_full.sizes["values_bytes"] // 2
    c1 = int(idx_full[t1, 1]) if t1 < idx_full.shape[0] else pw_full.sizes["meta_bytes"] // 4
    # the shard's index is the layer's, shifted by the slice start
    assert np.array_equal(idx[:, 0], idx_full[t0:t1, 0] - v0)
    assert np.array_equal(idx[:, 1], idx_full[t0:t1, 1] - c0)
    assert np.array_equal(idx[:, 2], idx_full[t0:t1, 2])
    vals_full = hts.bits_from_tensor(pw_full.values)
    vals = hts.bits_from_tensor(pw.values)
    assert np.array_equal(vals[: v1 - v0], vals_full[v0:v1])
    meta_full = pw_full.meta.cpu().numpy().view(np.uint32)
    meta = pw.meta.cpu().numpy().view(np.uint32)
    assert np.array_equal(meta[: c1 - c0], meta_full[c0:c1])


@pytest.mark.parametrize("M", [1, 16, 2048])
@pytest.mark.parametrize("shard", SHARDS)
def test_shard_product_is_the_layer_columns(shard, M):
    r0, r1 = shard
    Ws, ms = _shard(r0, r1)
    say(f"[shard-gemm] tile rows {r0}..{r1 - 1} M={M}")
    X, Y_full = _full_product(M)
    pw = hts.pack(hts.tensor_from_bits(Ws, "bf16", DEV), ms, 128, 128)
    # unsplit (a workspace too small for the parts of a split product): the same sums as the layer
    Yu = hts.gemm(X, pw, out_dtype=torch.float32, workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
    # default: a share this narrow at M = 2048 has few enough blocks to be split
    Y = hts.gemm(X, pw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(Yu, Y_full[:, 128 * r0:128 * r1])
    rows = np.arange(M)
    Xh = activations(CFG.cfg_id, LAYER.name)[rows]
    Y_ref = oracle.gemm_ref(Xh, oracle.masked_weights(Ws, "bf16", ms, 128, 128), "bf16")
    for what, Yc in (("unsplit", Yu), ("default", Y)):
        ok, rel = oracle.within_tolerance(Yc.cpu().numpy()[rows], Y_ref, TOL)
        say(f"    {what}: max err / max|ref| = {rel:.3e}")
        assert ok

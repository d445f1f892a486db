"""Shared fixtures of the GPU parity tests: named layers, their oracle results, device copies."""
import functools
import sys

import numpy as np

import oracle
import workloads as wl

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def named_layers():
    """(config, layer) for every layer of the named workloads."""
    return [(c, L) for c in wl.CONFIGS for L in c.layers]


def layer_id(cl):
    c, L = cl
    return f"{c.name}-{L.name}"


@functools.lru_cache(maxsize=16)
def weight(cfg_id: int, layer_name: str):
    c = wl.config(cfg_id)
    L = next(x for x in c.layers if x.name == layer_name)
    return wl.weight_bits(c, L)


@functools.lru_cache(maxsize=16)
def calib_scale(cfg_id: int, layer_name: str):
    """(calibration bits, oracle column scale) for a Wanda layer."""
    c = wl.config(cfg_id)
    L = next(x for x in c.layers if x.name == layer_name)
    Xc = wl.layer_calib_bits(c, L)
    return Xc, oracle.column_norms(Xc, L.dtype)


@functools.lru_cache(maxsize=16)
def oracle_map(cfg_id: int, layer_name: str):
    """Tile map: drawn (bernoulli / exact) or the oracle's Wanda map."""
    c = wl.config(cfg_id)
    L = next(x for x in c.layers if x.name == layer_name)
    if L.map_kind != "wanda":
        return wl.tile_map(c, L)
    _, cs = calib_scale(cfg_id, layer_name)
    cost = oracle.wanda_tile_cost(weight(cfg_id, layer_name), L.dtype, cs, L.bn, L.bk)
    return oracle.wanda_tile_map(cost, L.n_sparse_target)


@functools.lru_cache(maxsize=16)
def oracle_packed(cfg_id: int, layer_name: str):
    c = wl.config(cfg_id)
    L = next(x for x in c.layers if x.name == layer_name)
    cs = calib_scale(cfg_id, layer_name)[1] if L.map_kind == "wanda" else None
    W = weight(cfg_id, layer_name)
    m = oracle_map(cfg_id, layer_name)
    vals, meta, idx = oracle.pack(W, L.dtype, m, L.bn, L.bk, cs)
    Wm = oracle.unpack(vals, meta, idx, L.N, L.K, L.bn, L.bk)
    return vals, meta, idx, Wm


@functools.lru_cache(maxsize=16)
def activations(cfg_id: int, layer_name: str):
    c = wl.config(cfg_id)
    L = next(x for x in c.layers if x.name == layer_name)
    return wl.activation_bits(c, L, max(c.Ms))


@functools.lru_cache(maxsize=2)
def layer_ref(cfg_id: int, layer_name: str, M: int) -> np.ndarray:
    """Oracle Y = X[:M] . mask(W)^T (fp64) of a named layer, every row and column."""
    c = wl.config(cfg_id)
    L = next(x for x in c.layers if x.name == layer_name)
    Wm = oracle_packed(cfg_id, layer_name)[3]
    return oracle.gemm_ref(np.ascontiguousarray(activations(cfg_id, layer_name)[:M]), Wm, L.dtype)

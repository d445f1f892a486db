"""The seeded input generators: rounding and determinism (no method arithmetic lives there)."""
import hashlib

import numpy as np
import pytest
import torch

import workloads as wl


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(200000).astype(np.float32) * np.float32(s) for s in (0.02, 1.0, 1e-30, 1e4)])
    # halfway cases: a bf16 value plus exactly half an ulp, both parities of the kept bit
    u = (g.integers(0, 1 << 15, size=4096, dtype=np.uint32) << 16) | np.uint32(0x8000)
    x = np.concatenate([x, u.view(np.float32)[np.isfinite(u.view(np.float32))]])
    ours = wl.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_f16_rounding_matches_torch():
    g = np.random.default_rng(1)
    x = g.standard_normal(100000).astype(np.float32) * np.float32(0.02)
    x[:100] *= np.float32(1e-3)                     # subnormal range of binary16
    ours = wl.f32_to_f16_bits(x)
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def _h(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]


def test_tiny_config_is_deterministic():
    c = wl.config("tiny")
    L = c.layers[0]
    a = (wl.weight_bits(c, L), wl.activation_bits(c, L, 8), wl.tile_map(c, L))
    b = (wl.weight_bits(c, L), wl.activation_bits(c, L, 8), wl.tile_map(c, L))
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    assert [_h(x) for x in a] == TINY_HASHES


# SHA-256 prefixes of (W, X, map) of the tiny configuration, recorded once
TINY_HASHES = ["b876e87b615d6c53", "61da6f8fa9dbc7ff", "6b9fe411259c2fcc"]


def test_exact_maps_have_exact_counts():
    for c in wl.CONFIGS:
        for L in c.layers:
            if L.map_kind == "exact":
                m = wl.tile_map(c, L)
                assert int(m.sum()) == L.n_sparse_target == int(round(L.p * L.T))


def test_shapes_tile_exactly():
    for c in wl.CONFIGS:
        for L in c.layers:
            assert L.N % L.bn == 0 and L.K % L.bk == 0 and L.bk % 32 == 0


def test_wanda_targets():
    c = wl.config("7b_block")
    assert [L.n_sparse_target for L in c.layers] == [614, 614, 614, 614, 1651, 1651, 1651]

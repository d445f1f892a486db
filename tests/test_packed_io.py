"""Packed-weight files: a saved weight loads back byte for byte, and a damaged or inconsistent
file is refused. The CPU cases build the packed weight from the oracle's pack (host tensors), so
they run without a GPU; the GPU case packs on the device and checks that the product over the
loaded weight equals the product over the original bit for bit."""
import json
import struct

import numpy as np
import pytest
import torch

import oracle
import tile_gemm_amd as hts
from tile_gemm_amd import packed_io
import workloads as wl

CASES = [  # (N, K, bn, bk, dtype, map kind)
    (256, 512, 128, 128, "bf16", "random"),
    (256, 512, 64, 64, "f16", "random"),
    (256, 512, 128, 128, "fp8", "random"),
    (128, 256, 32, 32, "bf16", "random"),
    (256, 256, 128, 128, "bf16", "dense"),
    (256, 256, 128, 128, "f16", "sparse"),
]


def _host_packed(N, K, bn, bk, dtype, kind, seed=3):
    g = np.random.default_rng(seed)
    W = wl.gaussian_bits((N, K), 1.0 if dtype == "fp8" else 0.02, dtype, g)
    T = (N // bn) * (K // bk)
    m = {"random": (g.random(T) < 0.5), "dense": np.zeros(T), "sparse": np.ones(T)}[kind].astype(np.uint8)
    vals, meta, index = oracle.pack(W, dtype, m, bn, bk)
    desc = hts.make_desc(N, K, bn, bk, dtype)
    _, sizes = hts.hts_pack_plan(desc, m)
    vt = torch.from_numpy(vals.view(np.uint8 if dtype == "fp8" else np.int16).copy())
    mt = torch.from_numpy(meta.view(np.int32).copy()) if meta.size else torch.zeros(4, dtype=torch.int32)
    it = torch.from_numpy(index.view(np.int32).copy())
    return hts.PackedWeight(desc, it, vt, mt, sizes, m)


def _bytes(t, n):
    return t.reshape(-1).view(torch.uint8)[:n].numpy().tobytes()


@pytest.mark.parametrize("case", CASES, ids=[f"{c[4]}-{c[2]}x{c[3]}-{c[5]}" for c in CASES])
def test_round_trip_is_exact(case, tmp_path):
    pw = _host_packed(*case)
    f = tmp_path / "w.hts"
    pw.save(str(f))
    back = hts.PackedWeight.load(str(f), device="cpu")
    for k in ("N", "K", "bn", "bk", "dtype"):
        assert getattr(back.desc, k) == getattr(pw.desc, k), k
    assert back.sizes == pw.sizes
    assert np.array_equal(back.tile_map, pw.tile_map)
    assert torch.equal(back.index, pw.index)
    assert _bytes(back.values, pw.sizes["values_bytes"]) == _bytes(pw.values, pw.sizes["values_bytes"])
    assert _bytes(back.meta, pw.sizes["meta_bytes"]) == _bytes(pw.meta, pw.sizes["meta_bytes"])
    assert back.values.dtype == pw.values.dtype
    # sections start on 64-byte boundaries
    raw = f.read_bytes()
    hlen = struct.unpack("<I", raw[12:16])[0]
    h = json.loads(raw[16:16 + hlen])
    assert all(s["offset"] % 64 == 0 for s in h["sections"])
    assert h["abi"] == hts.hts_abi_version() and h["format"] == packed_io.FORMAT_VERSION


def _saved(tmp_path):
    pw = _host_packed(*CASES[0])
    f = tmp_path / "w.hts"
    pw.save(str(f))
    return pw, f, bytearray(f.read_bytes())


def _header(raw):
    hlen = struct.unpack("<I", raw[12:16])[0]
    return json.loads(bytes(raw[16:16 + hlen])), hlen


def _expect_refusal(tmp_path, raw, words):
    g = tmp_path / "bad.hts"
    g.write_bytes(bytes(raw))
    with pytest.raises(packed_io.PackedFileError, match=words):
        hts.PackedWeight.load(str(g), device="cpu")


def test_refuses_wrong_magic_and_version(tmp_path):
    _, _, raw = _saved(tmp_path)
    bad = bytearray(raw)
    bad[0:8] = b"NOTPACK\0"
    _expect_refusal(tmp_path, bad, "not a packed-weight file")
    bad = bytearray(raw)
    bad[8:12] = struct.pack("<I", 2)
    _expect_refusal(tmp_path, bad, "format version 2")
    _expect_refusal(tmp_path, raw[:10], "not a packed-weight file")


@pytest.mark.parametrize("section", ["tile_map", "index", "values", "meta"])
def test_refuses_a_flipped_bit_in_any_section(tmp_path, section):
    _, _, raw = _saved(tmp_path)
    h, _ = _header(raw)
    s = next(s for s in h["sections"] if s["name"] == section)
    raw[s["offset"] + s["bytes"] // 2] ^= 0x10
    _expect_refusal(tmp_path, raw, f"checksum of section {section}")


def test_refuses_truncation(tmp_path):
    _, _, raw = _saved(tmp_path)
    _expect_refusal(tmp_path, raw[:len(raw) - 100], "outside the file")
    _, hlen = _header(raw)
    _expect_refusal(tmp_path, raw[:16 + hlen // 2], "truncated header")


def test_refuses_an_index_that_does_not_match_the_map(tmp_path):
    pw = _host_packed(*CASES[0])
    flipped = pw.tile_map.copy()
    flipped[0] ^= 1
    liar = hts.PackedWeight(pw.desc, pw.index, pw.values, pw.meta, pw.sizes, flipped)
    f = tmp_path / "liar.hts"
    liar.save(str(f))   # checksums are right; the content is not
    with pytest.raises(packed_io.PackedFileError, match="tile map gives|does not match the tile map"):
        hts.PackedWeight.load(str(f), device="cpu")


def test_refuses_recorded_sizes_that_disagree(tmp_path):
    _, _, raw = _saved(tmp_path)
    h, hlen = _header(raw)
    h["n_sparse"] += 1
    text = json.dumps(h, sort_keys=True).encode()
    assert len(text) <= hlen
    raw[16:16 + hlen] = text.ljust(hlen, b" ")
    _expect_refusal(tmp_path, raw, "n_sparse")


def test_refuses_a_short_buffer_on_save(tmp_path):
    pw = _host_packed(*CASES[0])
    short = hts.PackedWeight(pw.desc, pw.index, pw.values[:10], pw.meta, pw.sizes, pw.tile_map)
    with pytest.raises(packed_io.PackedFileError, match="buffer holds"):
        short.save(str(tmp_path / "short.hts"))
    assert not (tmp_path / "short.hts").exists()


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,tile", [("bf16", 128), ("fp8", 128), ("f16", 64)])
def test_loaded_weight_gives_the_same_product(tmp_path, dtype, tile):
    from helpers import DEV
    g = np.random.default_rng(11)
    N, K, M = 512, 768, 40
    W = hts.tensor_from_bits(wl.gaussian_bits((N, K), 1.0 if dtype == "fp8" else 0.02, dtype, g), dtype, DEV)
    X = hts.tensor_from_bits(wl.gaussian_bits((M, K), 1.0, dtype, g), dtype, DEV)
    m = (g.random((N // tile) * (K // tile)) < 0.5).astype(np.uint8)
    pw = hts.pack(W, m, tile, tile)
    f = tmp_path / "w.hts"
    pw.save(str(f))
    back = hts.PackedWeight.load(str(f), device=DEV)
    assert torch.equal(back.index, pw.index)
    Y0 = hts.gemm(X, pw, out_dtype=torch.float32)
    Y1 = hts.gemm(X, back, out_dtype=torch.float32)
    assert torch.equal(Y0, Y1)

"""The C ABI on a host without a GPU: the library loads, exports every declared
entry point, builds the tile index exactly as the oracle's plan, and rejects
bad arguments before touching the GPU (no kernel is launched here)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import tile_gemm_amd as hts
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_entry_points():
    text = open(os.path.join(ROOT, "include", "hts.h")).read()
    return sorted(set(re.findall(r"^\s*(?:hts_status|uint32_t|const char\*)\s+(hts_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    L = hts.lib()
    names = declared_entry_points()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert sorted(hts.EXPORTED) == names


def test_version_and_status_strings():
    assert hts.hts_abi_version() == 1
    for code in range(9):
        assert hts.hts_status_string(code)
    assert hts.hts_status_string(99) == "unknown status"


def _maps():
    out = []
    for c in wl.CONFIGS:
        for L in c.layers:
            if L.map_kind == "wanda":
                m = wl.exact_map(L.T, L.n_sparse_target, wl.rng(c.cfg_id, L.layer_id, wl.TAG_MAP))
            else:
                m = wl.tile_map(c, L)
            out.append((L, m))
    return out


@pytest.mark.parametrize("case", range(len(_maps())))
def test_plan_matches_oracle(case):
    L, m = _maps()[case]
    desc = hts.make_desc(L.N, L.K, L.bn, L.bk, L.dtype)
    index, sizes = hts.hts_pack_plan(desc, m)
    o_index, o_sizes = oracle.plan(m, L.N, L.K, L.bn, L.bk, elem_bytes=1 if L.dtype == "fp8" else 2)
    assert np.array_equal(index, o_index)
    assert sizes["values_bytes"] == o_sizes["values_bytes"]
    assert sizes["meta_bytes"] == o_sizes["meta_bytes"]
    assert sizes["index_bytes"] == o_sizes["index_bytes"]
    assert sizes["n_sparse"] == o_sizes["n_sparse"]


def test_plan_edge_maps():
    N, K, bn, bk = 512, 384, 128, 128
    T = 12
    for m in (np.zeros(T, np.uint8), np.ones(T, np.uint8), np.arange(T, dtype=np.uint8) % 2,
              np.eye(1, T, 5, dtype=np.uint8).ravel()):
        idx, sz = hts.hts_pack_plan(hts.make_desc(N, K, bn, bk, "bf16"), m)
        assert np.array_equal(idx, oracle.plan(m, N, K, bn, bk)[0])
        assert sz["values_bytes"] == 2 * (N * K - int(m.sum()) * bn * bk // 2)


def _err(fn):
    with pytest.raises(hts.HTSError) as e:
        fn()
    return e.value.status


def test_plan_rejects_bad_arguments():
    m = np.zeros(16, np.uint8)
    assert _err(lambda: hts.hts_pack_plan(hts.make_desc(256, 256, 64, 64, "f16"), np.full(16, 2, np.uint8))) == 5
    assert _err(lambda: hts.hts_pack_plan(hts.make_desc(250, 256, 64, 64, "f16"), m)) == 3
    assert _err(lambda: hts.hts_pack_plan(hts.make_desc(256, 256, 16, 64, "f16"), np.zeros(64, np.uint8))) == 7
    d = hts.make_desc(256, 256, 64, 64, "f16")
    d.dtype = 2
    assert _err(lambda: hts.hts_pack_plan(d, m)) == 2
    d = hts.make_desc(256, 256, 64, 64, "f16")
    d.reserved = 1
    assert _err(lambda: hts.hts_pack_plan(d, m)) == 1
    assert _err(lambda: hts.hts_pack_plan(hts.make_desc(1 << 17, 1 << 15, 128, 128, "bf16"),
                                          np.zeros((1 << 10) * (1 << 8), np.uint8))) == 3


# fake device addresses: never dereferenced, every call below fails its host checks
A16, A8 = 0x10000, 0x10008


def test_gated_gemm_rejects_bad_arguments_before_any_launch():
    # hts_gemm_silu_mul: hts_gemm's checks, plus G (non-NULL, 16-byte aligned) and ldg (>= N, a
    # multiple of 4); M == 0 is a no-op even without G
    L = hts.lib()
    d = hts.make_desc(256, 256, 64, 64, "f16")

    def gated(G=A16, ldg=256, M=4, yd=2, index=A16):
        return L.hts_gemm_silu_mul(ctypes.byref(d), index, A16, A16, M, A16, 256, G, ldg, A16, 256, yd, None, 0, None)

    assert gated(G=None) == 1
    assert gated(G=A8) == 4
    assert gated(ldg=255) == 3
    assert gated(ldg=258) == 4
    assert gated(index=None) == 1
    assert gated(yd=7) == 2
    assert gated(G=None, M=0) == 0


def test_gemm_rejects_bad_arguments_before_any_launch():
    L = hts.lib()
    d = hts.make_desc(256, 256, 64, 64, "f16")
    by = ctypes.byref

    def gemm(desc=d, index=A16, values=A16, meta=A16, M=4, X=A16, ldx=256, Y=A16, ldy=256, yd=2):
        return L.hts_gemm(by(desc), index, values, meta, M, X, ldx, Y, ldy, yd, None, 0, None)

    assert gemm(M=-1) == 3
    assert gemm(yd=7) == 2
    assert gemm(index=None) == 1
    assert gemm(values=A8) == 4
    assert gemm(meta=A8) == 4
    assert gemm(ldx=255) == 3
    assert gemm(ldx=260) == 4
    assert gemm(ldy=254) == 3
    assert gemm(X=A8) == 4
    assert gemm(Y=None) == 1
    assert gemm(M=0) == 0                       # empty input: a no-op, nothing launched
    bad = hts.make_desc(256, 256, 64, 96, "f16")
    assert gemm(desc=bad) == 7
    assert b"multiple" in L.hts_last_error() or b"64 or 128" in L.hts_last_error()
    # above the streaming range a tile row must fit the tiled kernel's 256 tile columns
    wide = hts.make_desc(128, 128 * 257, 128, 128, "bf16")
    assert gemm(desc=wide, M=64, ldx=128 * 257, ldy=128) == 7
    assert b"tile columns" in L.hts_last_error()


def test_other_entry_points_reject_bad_arguments():
    L = hts.lib()
    by = ctypes.byref
    d = hts.make_desc(256, 256, 64, 64, "bf16")
    assert L.hts_pack(by(d), A16, A16, 255, None, A16, A16, None) == 3
    assert L.hts_pack(by(d), A16, A8, 256, None, A16, A16, None) == 4
    assert L.hts_pack(by(d), None, A16, 256, None, A16, A16, None) == 1
    assert L.hts_unpack(by(d), A16, A16, A16, A16, 100, None) == 3
    assert L.hts_dense_gemm(1, 4, 100, 256, A16, 256, A16, 256, A16, 256, 2, None, 0, None) == 3
    assert L.hts_dense_gemm(2, 4, 128, 256, A16, 256, A16, 256, A16, 256, 2, None, 0, None) == 2
    assert L.hts_dense_gemm(1, 0, 128, 256, A16, 256, A16, 256, A16, 256, 2, None, 0, None) == 0
    assert L.hts_col_norms(1, 0, 16, A16, 16, A16, None) == 3
    assert L.hts_col_norms(1, 4, 16, A16, 8, A16, None) == 3
    assert L.hts_wanda_tile_cost(by(d), A16, 256, None, A16, None) == 1
    assert L.hts_wanda_map(10, A16, 11, A16, None) == 3
    assert L.hts_wanda_map(10, A8 + 4, 3, A16, None) == 4
    n = ctypes.c_size_t(123)
    assert L.hts_gemm_workspace(by(d), 16, by(n)) == 0 and n.value == 0


def test_pack_masked_rejects_bad_arguments():
    L = hts.lib()
    by = ctypes.byref
    d = hts.make_desc(256, 256, 64, 64, "bf16")
    assert L.hts_pack_masked(by(d), A16, A16, 256, None, 256, A16, A16, None, None) == 1     # no mask
    assert L.hts_pack_masked(by(d), A16, A16, 256, A8, 256, A16, A16, None, None) == 4       # mask alignment
    assert L.hts_pack_masked(by(d), A16, A16, 256, A16, 200, A16, A16, None, None) == 3      # ldm < K
    assert L.hts_pack_masked(by(d), A16, A16, 256, A16, 264, A16, A16, None, None) == 4      # ldm % 16
    assert L.hts_pack_masked(by(d), A16, A16, 256, A16, 256, A16, A16, A8 + 2, None) == 4    # counter alignment
    bad = hts.make_desc(256, 200, 64, 64, "bf16")
    assert L.hts_pack_masked(by(bad), A16, A16, 256, A16, 256, A16, A16, None, None) == 3    # K % bk


def test_silu_mul_rejects_bad_arguments():
    L = hts.lib()
    assert L.hts_silu_mul(2, 4, 64, A16, 64, A16, 64, A16, 64, None) == 2       # f32 not supported
    assert L.hts_silu_mul(1, 4, 60, A16, 64, A16, 64, A16, 64, None) == 3       # N % 8
    assert L.hts_silu_mul(1, 4, 64, A16, 60, A16, 64, A16, 64, None) == 3       # ldg < N
    assert L.hts_silu_mul(1, 4, 64, A8, 64, A16, 64, A16, 64, None) == 4        # alignment
    assert L.hts_silu_mul(1, 4, 64, None, 64, A16, 64, A16, 64, None) == 1      # null
    assert L.hts_silu_mul(1, 0, 64, None, 64, None, 64, None, 64, None) == 0    # M == 0: nothing to do


def test_fp8_arguments():
    L = hts.lib()
    by = ctypes.byref
    # 8-bit weights take 128x128 tiles only, and sizes count one byte per element
    assert _err(lambda: hts.hts_pack_plan(hts.make_desc(256, 256, 64, 64, "fp8"), np.zeros(16, np.uint8))) == 7
    m = np.array([1, 0, 0, 1], np.uint8)
    idx, sz = hts.hts_pack_plan(hts.make_desc(256, 256, 128, 128, "fp8"), m)
    assert np.array_equal(idx, oracle.plan(m, 256, 256, 128, 128, elem_bytes=1)[0])
    assert sz["values_bytes"] == 256 * 256 - 2 * 128 * 128 // 2
    assert sz["meta_bytes"] == 2 * 128 * 128 // 8
    d = hts.make_desc(256, 256, 128, 128, "fp8")
    # leading dimensions are whole 16-byte chunks: multiples of 16 one-byte elements
    assert L.hts_pack(by(d), A16, A16, 264, None, A16, A16, None) == 4
    assert L.hts_unpack(by(d), A16, A16, A16, A16, 264, None) == 4
    assert L.hts_gemm(by(d), A16, A16, A16, 4, A16, 264, A16, 256, 2, None, 0, None) == 4
    assert L.hts_gemm(by(d), A16, A16, A16, 4, A16, 256, A16, 256, 3, None, 0, None) == 2   # Y is never 8-bit
    # the Wanda helpers stay 16-bit
    assert L.hts_wanda_tile_cost(by(d), A16, 256, A16, A16, None) == 2
    assert L.hts_col_norms(3, 4, 256, A16, 256, A16, None) == 2
    # the 8-bit dense product needs N and K in whole 128-wide tiles
    assert L.hts_dense_gemm(3, 4, 192, 256, A16, 256, A16, 256, A16, 256, 2, None, 0, None) == 3
    assert L.hts_dense_gemm(3, 0, 256, 256, A16, 256, A16, 256, A16, 256, 2, None, 0, None) == 0


def test_small_tiles_plan_and_workspace():
    L = hts.lib()
    by = ctypes.byref
    # 32x32, 32x128 and 128x32 tiles: the plan as for any tile; the streaming range needs no
    # workspace, larger M an unpacked copy of the weight
    for bn, bk in ((32, 32), (32, 128), (128, 32)):
        N, K = 256, 384
        g = np.random.default_rng(bn + bk)
        m = (g.random((N // bn) * (K // bk)) < 0.5).astype(np.uint8)
        d = hts.make_desc(N, K, bn, bk, "bf16")
        idx, sz = hts.hts_pack_plan(d, m)
        o_idx, o_sz = oracle.plan(m, N, K, bn, bk)
        assert np.array_equal(idx, o_idx) and sz["values_bytes"] == o_sz["values_bytes"]
        assert sz["meta_bytes"] == o_sz["meta_bytes"]
        # the streaming kernel covers M <= 32 on 128-wide tiles (two X row groups), else M <= 16
        top = 32 if bk == 128 else 16
        assert hts.hts_gemm_workspace(d, top) == 0
        assert hts.hts_gemm_workspace(d, top + 1) == N * K * 2
        # missing or short workspace: HTS_ERR_WORKSPACE, misaligned: HTS_ERR_ALIGN, before any launch
        assert L.hts_gemm(by(d), A16, A16, A16, top + 1, A16, K, A16, N, 2, None, 0, None) == 6
        assert L.hts_gemm(by(d), A16, A16, A16, top + 1, A16, K, A16, N, 2, A16, N * K, None) == 6
        assert L.hts_gemm(by(d), A16, A16, A16, top + 1, A16, K, A16, N, 2, A8, N * K * 2, None) == 4
    assert hts.hts_gemm_workspace(hts.make_desc(256, 384, 128, 128, "bf16"), 2048) == 0
    assert _err(lambda: hts.hts_pack_plan(hts.make_desc(256, 256, 32, 32, "fp8"), np.zeros(64, np.uint8))) == 7


def _r256(x):
    return (x + 255) // 256 * 256


def test_split_product_workspace_sizes(monkeypatch):
    # the parts of a split product: nsplit * M * N floats when the tiled kernel would have at most
    # 256 output blocks; nsplit = min(8, 512 // blocks), lowered until every part has >= 4 slices
    N, K = 11008, 4096
    d = hts.make_desc(N, K, 128, 128, "bf16")
    # (M <= 32 runs on the streaming kernel: 16-bit data on 128-wide tiles)
    for M, ns in ((1, 0), (16, 0), (17, 0), (32, 0), (33, 5), (128, 5), (129, 2), (256, 2), (257, 0), (2048, 0)):
        assert hts.hts_gemm_workspace(d, M) == (_r256(ns * M * N * 4) if ns else 0), M
        assert hts.hts_dense_gemm_workspace("bf16", M, N, K) == (_r256(ns * M * N * 4) if ns else 0), M
    # 8-bit: 128-wide slices (32 per tile row here); 64x64 tiles: 64-row blocks
    assert hts.hts_gemm_workspace(hts.make_desc(N, K, 128, 128, "fp8"), 17) == 0     # streams at M <= 32
    assert hts.hts_gemm_workspace(hts.make_desc(N, K, 128, 128, "fp8"), 33) == _r256(5 * 33 * N * 4)
    assert hts.hts_gemm_workspace(hts.make_desc(4096, 4096, 64, 64, "bf16"), 17) == _r256(8 * 17 * 4096 * 4)
    # 64-row tiles go two tile rows to a 128-row block: at M = 200, 32 x 2 = 64 blocks -> 8 parts; with
    # one tile row per block (HTS_PREFILL_TWO_ROWS=0) 64 x 2 = 128 blocks -> 4 parts
    d64 = hts.make_desc(4096, 4096, 64, 64, "bf16")
    assert hts.hts_gemm_workspace(d64, 200) == _r256(8 * 200 * 4096 * 4)
    monkeypatch.setenv("HTS_PREFILL_TWO_ROWS", "0")
    assert hts.hts_gemm_workspace(d64, 200) == _r256(4 * 200 * 4096 * 4)
    monkeypatch.delenv("HTS_PREFILL_TWO_ROWS")
    # few slices: K = 256 has 4 (bf16), too few to split
    assert hts.hts_gemm_workspace(hts.make_desc(1024, 256, 128, 128, "bf16"), 64) == 0
    # 32-wide tiles: the unpacked weight, then the parts of the dense product
    d32 = hts.make_desc(N, K, 32, 32, "bf16")
    assert hts.hts_gemm_workspace(d32, 17) == N * K * 2          # the unpacked product streams at M <= 32
    assert hts.hts_gemm_workspace(d32, 33) == N * K * 2 + _r256(5 * 33 * N * 4)
    # HTS_DECODE_MAX_M lowers the streaming range: M = 17 is then split
    monkeypatch.setenv("HTS_DECODE_MAX_M", "16")
    assert hts.hts_gemm_workspace(d, 17) == _r256(5 * 17 * N * 4)
    monkeypatch.delenv("HTS_DECODE_MAX_M")
    # override: a forced count
    monkeypatch.setenv("HTS_PREFILL_SPLIT", "3")
    assert hts.hts_gemm_workspace(d, 300) == _r256(3 * 300 * N * 4)


def test_noalloc_rejects_before_any_device_call():
    # the scratch maximum (64 MiB) and the argument checks come before any HIP call
    desc = hts.make_desc(11008, 4096, 32, 32, "bf16")
    L = hts.lib()
    st = L.hts_gemm_noalloc(ctypes.byref(desc), 16, 16, 16, 64, 16, 4096, 16, 11008, hts.HTS_F32, None)
    assert st == 6 and b"64" in L.hts_last_error()
    st = L.hts_gemm_noalloc(ctypes.byref(desc), 16, 16, 16, -1, 16, 4096, 16, 11008, hts.HTS_F32, None)
    assert st == 3
    assert L.hts_gemm_noalloc(None, 16, 16, 16, 1, 16, 4096, 16, 11008, hts.HTS_F32, None) == 1


def test_peak_library_exports_every_declared_symbol():
    # libhts_peak.so: the measured roofline denominators declared in include/hts_peak.h
    import tile_gemm_amd.peak as peak
    text = open(os.path.join(ROOT, "include", "hts_peak.h")).read()
    names = sorted(set(re.findall(r"^\s*(?:int|double)\s+(hts_\w+)\s*\(", text, re.M)))
    L = peak.lib()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(peak.EXPORTED) == names
    # algorithmic flops per instruction: kept multiply-adds only (sparse = half its dense K)
    assert [L.hts_peak_mfma_flops_per_instruction(k) for k in range(5)] == [16384.0, 16384.0, 16384.0, 32768.0, 65536.0]
    assert L.hts_peak_mfma_flops_per_instruction(9) == 0.0
    # invalid arguments are rejected before any launch
    assert L.hts_peak_mfma(0, 0, 1, 16, None) == 1
    assert L.hts_peak_stream_read(None, 1024, 16, 1, None) == 1
    assert L.hts_peak_onchip(0, None, 1 << 21, 1, 1, 16, None) == 1
    assert L.hts_peak_onchip(0, 16, 1024, 1, 1, 16, None) == 1
    assert L.hts_peak_onchip(0, 16, 1 << 21, 0, 1, 16, None) == 1

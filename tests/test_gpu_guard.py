"""Guard bands: every output the library writes is written whole, and nothing around it.

Each output (Y of every product path, the packed values and codes, an unpacked weight, the
workspace of split products and of the unpack + dense path) is a view into a larger device
buffer whose remaining bytes -- a band before, a band after, and for 2-D outputs the gap between
rows -- hold a canary bit pattern. After the call the bands must still hold it, and an output
whose elements cannot take that pattern (Y, the unpacked weight: it is a NaN, which no product or
finite weight produces) must hold none of it, i.e. be written whole. Packed bytes can take any
value, so for them only the bands are checked.
"""
import numpy as np
import pytest
import torch

import tile_gemm_amd as hts
import workloads as wl
from helpers import DEV, say

pytestmark = pytest.mark.gpu
PAD = 4096            # elements of band before and after
CANARY = {1: 0x7F, 2: 0x7E5A, 4: 0x7FC0DEAD}   # by element size: NaN bit patterns


def _bits_dtype(size):
    return {1: torch.uint8, 2: torch.int16, 4: torch.int32}[size]


def _canary_value(size):
    v = CANARY[size]
    return v - (1 << (8 * size)) if size > 1 and v >= (1 << (8 * size - 1)) else v


class Guarded:
    """rows x cols of `dtype` with leading dimension ld, inside canary bands."""

    def __init__(self, rows, cols, dtype, ld=None):
        self.rows, self.cols = rows, cols
        self.ld = cols if ld is None else ld
        self.size = torch.empty(0, dtype=dtype).element_size()
        n = 2 * PAD + rows * self.ld
        self.bits = torch.full((n,), _canary_value(self.size), dtype=_bits_dtype(self.size), device=DEV)
        self.view = self.bits.view(dtype)[PAD:PAD + rows * self.ld].view(rows, self.ld)[:, :cols]

    def check(self, what):
        torch.cuda.synchronize()
        b = self.bits.cpu()
        c = _canary_value(self.size)
        assert bool((b[:PAD] == c).all()), f"{what}: write before the output"
        assert bool((b[PAD + self.rows * self.ld:] == c).all()), f"{what}: write after the output"
        body = b[PAD:PAD + self.rows * self.ld].view(self.rows, self.ld)
        if self.ld > self.cols:
            assert bool((body[:, self.cols:] == c).all()), f"{what}: write between rows"
        assert not bool((body[:, :self.cols] == c).any()), f"{what}: part of the output not written"


def _layer(N, K, dtype, seed):
    g = np.random.default_rng(seed)
    W = wl.gaussian_bits((N, K), 0.02 if dtype != "fp8" else 1.0, dtype, g)
    return W, g


def _packed(W, dtype, m, bn, bk):
    return hts.pack(hts.tensor_from_bits(W, dtype, DEV), m, bn, bk)


PRODUCTS = [  # (N, K, M, dtype, tile, path)
    (512, 768, 1, "bf16", 128, "streaming"),
    (512, 768, 16, "bf16", 128, "streaming, X staged"),
    (512, 768, 24, "bf16", 128, "streaming, two X row groups"),
    (512, 768, 5, "f16", 64, "streaming, 64-wide tiles"),
    (512, 768, 300, "bf16", 128, "tiled, split"),
    (4096, 512, 1100, "bf16", 128, "tiled, unsplit"),
    (512, 768, 1, "fp8", 128, "8-bit streaming"),
    (512, 768, 300, "fp8", 128, "8-bit tiled"),
    (256, 512, 100, "bf16", 32, "32-wide tiles: unpack + dense"),
]


@pytest.mark.parametrize("N,K,M,dtype,tile,path", PRODUCTS, ids=[p[-1] for p in PRODUCTS])
def test_products_write_only_their_output(N, K, M, dtype, tile, path):
    W, g = _layer(N, K, dtype, N + K + M)
    X = wl.gaussian_bits((M, K), 1.0, dtype, g)
    m = (g.random((N // tile) * (K // tile)) < 0.5).astype(np.uint8)
    pw = _packed(W, dtype, m, tile, tile)
    Xt = hts.tensor_from_bits(X, dtype, DEV)
    say(f"[guard] {path} N={N} K={K} M={M}")
    ws_n = hts.hts_gemm_workspace(pw.desc, M)
    ws = Guarded(1, ws_n, torch.uint8) if ws_n else None
    Y = Guarded(M, N, torch.float32, ld=N + 40)
    hts.hts_gemm(pw.desc, pw.index, pw.values, pw.meta, Xt, Y.view, workspace=None if ws is None else ws.view[0],
                 M=M)
    Y.check(f"{path}: Y")
    if ws is not None:
        # the workspace may be used in part; only its bands must be intact
        torch.cuda.synchronize()
        b = ws.bits.cpu()
        assert bool((b[:PAD] == CANARY[1]).all()) and bool((b[PAD + ws_n:] == CANARY[1]).all()), \
            f"{path}: write outside the workspace"
    Y16 = Guarded(M, N, torch.bfloat16, ld=N + 8)
    hts.hts_gemm(pw.desc, pw.index, pw.values, pw.meta, Xt, Y16.view, workspace=None if ws is None else ws.view[0],
                 M=M)
    Y16.check(f"{path}: 16-bit Y")


@pytest.mark.parametrize("M", [1, 24, 300])
def test_gated_and_dense_and_noalloc_write_only_their_output(M):
    N, K = 512, 768
    W, g = _layer(N, K, "bf16", 7 + M)
    X = wl.gaussian_bits((M, K), 1.0, "bf16", g)
    G = wl.gaussian_bits((M, N), 1.0, "bf16", g)
    m = (g.random((N // 128) * (K // 128)) < 0.5).astype(np.uint8)
    pw = _packed(W, "bf16", m, 128, 128)
    Xt, Gt = hts.tensor_from_bits(X, "bf16", DEV), hts.tensor_from_bits(G, "bf16", DEV)
    ws_n = hts.hts_gemm_workspace(pw.desc, M)
    ws = torch.empty(max(ws_n, 16), dtype=torch.uint8, device=DEV)
    Y = Guarded(M, N, torch.bfloat16, ld=N + 16)
    hts.hts_gemm_silu_mul(pw.desc, pw.index, pw.values, pw.meta, Xt, Gt, Y.view, workspace=ws)
    Y.check(f"gated M={M}")
    Yd = Guarded(M, N, torch.float32, ld=N + 4)
    wsd_n = hts.hts_dense_gemm_workspace(Xt.dtype, M, N, K)
    wsd = torch.empty(max(wsd_n, 16), dtype=torch.uint8, device=DEV)
    hts.hts_dense_gemm(Xt, hts.tensor_from_bits(W, "bf16", DEV), Yd.view, workspace=wsd)
    Yd.check(f"dense M={M}")
    Yn = Guarded(M, N, torch.float32, ld=N + 4)
    hts.hts_gemm_noalloc(pw.desc, pw.index, pw.values, pw.meta, Xt, Yn.view)
    Yn.check(f"allocation-free M={M}")


@pytest.mark.parametrize("dtype,tile", [("bf16", 128), ("f16", 64), ("fp8", 128), ("bf16", 32)])
def test_pack_and_unpack_write_only_their_output(dtype, tile):
    N, K = 256, 512
    W, g = _layer(N, K, dtype, tile)
    m = (g.random((N // tile) * (K // tile)) < 0.5).astype(np.uint8)
    Wt = hts.tensor_from_bits(W, dtype, DEV)
    desc = hts.make_desc(N, K, tile, tile, Wt.dtype)
    index_np, sizes = hts.hts_pack_plan(desc, m)
    index = torch.from_numpy(index_np.view(np.int32).copy()).to(DEV)
    vb, mb = sizes["values_bytes"], sizes["meta_bytes"]
    values = Guarded(1, vb, torch.uint8)
    meta = Guarded(1, mb // 4, torch.int32) if mb else None
    say(f"[guard] pack {dtype} {tile}x{tile}: {vb} + {mb} bytes")
    hts.hts_pack(desc, index, Wt, None, values.view[0], None if meta is None else meta.view[0])
    torch.cuda.synchronize()
    vbits = values.bits.cpu()
    assert bool((vbits[:PAD] == CANARY[1]).all()) and bool((vbits[PAD + vb:] == CANARY[1]).all()), "pack: values"
    if meta is not None:
        mbits = meta.bits.cpu()
        c = _canary_value(4)
        assert bool((mbits[:PAD] == c).all()) and bool((mbits[PAD + mb // 4:] == c).all()), "pack: codes"
    Wout = Guarded(N, K, Wt.dtype, ld=K + 16)
    hts.hts_unpack(desc, index, values.view[0], None if meta is None else meta.view[0], Wout.view)
    Wout.check(f"unpack {dtype} {tile}x{tile}")

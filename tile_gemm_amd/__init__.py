"""Python binding of libhts: hybrid tile-sparse (dense / 2:4) linear layers on MI355X.

Argument marshalling only.  Every step runs in the HIP kernels of libhts.so
(built in-tree by ``tile_gemm_amd.build``); torch supplies device memory and the
current stream.  There is no fallback: if the library is missing or no GPU is
present, the calls raise.

Low-level functions carry the C names (``hts_pack_plan``, ``hts_pack``,
``hts_unpack``, ``hts_gemm``, ``hts_dense_gemm``, ...); ``pack``, ``gemm``,
``unpack``, ``dense_gemm``, ``pack_masked``, ``wanda_tile_map`` and
``wanda_global_maps`` are tensor-level helpers built on them.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import numpy as np
import torch  # loads the HIP runtime that libhts binds to (same soname)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhts.so")

HTS_F16, HTS_BF16, HTS_F32, HTS_FP8_E4M3 = 0, 1, 2, 3
HTS_TILE_DENSE, HTS_TILE_SPARSE24 = 0, 1
STATUS_NAMES = {0: "HTS_OK", 1: "HTS_ERR_INVALID_ARG", 2: "HTS_ERR_DTYPE", 3: "HTS_ERR_SHAPE",
                4: "HTS_ERR_ALIGN", 5: "HTS_ERR_MAP", 6: "HTS_ERR_WORKSPACE", 7: "HTS_ERR_UNSUPPORTED",
                8: "HTS_ERR_HIP"}


class HTSError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class hts_desc(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int64), ("K", ctypes.c_int64), ("bn", ctypes.c_int32), ("bk", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class hts_sizes(ctypes.Structure):
    _fields_ = [("values_bytes", ctypes.c_uint64), ("meta_bytes", ctypes.c_uint64),
                ("index_bytes", ctypes.c_uint64), ("n_sparse", ctypes.c_int64)]


_VP = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SIGS = {
    "hts_abi_version": (ctypes.c_uint32, []),
    "hts_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "hts_last_error": (ctypes.c_char_p, []),
    "hts_pack_plan": (ctypes.c_int, [ctypes.POINTER(hts_desc), _VP, _VP, ctypes.POINTER(hts_sizes)]),
    "hts_pack": (ctypes.c_int, [ctypes.POINTER(hts_desc), _VP, _VP, _I64, _VP, _VP, _VP, _VP]),
    "hts_pack_masked": (ctypes.c_int, [ctypes.POINTER(hts_desc), _VP, _VP, _I64, _VP, _I64, _VP, _VP, _VP, _VP]),
    "hts_unpack": (ctypes.c_int, [ctypes.POINTER(hts_desc), _VP, _VP, _VP, _VP, _I64, _VP]),
    "hts_gemm_workspace": (ctypes.c_int, [ctypes.POINTER(hts_desc), _I64, ctypes.POINTER(ctypes.c_size_t)]),
    "hts_gemm": (ctypes.c_int, [ctypes.POINTER(hts_desc), _VP, _VP, _VP, _I64, _VP, _I64, _VP, _I64, _I32,
                                _VP, ctypes.c_size_t, _VP]),
    "hts_gemm_noalloc": (ctypes.c_int, [ctypes.POINTER(hts_desc), _VP, _VP, _VP, _I64, _VP, _I64, _VP, _I64, _I32,
                                        _VP]),
    "hts_gemm_silu_mul": (ctypes.c_int, [ctypes.POINTER(hts_desc), _VP, _VP, _VP, _I64, _VP, _I64, _VP, _I64, _VP,
                                         _I64, _I32, _VP, ctypes.c_size_t, _VP]),
    "hts_dense_gemm": (ctypes.c_int, [_I32, _I64, _I64, _I64, _VP, _I64, _VP, _I64, _VP, _I64, _I32, _VP,
                                      ctypes.c_size_t, _VP]),
    "hts_dense_gemm_workspace": (ctypes.c_int, [_I32, _I64, _I64, _I64, ctypes.POINTER(ctypes.c_size_t)]),
    "hts_silu_mul": (ctypes.c_int, [_I32, _I64, _I64, _VP, _I64, _VP, _I64, _VP, _I64, _VP]),
    "hts_col_norms": (ctypes.c_int, [_I32, _I64, _I64, _VP, _I64, _VP, _VP]),
    "hts_wanda_tile_cost": (ctypes.c_int, [ctypes.POINTER(hts_desc), _VP, _I64, _VP, _VP, _VP]),
    "hts_wanda_map": (ctypes.c_int, [_I64, _VP, _I64, _VP, _VP]),
}
EXPORTED = tuple(_SIGS)

_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """The loaded libhts.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m tile_gemm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != 0:
        raise HTSError(status, lib().hts_last_error().decode())


def _dt(t) -> int:
    m = {torch.float16: HTS_F16, torch.bfloat16: HTS_BF16, torch.float32: HTS_F32,
         torch.float8_e4m3fn: HTS_FP8_E4M3,
         "f16": HTS_F16, "bf16": HTS_BF16, "f32": HTS_F32, "fp8": HTS_FP8_E4M3}
    if t not in m:
        raise HTSError(2, f"unsupported element type {t}")
    return m[t]


def _torch_dt(code: int):
    return {HTS_F16: torch.float16, HTS_BF16: torch.bfloat16, HTS_F32: torch.float32,
            HTS_FP8_E4M3: torch.float8_e4m3fn}[code]


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def make_desc(N: int, K: int, bn: int, bk: int, dtype) -> hts_desc:
    return hts_desc(N, K, bn, bk, _dt(dtype), 0)


# --------------------------------------------------------------------------
# the C entry points, one to one
# --------------------------------------------------------------------------

def hts_abi_version() -> int:
    return lib().hts_abi_version()


def hts_status_string(status: int) -> str:
    return lib().hts_status_string(status).decode()


def hts_pack_plan(desc: hts_desc, tile_map: np.ndarray):
    """Host-side plan: (index uint32[T,4] numpy, sizes dict)."""
    tmap = np.ascontiguousarray(tile_map, dtype=np.uint8).ravel()
    T = 0
    if desc.bn > 0 and desc.bk > 0 and desc.N > 0 and desc.K > 0 and desc.N % desc.bn == 0 \
            and desc.K % desc.bk == 0:
        T = (desc.N // desc.bn) * (desc.K // desc.bk)
        if tmap.size != T:   # the library reads exactly T entries
            raise HTSError(3, f"tile map has {tmap.size} entries, the grid has {T}")
    # (an invalid descriptor is rejected by the library before the map is read)
    index = np.zeros((max(T, 1), 4), dtype=np.uint32)
    sizes = hts_sizes()
    _check(lib().hts_pack_plan(ctypes.byref(desc), tmap.ctypes.data, index.ctypes.data, ctypes.byref(sizes)))
    return index[:T], {"values_bytes": sizes.values_bytes, "meta_bytes": sizes.meta_bytes,
                       "index_bytes": sizes.index_bytes, "n_sparse": sizes.n_sparse}


def hts_pack(desc, index, W, col_scale, values, meta, ldw=None, stream=None) -> None:
    _check(lib().hts_pack(ctypes.byref(desc), _ptr(index), _ptr(W), W.stride(0) if ldw is None else ldw,
                          _ptr(col_scale), _ptr(values), _ptr(meta), _stream(stream)))


def hts_pack_masked(desc, index, W, mask, values, meta, malformed=None, ldw=None, ldm=None,
                    stream=None) -> None:
    _check(lib().hts_pack_masked(ctypes.byref(desc), _ptr(index), _ptr(W), W.stride(0) if ldw is None else ldw,
                                 _ptr(mask), mask.stride(0) if ldm is None else ldm, _ptr(values), _ptr(meta),
                                 _ptr(malformed), _stream(stream)))


def hts_unpack(desc, index, values, meta, W_out, ldw=None, stream=None) -> None:
    _check(lib().hts_unpack(ctypes.byref(desc), _ptr(index), _ptr(values), _ptr(meta), _ptr(W_out),
                            W_out.stride(0) if ldw is None else ldw, _stream(stream)))


def hts_gemm_workspace(desc, M: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().hts_gemm_workspace(ctypes.byref(desc), M, ctypes.byref(n)))
    return n.value


def hts_gemm(desc, index, values, meta, X, Y, y_dtype=None, workspace=None, stream=None, M=None) -> None:
    M = X.shape[0] if M is None else M
    yd = _dt(Y.dtype) if y_dtype is None else y_dtype
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().hts_gemm(ctypes.byref(desc), _ptr(index), _ptr(values), _ptr(meta), M, _ptr(X), X.stride(0),
                          _ptr(Y), Y.stride(0), yd, _ptr(workspace), ws_bytes, _stream(stream)))


def hts_gemm_noalloc(desc, index, values, meta, X, Y, y_dtype=None, stream=None, M=None) -> None:
    M = X.shape[0] if M is None else M
    yd = _dt(Y.dtype) if y_dtype is None else y_dtype
    _check(lib().hts_gemm_noalloc(ctypes.byref(desc), _ptr(index), _ptr(values), _ptr(meta), M, _ptr(X), X.stride(0),
                                  _ptr(Y), Y.stride(0), yd, _stream(stream)))


def hts_gemm_silu_mul(desc, index, values, meta, X, G, Y, y_dtype=None, workspace=None, stream=None) -> None:
    M = X.shape[0]
    yd = _dt(Y.dtype) if y_dtype is None else y_dtype
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().hts_gemm_silu_mul(ctypes.byref(desc), _ptr(index), _ptr(values), _ptr(meta), M, _ptr(X),
                                   X.stride(0), _ptr(G), G.stride(0), _ptr(Y), Y.stride(0), yd, _ptr(workspace),
                                   ws_bytes, _stream(stream)))


def hts_dense_gemm_workspace(dtype, M: int, N: int, K: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().hts_dense_gemm_workspace(_dt(dtype), M, N, K, ctypes.byref(n)))
    return n.value


def hts_dense_gemm(X, W, Y, workspace=None, stream=None) -> None:
    M, K = X.shape
    N = W.shape[0]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().hts_dense_gemm(_dt(X.dtype), M, N, K, _ptr(X), X.stride(0), _ptr(W), W.stride(0), _ptr(Y),
                                Y.stride(0), _dt(Y.dtype), _ptr(workspace), ws_bytes, _stream(stream)))


def hts_col_norms(X, out, stream=None) -> None:
    rows, K = X.shape
    _check(lib().hts_col_norms(_dt(X.dtype), rows, K, _ptr(X), X.stride(0), _ptr(out), _stream(stream)))


def hts_silu_mul(G, U, H, stream=None) -> None:
    M, N = G.shape
    _check(lib().hts_silu_mul(_dt(G.dtype), M, N, _ptr(G), G.stride(0), _ptr(U), U.stride(0), _ptr(H), H.stride(0),
                              _stream(stream)))


def silu_mul(G: torch.Tensor, U: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """H = silu(G) * U (the gated-MLP step between the up / gate and down projections)."""
    if out is None:
        out = torch.empty_like(G)
    hts_silu_mul(G, U, out, stream=stream)
    return out


def hts_wanda_tile_cost(desc, W, col_scale, cost, stream=None) -> None:
    _check(lib().hts_wanda_tile_cost(ctypes.byref(desc), _ptr(W), W.stride(0), _ptr(col_scale), _ptr(cost),
                                     _stream(stream)))


def hts_wanda_map(cost, n_sparse: int, tile_map, stream=None) -> None:
    _check(lib().hts_wanda_map(cost.numel(), _ptr(cost), n_sparse, _ptr(tile_map), _stream(stream)))


# --------------------------------------------------------------------------
# tensor-level helpers
# --------------------------------------------------------------------------

@dataclasses.dataclass
class PackedWeight:
    """A packed hybrid weight on the device: values, metadata and the tile index."""
    desc: hts_desc
    index: torch.Tensor      # int32[T,4] on device (uint32 records)
    values: torch.Tensor     # int16[...] raw 16-bit values
    meta: torch.Tensor       # int32[...] metadata words
    sizes: dict
    tile_map: np.ndarray

    @property
    def N(self) -> int:
        return self.desc.N

    @property
    def K(self) -> int:
        return self.desc.K

    @property
    def dtype(self):
        return _torch_dt(self.desc.dtype)

    @property
    def packed_bytes(self) -> int:
        return int(self.sizes["values_bytes"] + self.sizes["meta_bytes"] + self.sizes["index_bytes"])

    def save(self, path: str) -> None:
        """Write this packed weight to a versioned, checksummed file (see ``packed_io``)."""
        from . import packed_io
        packed_io.save(self, path)

    @staticmethod
    def load(path: str, device="cuda") -> "PackedWeight":
        """Read a file written by ``save`` onto ``device`` without packing again."""
        from . import packed_io
        return packed_io.load(path, device)


def _buffers_for(desc: hts_desc, sizes: dict, index_np: np.ndarray, device):
    index = torch.from_numpy(index_np.view(np.int32).copy()).to(device)
    if desc.dtype == HTS_FP8_E4M3:
        values = torch.empty(max(sizes["values_bytes"], 16), dtype=torch.uint8, device=device)
    else:
        values = torch.empty(max(sizes["values_bytes"] // 2, 8), dtype=torch.int16, device=device)
    meta = torch.empty(max(sizes["meta_bytes"] // 4, 4), dtype=torch.int32, device=device)
    return index, values, meta, sizes


def _device_buffers(desc: hts_desc, tile_map: np.ndarray, device):
    index_np, sizes = hts_pack_plan(desc, tile_map)
    return _buffers_for(desc, sizes, index_np, device)


def pack(W: torch.Tensor, tile_map: np.ndarray, bn: int, bk: int,
         col_scale: Optional[torch.Tensor] = None, stream=None) -> PackedWeight:
    """Pack a row-major W[N,K] (16-bit, or 8-bit E4M3) on the GPU under a host tile map (uint8,
    row-major tiles)."""
    N, K = W.shape
    desc = make_desc(N, K, bn, bk, W.dtype)
    index, values, meta, sizes = _device_buffers(desc, tile_map, W.device)
    hts_pack(desc, index, W, col_scale, values, meta, stream=stream)
    return PackedWeight(desc, index, values, meta, sizes, np.asarray(tile_map, dtype=np.uint8).ravel().copy())


def pack_masked(W: torch.Tensor, tile_map: np.ndarray, mask: torch.Tensor, bn: int, bk: int,
                stream=None):
    """Pack W with the 2:4 pairs a device uint8 keep mask [N,K] marks (nonzero = keep).

    Returns (PackedWeight, malformed) where malformed is a device uint32 tensor holding the number
    of groups in 2:4 tiles that do not mark exactly two weights."""
    N, K = W.shape
    if mask.dtype != torch.uint8 or tuple(mask.shape) != (N, K):
        raise HTSError(1, "mask must be a uint8 tensor of the shape of W")
    desc = make_desc(N, K, bn, bk, W.dtype)
    index, values, meta, sizes = _device_buffers(desc, tile_map, W.device)
    malformed = torch.empty(1, dtype=torch.int32, device=W.device)
    hts_pack_masked(desc, index, W, mask, values, meta, malformed, stream=stream)
    return (PackedWeight(desc, index, values, meta, sizes, np.asarray(tile_map, dtype=np.uint8).ravel().copy()),
            malformed)


def unpack(pw: PackedWeight, stream=None) -> torch.Tensor:
    W = torch.empty((pw.N, pw.K), dtype=pw.dtype, device=pw.values.device)
    hts_unpack(pw.desc, pw.index, pw.values, pw.meta, W, stream=stream)
    return W


def gemm(X: torch.Tensor, pw: PackedWeight, out_dtype=None, out: Optional[torch.Tensor] = None,
         stream=None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y[M,N] = X[M,K] . mask(W)^T from the packed weight (fp32 accumulation).  The workspace the
    library asks for (the unpacked weight of 32-wide tiles above the streaming range, the parts of a split
    product) is allocated here when none is given."""
    M = X.shape[0]
    if out is None:
        out = torch.empty((M, pw.N), dtype=out_dtype or _default_out(X.dtype), device=X.device)
    if workspace is None:
        nbytes = hts_gemm_workspace(pw.desc, M)
        if nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=X.device)
    hts_gemm(pw.desc, pw.index, pw.values, pw.meta, X, out, workspace=workspace, stream=stream)
    return out


def gemm_silu_mul(X: torch.Tensor, pw: PackedWeight, G: torch.Tensor, out: Optional[torch.Tensor] = None,
                  stream=None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = silu(G) * (X . mask(W)^T): the product with the gated-MLP step in its output stage.  G
    and Y share a type (the output type); G may be Y."""
    M = X.shape[0]
    if G.shape != (M, pw.N):
        raise ValueError(f"G has shape {tuple(G.shape)}, expected {(M, pw.N)}")
    if out is None:
        out = torch.empty((M, pw.N), dtype=G.dtype, device=X.device)
    if out.dtype != G.dtype:
        raise ValueError("G and the output must share a type")
    if workspace is None:
        nbytes = hts_gemm_workspace(pw.desc, M)
        if nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=X.device)
    hts_gemm_silu_mul(pw.desc, pw.index, pw.values, pw.meta, X, G, out, workspace=workspace, stream=stream)
    return out


def _default_out(dt):
    """Output type when none is given: the input type, fp32 for 8-bit inputs."""
    return torch.float32 if dt == torch.float8_e4m3fn else dt


def dense_gemm(X: torch.Tensor, W: torch.Tensor, out_dtype=None, out: Optional[torch.Tensor] = None,
               stream=None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The same-library dense product Y = X . W^T (no tile index); the workspace of a split
    product is allocated here when none is given."""
    if out is None:
        out = torch.empty((X.shape[0], W.shape[0]), dtype=out_dtype or _default_out(X.dtype), device=X.device)
    if workspace is None:
        nbytes = hts_dense_gemm_workspace(X.dtype, X.shape[0], W.shape[0], X.shape[1])
        if nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=X.device)
    hts_dense_gemm(X, W, out, workspace=workspace, stream=stream)
    return out


def col_norms(Xcal: torch.Tensor, stream=None) -> torch.Tensor:
    out = torch.empty(Xcal.shape[1], dtype=torch.float32, device=Xcal.device)
    hts_col_norms(Xcal, out, stream=stream)
    return out


def wanda_tile_map(W: torch.Tensor, col_scale: torch.Tensor, bn: int, bk: int, n_sparse: int,
                   stream=None) -> torch.Tensor:
    """Device uint8 tile map: the n_sparse tiles with the least dropped Wanda mass become 2:4."""
    N, K = W.shape
    desc = make_desc(N, K, bn, bk, W.dtype)
    T = (N // bn) * (K // bk)
    cost = torch.empty(T, dtype=torch.float64, device=W.device)
    hts_wanda_tile_cost(desc, W, col_scale, cost, stream=stream)
    m = torch.empty(T, dtype=torch.uint8, device=W.device)
    hts_wanda_map(cost, n_sparse, m, stream=stream)
    return m


def wanda_global_maps(Ws, col_scales, bn: int, bk: int, n_sparse: int, stream=None):
    """Device tile maps of several layers from one shared sparse-tile budget: the n_sparse tiles
    with the least dropped Wanda mass among all the layers' tiles become 2:4 (ties: layer order,
    then tile number).  The costs of all layers go into one device buffer, one slice per layer."""
    descs, Ts = [], []
    for W in Ws:
        N, K = W.shape
        descs.append(make_desc(N, K, bn, bk, W.dtype))
        Ts.append((N // bn) * (K // bk))
    cost = torch.empty(sum(Ts), dtype=torch.float64, device=Ws[0].device)
    off = 0
    for d, W, cs, T in zip(descs, Ws, col_scales, Ts):
        _check(lib().hts_wanda_tile_cost(ctypes.byref(d), _ptr(W), W.stride(0), _ptr(cs),
                                         ctypes.c_void_p(cost.data_ptr() + 8 * off), _stream(stream)))
        off += T
    m = torch.empty(sum(Ts), dtype=torch.uint8, device=Ws[0].device)
    hts_wanda_map(cost, n_sparse, m, stream=stream)
    return list(torch.split(m, Ts))


def tensor_from_bits(bits: np.ndarray, dtype: str, device) -> torch.Tensor:
    """A torch tensor (16-bit, or float8_e4m3fn for "fp8") holding exactly these bit patterns."""
    if dtype == "fp8":
        return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint8)).view(torch.float8_e4m3fn).to(device)
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).to(device)


def bits_from_tensor(t: torch.Tensor) -> np.ndarray:
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return t.detach().contiguous().view(torch.uint8).cpu().numpy()
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

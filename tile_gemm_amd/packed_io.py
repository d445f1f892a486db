"""Versioned files for packed hybrid weights (save once after packing, load without re-packing).

A file holds one packed weight exactly as the library stores it on the device: the descriptor,
the host tile map, the tile index, the packed values and the 2:4 metadata words. Nothing in it is
executable: the header is JSON, the sections are raw little-endian bytes.

Layout (format 1):

    offset 0   8 bytes   magic b"HTSPACK\\0"
    offset 8   uint32    format version (1)
    offset 12  uint32    header length H in bytes
    offset 16  H bytes   UTF-8 JSON header
    then       sections, each starting at a multiple of 64 bytes, in the order the header lists

The header records N, K, bn, bk, the element type by name, the packed sizes, the ABI version of
the library that wrote it, and for each section (tile_map, index, values, meta) its offset,
length and CRC-32. Loading checks the magic, the version, every length and CRC, and re-plans the
tile map with `hts_pack_plan`: the stored index and sizes must equal the plan bit for bit, so a
file whose map and index disagree is rejected before any device memory is touched.
"""
from __future__ import annotations

import json
import os
import struct
import zlib

import numpy as np
import torch

MAGIC = b"HTSPACK\0"
FORMAT_VERSION = 1
_ALIGN = 64
_DTYPE_NAMES = {0: "f16", 1: "bf16", 3: "fp8_e4m3"}


class PackedFileError(ValueError):
    """The file is not a packed weight this library can load (wrong magic, version, length,
    checksum, or an index that does not match its tile map)."""


def _host_bytes(t: torch.Tensor, nbytes: int) -> bytes:
    flat = t.detach().reshape(-1).view(torch.uint8)
    if flat.numel() < nbytes:
        raise PackedFileError(f"buffer holds {flat.numel()} bytes, the packed size is {nbytes}")
    return flat[:nbytes].cpu().numpy().tobytes()


def save(pw, path: str) -> None:
    """Write `pw` (a PackedWeight) to `path`. The device buffers are copied to the host first;
    the caller's stream work on them must be complete (this synchronises the device)."""
    import tile_gemm_amd as hts
    d = pw.desc
    if d.dtype not in _DTYPE_NAMES:
        raise PackedFileError(f"element type code {d.dtype} cannot be saved")
    if pw.values.is_cuda:
        torch.cuda.synchronize(pw.values.device)
    sz = pw.sizes
    sections = [
        ("tile_map", np.ascontiguousarray(pw.tile_map, dtype=np.uint8).tobytes()),
        ("index", _host_bytes(pw.index, int(sz["index_bytes"]))),
        ("values", _host_bytes(pw.values, int(sz["values_bytes"]))),
        ("meta", _host_bytes(pw.meta, int(sz["meta_bytes"]))),
    ]
    header = {
        "format": FORMAT_VERSION, "abi": int(hts.hts_abi_version()),
        "N": int(d.N), "K": int(d.K), "bn": int(d.bn), "bk": int(d.bk), "dtype": _DTYPE_NAMES[d.dtype],
        "values_bytes": int(sz["values_bytes"]), "meta_bytes": int(sz["meta_bytes"]),
        "index_bytes": int(sz["index_bytes"]), "n_sparse": int(sz["n_sparse"]), "sections": [],
    }
    # offsets depend on the header length, which depends on the offsets: fix the header size by
    # padding it to a multiple of the alignment and iterate until it is stable
    hlen = 0
    for _ in range(4):
        off = (16 + hlen + _ALIGN - 1) // _ALIGN * _ALIGN
        header["sections"] = []
        for name, blob in sections:
            header["sections"].append({"name": name, "offset": off, "bytes": len(blob),
                                       "crc32": zlib.crc32(blob) & 0xFFFFFFFF})
            off = (off + len(blob) + _ALIGN - 1) // _ALIGN * _ALIGN
        text = json.dumps(header, sort_keys=True).encode()
        if len(text) <= hlen:
            break
        hlen = (len(text) + _ALIGN - 1) // _ALIGN * _ALIGN
    text = text.ljust(hlen, b" ")
    tmp = f"{path}.tmp{os.getpid()}"
    with open(tmp, "wb") as f:
        f.write(MAGIC + struct.pack("<II", FORMAT_VERSION, hlen) + text)
        for (name, blob), s in zip(sections, header["sections"]):
            f.write(b"\0" * (s["offset"] - f.tell()))
            f.write(blob)
    os.replace(tmp, path)   # a reader never sees a half-written file


def load(path: str, device="cuda"):
    """Read a packed weight written by `save` onto `device`; raises PackedFileError if the file
    is malformed or does not match its own tile map."""
    import tile_gemm_amd as hts
    with open(path, "rb") as f:
        raw = f.read()
    if len(raw) < 16 or raw[:8] != MAGIC:
        raise PackedFileError(f"{path}: not a packed-weight file")
    version, hlen = struct.unpack("<II", raw[8:16])
    if version != FORMAT_VERSION:
        raise PackedFileError(f"{path}: format version {version}, this library reads {FORMAT_VERSION}")
    if 16 + hlen > len(raw):
        raise PackedFileError(f"{path}: truncated header")
    try:
        h = json.loads(raw[16:16 + hlen].decode())
    except (UnicodeDecodeError, json.JSONDecodeError) as e:
        raise PackedFileError(f"{path}: unreadable header ({e})") from None
    if h.get("format") != FORMAT_VERSION:
        raise PackedFileError(f"{path}: header format {h.get('format')}")
    names = {v: k for k, v in _DTYPE_NAMES.items()}
    if h.get("dtype") not in names:
        raise PackedFileError(f"{path}: element type {h.get('dtype')!r}")
    blobs = {}
    for s in h.get("sections", []):
        a, n = int(s["offset"]), int(s["bytes"])
        if a < 16 + hlen or a + n > len(raw):
            raise PackedFileError(f"{path}: section {s['name']} lies outside the file")
        blob = raw[a:a + n]
        if zlib.crc32(blob) & 0xFFFFFFFF != int(s["crc32"]):
            raise PackedFileError(f"{path}: checksum of section {s['name']} does not match")
        blobs[s["name"]] = blob
    for name in ("tile_map", "index", "values", "meta"):
        if name not in blobs:
            raise PackedFileError(f"{path}: section {name} missing")
    desc = hts.make_desc(int(h["N"]), int(h["K"]), int(h["bn"]), int(h["bk"]),
                         {"f16": "f16", "bf16": "bf16", "fp8_e4m3": "fp8"}[h["dtype"]])
    tile_map = np.frombuffer(blobs["tile_map"], dtype=np.uint8).copy()
    try:
        index_np, sizes = hts.hts_pack_plan(desc, tile_map)
    except hts.HTSError as e:
        raise PackedFileError(f"{path}: descriptor or tile map rejected ({e})") from None
    for k in ("values_bytes", "meta_bytes", "index_bytes", "n_sparse"):
        if int(sizes[k]) != int(h[k]):
            raise PackedFileError(f"{path}: {k} is {h[k]}, the tile map gives {sizes[k]}")
    if index_np.tobytes() != blobs["index"]:
        raise PackedFileError(f"{path}: the stored tile index does not match the tile map")
    for k, name in (("values_bytes", "values"), ("meta_bytes", "meta")):
        if len(blobs[name]) != int(sizes[k]):
            raise PackedFileError(f"{path}: section {name} holds {len(blobs[name])} bytes, expected {sizes[k]}")
    index, values, meta, _ = hts._buffers_for(desc, sizes, index_np, device)
    for t, blob in ((values, blobs["values"]), (meta, blobs["meta"])):
        if blob:
            src = torch.frombuffer(bytearray(blob), dtype=torch.uint8)
            t.reshape(-1).view(torch.uint8)[:len(blob)].copy_(src)
    return hts.PackedWeight(desc, index, values, meta, sizes, tile_map)

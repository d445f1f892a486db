"""Benchmark of the hybrid tile-sparse (dense / 2:4) linear layer on one MI355X.

Default workload: the LLaMA-2-7B MLP up-projection W[11008, 4096] bf16, 128x128
tiles, 25 % of the tiles 2:4 (12.5 % overall sparsity), X ~ N(0,1) bf16.
A step is one hybrid product at M = 2048 (the prefill shape) with the packed
weight already resident in HBM; `value` is its algorithmic throughput
2*M*(kept weights)/t.  The same run also measures the decode shapes M = 1 and
M = 16 (HBM-bound; reported in GB/s of algorithmic bytes), the same-library
dense product on the same shapes (speedup), torch.matmul for context, pack and
unpack, and the CPU oracle on the host cores.

Weights and activations are synthetic (seeded Gaussian layers of the 7B shape);
packed-weight copies are rotated so the working set exceeds the 256 MB Infinity
Cache.  Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "fp8": 5000.0}   # dense MFMA, published
ROTATE_BYTES = 600 << 20       # > 2x the 256 MB Infinity Cache


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", default="7b_up", help="7b_up | 13b | sweep (other configs are parity cases)")
    p.add_argument("--layer", type=int, default=0)
    p.add_argument("--quick", action="store_true", help="profiling run: a few launches of each kernel, no oracle")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline leg")
    p.add_argument("--no-block", action="store_true", help="skip the decoder-block leg")
    p.add_argument("--no-fp8", action="store_true", help="skip the 8-bit (E4M3) leg")
    p.add_argument("--no-tiles", action="store_true", help="skip the tile-size leg")
    p.add_argument("--no-shard", action="store_true", help="skip the one-GPU-share (8-way N split) leg")
    p.add_argument("--no-mid", action="store_true", help="skip the moderate-M (17..256) leg")
    p.add_argument("--no-13b", action="store_true", help="skip the 13B-shaped layers")
    p.add_argument("--no-sweep", action="store_true", help="skip the sparsity sweep")
    p.add_argument("--no-decompress", action="store_true", help="skip the expansion-fallback leg")
    p.add_argument("--no-peaks", action="store_true", help="skip the measured-peak microbenchmarks")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run three plain 256 MiB device copies (scale for the FETCH_SIZE / WRITE_SIZE counters)")
    return p.parse_args()


# Sources whose change invalidates a recorded counter measurement of the tiled kernel.
PREFILL_SOURCES = ["tile_gemm_amd/csrc/gemm_prefill.hip", "tile_gemm_amd/csrc/prefill_common.h",
                   "tile_gemm_amd/csrc/gemm_common.h", "tile_gemm_amd/csrc/device_common.h"]
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "gemm_prefill_7b_up_m2048_hbm_traffic.md")


def prefill_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in PREFILL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload_key: str):
    """HBM bytes per launch of the tiled kernel from the committed counter summary, or None when
    there is none for this workload or the kernel sources changed since it was taken."""
    try:
        with open(TRAFFIC_RECORD) as fh:
            text = fh.read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        line = line.strip().strip("`")
        if ":" in line and line.split(":", 1)[0].strip() in ("source_hash", "workload_key", "traffic_bytes_per_launch"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("source_hash") != prefill_source_hash() or fields.get("workload_key") != workload_key:
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def run_fp8(hts, wl, dev, time_graph, time_launches, quick):
    """The 7B up-projection with 8-bit E4M3 weights and activations (prune then quantize), 25 % of
    the tiles 2:4: decode shapes (HBM-bound, graph-timed) and M = 2048, against the same-library
    dense 8-bit product.  Y is bf16."""
    import torch
    cfg = wl.config("7b_up_fp8")
    L = cfg.layers[0]
    W = hts.tensor_from_bits(wl.weight_bits(cfg, L), "fp8", dev)
    tmap = wl.tile_map(cfg, L)
    Xall = hts.tensor_from_bits(wl.activation_bits(cfg, L, max(cfg.Ms)), "fp8", dev)
    pw0 = hts.pack(W, tmap, L.bn, L.bk)
    torch.cuda.synchronize()
    packed = pw0.packed_bytes
    dense = L.N * L.K
    n_rot = max(2, -(-ROTATE_BYTES // packed))
    pws = [pw0] + [hts.PackedWeight(pw0.desc, pw0.index.clone(), pw0.values.clone(), pw0.meta.clone(),
                                    pw0.sizes, pw0.tile_map) for _ in range(n_rot - 1)]
    n_rot_d = max(2, -(-ROTATE_BYTES // dense))
    Ws = [W] + [W.clone() for _ in range(n_rot_d - 1)]
    kept = L.N * L.K - int(tmap.sum()) * L.bn * L.bk // 2
    out = {"workload": f"{L.name}: W[{L.N}x{L.K}] E4M3, 128x128 tiles, {int(tmap.sum())}/{L.T} tiles 2:4, "
                       "X E4M3, Y bf16", "packed_bytes": packed, "dense_bytes": dense, "decode": []}
    for M in [m for m in cfg.Ms if m <= 16]:
        Xm = Xall[:M].contiguous()
        Ys = [torch.empty((M, L.N), dtype=torch.bfloat16, device=dev) for _ in range(max(n_rot, n_rot_d))]
        per = 4 if quick else 8 * max(n_rot, n_rot_d)
        t_h = time_graph(lambda i: hts.gemm(Xm, pws[i % n_rot], out=Ys[i % n_rot]), per, 2 if quick else 25)
        t_d = time_graph(lambda i: hts.dense_gemm(Xm, Ws[i % n_rot_d], out=Ys[i % n_rot_d]), per, 2 if quick else 25)
        alg = packed + M * L.K + 2 * M * L.N
        out["decode"].append({"M": M, "us": round(t_h * 1e6, 3), "GB/s": round(alg / t_h / 1e9, 1),
                              "frac_hbm": round(alg / t_h / 1e9 / HBM_PEAK_GBS, 4), "algorithmic_bytes": alg,
                              "dense_same_library_us": round(t_d * 1e6, 3), "speedup_vs_dense": round(t_d / t_h, 3)})
    M = max(cfg.Ms)
    Ys = [torch.empty((M, L.N), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    n = 10 if quick else 50
    t_h = time_launches(lambda i: hts.gemm(Xall, pws[i % n_rot], out=Ys[i % 2]), n)
    t_d = time_launches(lambda i: hts.dense_gemm(Xall, Ws[i % n_rot_d], out=Ys[i % 2]), n)
    out["prefill"] = {"M": M, "us": round(t_h * 1e6, 2), "TFLOP/s": round(2.0 * M * kept / t_h / 1e12, 1),
                      "frac_mfma_fp8": round(2.0 * M * kept / t_h / 1e12 / MFMA_PEAK_TFLOPS["fp8"], 4),
                      "dense_same_library_us": round(t_d * 1e6, 2),
                      "dense_same_library_TFLOP/s": round(2.0 * M * L.N * L.K / t_d / 1e12, 1),
                      "speedup_vs_dense": round(t_d / t_h, 3)}
    return out


def run_tile_sizes(hts, wl, dev, time_graph, time_launches, quick):
    """Tile-size ablation on the 7B up-projection (bf16, 25 % of the tiles 2:4 at every size):
    128x128, 64x64 and 32x32 maps at M = 1, 16 (graph-timed) and 2048 (32x32 at M = 2048 runs
    unpack + the dense product through the workspace)."""
    import torch
    cfg = wl.config("7b_up")
    L = cfg.layers[0]
    W = hts.tensor_from_bits(wl.weight_bits(cfg, L), L.dtype, dev)
    Xall = hts.tensor_from_bits(wl.activation_bits(cfg, L, max(cfg.Ms)), L.dtype, dev)
    out = {}
    for t in (128, 64, 32):
        T = (L.N // t) * (L.K // t)
        m = wl.exact_map(T, int(round(0.25 * T)), wl.rng(cfg.cfg_id, L.layer_id, wl.TAG_MAP, (t,)))
        pw0 = hts.pack(W, m, t, t)
        torch.cuda.synchronize()
        n_rot = max(2, -(-ROTATE_BYTES // pw0.packed_bytes))
        pws = [pw0] + [hts.PackedWeight(pw0.desc, pw0.index.clone(), pw0.values.clone(), pw0.meta.clone(),
                                        pw0.sizes, pw0.tile_map) for _ in range(n_rot - 1)]
        row = {"packed_bytes": pw0.packed_bytes}
        for M in (1, 16):
            Xm = Xall[:M].contiguous()
            Ys = [torch.empty((M, L.N), dtype=torch.bfloat16, device=dev) for _ in range(n_rot)]
            tm = time_graph(lambda i: hts.gemm(Xm, pws[i % n_rot], out=Ys[i % n_rot]), 4 if quick else 8 * n_rot,
                            2 if quick else 20)
            row[f"M{M}_us"] = round(tm * 1e6, 2)
        M = max(cfg.Ms)
        Y = torch.empty((M, L.N), dtype=torch.bfloat16, device=dev)
        nbytes = hts.hts_gemm_workspace(pw0.desc, M)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None
        tm = time_launches(lambda i: hts.gemm(Xall, pws[i % n_rot], out=Y, workspace=ws), 5 if quick else 30)
        row[f"M{M}_us"] = round(tm * 1e6, 1)
        row["path_at_M2048"] = "unpack + dense product (workspace)" if nbytes else "tiled hybrid kernel"
        out[f"{t}x{t}"] = row
        del pws, pw0
    return out


def run_mid_m(hts, wl, dev, time_graph, quick):
    """The 7B up-projection between decode and full prefill (M = 17 .. 256).  Up to M = 32 the
    streaming kernel feeds each weight fragment to two groups of 16 X rows; above, the tiled
    product has few output blocks and is split over K (the workspace holds the parts).
    Graph-timed with rotated weights; the same-library dense product and torch for comparison."""
    import torch
    cfg = wl.config("7b_up")
    L = cfg.layers[0]
    m = wl.tile_map(cfg, L)
    W = hts.tensor_from_bits(wl.weight_bits(cfg, L), L.dtype, dev)
    Xall = hts.tensor_from_bits(wl.activation_bits(cfg, L, max(cfg.Ms)), L.dtype, dev)
    pw0 = hts.pack(W, m, L.bn, L.bk)
    torch.cuda.synchronize()
    n_rot = max(2, -(-ROTATE_BYTES // pw0.packed_bytes))
    pws = [pw0] + [hts.PackedWeight(pw0.desc, pw0.index.clone(), pw0.values.clone(), pw0.meta.clone(),
                                    pw0.sizes, pw0.tile_map) for _ in range(n_rot - 1)]
    n_rd = max(2, -(-ROTATE_BYTES // (2 * L.N * L.K)))
    Wd = [W] + [W.clone() for _ in range(n_rd - 1)]
    kept = L.N * L.K - int(m.sum()) * L.bn * L.bk // 2
    rows = []
    for M in (17, 32, 64, 128, 256):
        Xm = Xall[:M].contiguous()
        n = max(n_rot, n_rd)
        Ys = [torch.empty((M, L.N), dtype=torch.bfloat16, device=dev) for _ in range(n)]
        wsh = hts.hts_gemm_workspace(pw0.desc, M)
        wsd = hts.hts_dense_gemm_workspace(Xm.dtype, M, L.N, L.K)
        WSh = torch.empty(wsh, dtype=torch.uint8, device=dev) if wsh else None
        WSd = torch.empty(wsd, dtype=torch.uint8, device=dev) if wsd else None
        per, reps = (2, 2) if quick else (8 * n, 5)     # 8 launches per weight copy: graph launch cost amortized
        t_h = time_graph(lambda i: hts.gemm(Xm, pws[i % n_rot], out=Ys[i % n], workspace=WSh), per, reps)
        t_d = time_graph(lambda i: hts.dense_gemm(Xm, Wd[i % n_rd], out=Ys[i % n], workspace=WSd), per, reps)
        t_t = time_graph(lambda i: torch.matmul(Xm, Wd[i % n_rd].t(), out=Ys[i % n]), per, reps)
        rows.append({"M": M, "us": round(t_h * 1e6, 2), "TFLOP/s": round(2.0 * M * kept / t_h / 1e12, 1),
                     "weight_GB/s": round(pw0.packed_bytes / t_h / 1e9, 1), "workspace_bytes": wsh,
                     "dense_same_library_us": round(t_d * 1e6, 2), "torch_matmul_us": round(t_t * 1e6, 2),
                     "speedup_vs_dense": round(t_d / t_h, 3)})
    return rows


def run_shard(hts, wl, dev, time_graph, time_launches, quick):
    """One GPU's share of the 7B up-projection under 8-way column-parallel sharding: tile rows
    0..10 (N = 1408, K = 4096) with their part of the map, at M = 1, 16 (graph-timed) and 2048,
    against the same-library dense product and torch (hipBLASLt) on the same rows."""
    import torch
    cfg = wl.config("7b_up")
    L = cfg.layers[0]
    Tk = L.K // L.bk
    rows = 11
    Wb = np.ascontiguousarray(wl.weight_bits(cfg, L)[:rows * L.bn])
    m = np.ascontiguousarray(wl.tile_map(cfg, L).reshape(-1, Tk)[:rows].ravel())
    N = Wb.shape[0]
    W = hts.tensor_from_bits(Wb, L.dtype, dev)
    Xall = hts.tensor_from_bits(wl.activation_bits(cfg, L, max(cfg.Ms)), L.dtype, dev)
    pw0 = hts.pack(W, m, L.bn, L.bk)
    torch.cuda.synchronize()
    n_rot = max(2, -(-ROTATE_BYTES // pw0.packed_bytes))
    pws = [pw0] + [hts.PackedWeight(pw0.desc, pw0.index.clone(), pw0.values.clone(), pw0.meta.clone(),
                                    pw0.sizes, pw0.tile_map) for _ in range(n_rot - 1)]
    n_rd = max(2, -(-ROTATE_BYTES // (2 * N * L.K)))
    Wd = [W] + [W.clone() for _ in range(n_rd - 1)]
    out = {"workload": f"7B up-projection tile rows 0..{rows - 1}: W[{N}x{L.K}] bf16, {int(m.sum())}/{m.size} "
                       "tiles 2:4 (one GPU of an 8-way N split)",
           "packed_bytes": pw0.packed_bytes}
    for M in (1, 16, max(cfg.Ms)):
        Xm = Xall[:M].contiguous()
        n = max(n_rot, n_rd)
        Ys = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(n)]
        wsh = hts.hts_gemm_workspace(pw0.desc, M)
        wsd = hts.hts_dense_gemm_workspace(Xm.dtype, M, N, L.K)
        WSh = torch.empty(wsh, dtype=torch.uint8, device=dev) if wsh else None
        WSd = torch.empty(wsd, dtype=torch.uint8, device=dev) if wsd else None
        if M <= 16:
            per, reps = (4, 2) if quick else (8 * n_rot, 20)
            t_h = time_graph(lambda i: hts.gemm(Xm, pws[i % n_rot], out=Ys[i % n]), per, reps)
            t_d = time_graph(lambda i: hts.dense_gemm(Xm, Wd[i % n_rd], out=Ys[i % n]), per, reps)
            t_t = time_graph(lambda i: torch.matmul(Xm, Wd[i % n_rd].t(), out=Ys[i % n]), per, reps)
        else:
            reps = 5 if quick else 60
            t_h = time_launches(lambda i: hts.gemm(Xm, pws[i % n_rot], out=Ys[i % n], workspace=WSh), reps)
            t_d = time_launches(lambda i: hts.dense_gemm(Xm, Wd[i % n_rd], out=Ys[i % n], workspace=WSd), reps)
            t_t = time_launches(lambda i: torch.matmul(Xm, Wd[i % n_rd].t(), out=Ys[i % n]), reps)
        alg = pw0.packed_bytes + 2 * M * L.K + 2 * M * N
        flops = 2.0 * M * (N * L.K - int(m.sum()) * L.bn * L.bk // 2)    # kept weights only
        row = {"M": M, "us": round(t_h * 1e6, 2), "dense_same_library_us": round(t_d * 1e6, 2),
               "torch_matmul_us": round(t_t * 1e6, 2), "speedup_vs_dense": round(t_d / t_h, 3),
               "workspace_bytes": wsh}
        if M <= 16:
            row["GB/s"] = round(alg / t_h / 1e9, 1)
            row["frac_hbm"] = round(alg / t_h / (HBM_PEAK_GBS * 1e9), 4)
        else:
            row["TFLOP/s"] = round(flops / t_h / 1e12, 1)
        out[f"M{M}"] = row
    return out


def packed_copies(hts, pw0, n):
    """pw0 and n-1 device copies of it (rotation beyond the Infinity Cache)."""
    return [pw0] + [hts.PackedWeight(pw0.desc, pw0.index.clone(), pw0.values.clone(), pw0.meta.clone(),
                                     pw0.sizes, pw0.tile_map) for _ in range(n - 1)]


def run_layer(hts, wl, dev, time_graph, time_launches, quick, cfg, L, Ms):
    """One named layer at each M: the hybrid product against the same weight packed with an
    all-dense map (same kernels and storage order), the row-major same-library dense product and
    torch.matmul, every one timed the same way -- M <= 32 as HIP-graph replays of 8 launches per
    rotated weight copy, larger M as back-to-back launches (best of 3 windows) -- with weight
    copies rotated beyond the Infinity Cache.  M <= 16 is reported in GB/s of algorithmic bytes
    (packed weight + X + Y), larger M in TFLOP/s of kept multiply-adds."""
    import torch
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[L.dtype]
    W = hts.tensor_from_bits(wl.weight_bits(cfg, L), L.dtype, dev)
    tmap = wl.tile_map(cfg, L)
    Xall = hts.tensor_from_bits(wl.activation_bits(cfg, L, max(Ms)), L.dtype, dev)
    pw0 = hts.pack(W, tmap, L.bn, L.bk)
    pd0 = hts.pack(W, np.zeros_like(tmap), L.bn, L.bk)
    torch.cuda.synchronize()
    n_rot = max(2, -(-ROTATE_BYTES // pw0.packed_bytes))
    n_rd = max(2, -(-ROTATE_BYTES // (2 * L.N * L.K)))
    pws, pds = packed_copies(hts, pw0, n_rot), packed_copies(hts, pd0, n_rd)
    Ws = [W] + [W.clone() for _ in range(n_rd - 1)]
    ns = int(tmap.sum())
    kept = L.N * L.K - ns * L.bn * L.bk // 2
    rows = []
    for M in Ms:
        X = Xall[:M].contiguous()
        n = max(n_rot, n_rd)
        Ys = [torch.empty((M, L.N), dtype=tdt, device=dev) for _ in range(n if M <= 32 else 2)]
        ws = hts.hts_gemm_workspace(pw0.desc, M)
        WS = torch.empty(ws, dtype=torch.uint8, device=dev) if ws else None
        wd = hts.hts_dense_gemm_workspace(X.dtype, M, L.N, L.K)
        WSd = torch.empty(wd, dtype=torch.uint8, device=dev) if wd else None
        fns = {"hyb": lambda i: hts.gemm(X, pws[i % n_rot], out=Ys[i % len(Ys)], workspace=WS),
               "dpk": lambda i: hts.gemm(X, pds[i % n_rd], out=Ys[i % len(Ys)], workspace=WS),
               "den": lambda i: hts.dense_gemm(X, Ws[i % n_rd], out=Ys[i % len(Ys)], workspace=WSd),
               "mm": lambda i: torch.matmul(X, Ws[i % n_rd].t(), out=Ys[i % len(Ys)])}
        if M <= 32:
            per, reps = (4, 2) if quick else (8 * n, 10)
            t = {k: time_graph(f, per, reps) for k, f in fns.items()}
        else:
            t = {k: time_launches(f, 5 if quick else 30) for k, f in fns.items()}
        row = {"M": M, "us": round(t["hyb"] * 1e6, 2), "dense_packed_us": round(t["dpk"] * 1e6, 2),
               "dense_same_library_us": round(t["den"] * 1e6, 2), "torch_matmul_us": round(t["mm"] * 1e6, 2),
               "speedup_vs_dense_packed": round(t["dpk"] / t["hyb"], 3),
               "speedup_vs_dense": round(t["den"] / t["hyb"], 3)}
        if M <= 16:
            alg = pw0.packed_bytes + 2 * M * L.K + 2 * M * L.N
            row.update({"GB/s": round(alg / t["hyb"] / 1e9, 1), "frac_hbm": round(alg / t["hyb"] / 1e9 / HBM_PEAK_GBS, 4),
                        "algorithmic_bytes": alg})
        else:
            tf = 2.0 * M * kept / t["hyb"] / 1e12
            row.update({"TFLOP/s": round(tf, 1), "frac_mfma": round(tf / MFMA_PEAK_TFLOPS[L.dtype], 4),
                        "dense_equivalent_TFLOP/s": round(2.0 * M * L.N * L.K / t["hyb"] / 1e12, 1)})
        rows.append(row)
    out = {"layer": f"{L.name}: W[{L.N}x{L.K}] {L.dtype}, {L.bn}x{L.bk} tiles, {ns}/{L.T} tiles 2:4 "
                    f"({100.0 * 0.5 * ns / L.T:.1f}% sparsity)",
           "packed_bytes": pw0.packed_bytes, "rows": rows}
    del pws, pds, Ws
    return out


def run_13b(hts, wl, dev, time_graph, time_launches, quick):
    """The two 13B-shaped layers (5120x5120 and 13824x5120, half the tiles 2:4) at M = 1, 16, 4096."""
    cfg = wl.config("13b")
    return [run_layer(hts, wl, dev, time_graph, time_launches, quick, cfg, L, list(cfg.Ms)) for L in cfg.layers]


def run_sweep(hts, wl, dev, time_graph, time_launches, quick):
    """The 4096x4096 fp16 layer at sparse-tile fractions p = 0, .25, .5, .75, 1 (0-50% sparsity), M = 1
    and 2048, with the speed-up ceilings of the packed format (bytes at M = 1, kept flops at 2048)."""
    cfg = wl.config("sweep")
    out = []
    for L in cfg.layers:
        r = run_layer(hts, wl, dev, time_graph, time_launches, quick, cfg, L, list(cfg.Ms))
        p = int(wl.tile_map(cfg, L).sum()) / L.T
        r["p"] = p
        r["ceiling_bytes"] = round(2.0 / (2.0 - 0.875 * p), 3)
        r["ceiling_flops"] = round(1.0 / (1.0 - 0.5 * p), 3)
        out.append(r)
    return out


def run_decompress(hts, wl, dev, time_graph, time_launches, quick):
    """The 7B up-projection with 2:4 tiles expanded in registers to the dense matrix instruction
    (the measured fallback of the sparse instruction), at M = 1, 16, 2048."""
    cfg = wl.config("7b_up")
    old = os.environ.get("HTS_SPARSE_PATH")
    os.environ["HTS_SPARSE_PATH"] = "decompress"
    try:
        r = run_layer(hts, wl, dev, time_graph, time_launches, quick, cfg, cfg.layers[0], list(cfg.Ms))
    finally:
        if old is None:
            os.environ.pop("HTS_SPARSE_PATH", None)
        else:
            os.environ["HTS_SPARSE_PATH"] = old
    return r


def run_peaks(quick):
    """Measured denominators: one streaming read of 2 GiB, and the matrix-core instructions of the
    product with register operands (algorithmic TFLOP/s: kept multiply-adds)."""
    import tile_gemm_amd.peak as peak
    out = {"hbm_stream_read_GB/s": round(peak.stream_read_gbs(reps=2 if quick else 5), 1)}
    for k in peak.KINDS:
        out[f"{k}_TFLOP/s"] = round(peak.mfma_tflops(k, reps=2 if quick else 5), 1)
    # on-chip paths per CU, in bytes per cycle at the clock the 16-bit matrix cores ran at above
    # (1,024 flops per cycle per SIMD, 4 SIMDs per CU)
    clk = out["bf16_dense_TFLOP/s"] * 1e12 / (1024 * 4 * 256)
    out["clock_from_mfma_GHz"] = round(clk / 1e9, 3)
    for m in peak.ONCHIP:
        g = peak.onchip_gbs(m, reps=2 if quick else 5)
        out[f"{m}_GB/s"] = round(g, 1)
        out[f"{m}_B_per_clk_per_CU"] = round(g * 1e9 / 256 / clk, 1)
    return out


def run_block(hts, wl, dev, time_graph, quick):
    """One 7B decoder block's seven projections (+ the gated-MLP step) at M = 2048 on packed weights
    with Wanda tile maps at 30 % overall sparsity -- per layer and with one global budget -- against
    the same pipeline on the same-library dense product and on torch (hipBLASLt) for context.
    Maps are derived on the GPU (column norms of the calibration rows, tile costs, selection)."""
    import torch
    import tile_gemm_amd.block as block
    cfg = wl.config("7b_block")
    M = 2048
    Ws, css = {}, {}
    for L in cfg.layers:
        Ws[L.name] = hts.tensor_from_bits(wl.weight_bits(cfg, L), L.dtype, dev)
        css[L.name] = hts.col_norms(hts.tensor_from_bits(wl.layer_calib_bits(cfg, L), L.dtype, dev))
    maps = {"per_layer": {L.name: hts.wanda_tile_map(Ws[L.name], css[L.name], L.bn, L.bk, L.n_sparse_target)
                          for L in cfg.layers}}
    T = sum(L.T for L in cfg.layers)
    glob = hts.wanda_global_maps([Ws[L.name] for L in cfg.layers], [css[L.name] for L in cfg.layers], 128, 128,
                                 int(round(2 * 0.3 * T)))
    maps["global"] = {L.name: m for L, m in zip(cfg.layers, glob)}
    X = hts.tensor_from_bits(wl.activation_bits(cfg, cfg.layers[0], M), "bf16", dev)
    reps = 3 if quick else 10
    out = {"workload": "LLaMA-2-7B decoder block linear layers (q, k, v, o 4096x4096; gate, up 11008x4096; "
                       "down 4096x11008; bf16) + silu(gate)*up, M=2048; o reads q in place of the attention output",
           "M": M}
    dense_bufs = block.buffers(M, Ws, X.dtype, dev)
    t_dense = time_graph(lambda i: block.forward(X, Ws, dense_bufs), 1, reps)
    dense_flops = block.kept_flops(M, Ws)
    for kind, mp in maps.items():
        packed = {L.name: hts.pack(Ws[L.name], mp[L.name].cpu().numpy(), L.bn, L.bk) for L in cfg.layers}
        bufs = block.buffers(M, packed, X.dtype, dev)
        t = time_graph(lambda i: block.forward(X, packed, bufs), 1, reps)
        # the up product writing silu(gate) * up itself (the dense block has no such variant)
        t_f = time_graph(lambda i: block.forward(X, packed, bufs, fused=True), 1, reps)
        flops = block.kept_flops(M, packed)
        ns = {L.name: int(mp[L.name].sum().item()) for L in cfg.layers}
        out[kind] = {"us": round(t * 1e6, 1), "TFLOP/s": round(flops / t / 1e12, 1),
                     "speedup_vs_dense": round(t_dense / t, 3),
                     "fused_gate_us": round(t_f * 1e6, 1), "fused_gate_speedup_vs_dense": round(t_dense / t_f, 3),
                     "sparse_tiles": ns, "overall_sparsity": round(0.5 * sum(ns.values()) / T, 4)}
        del packed, bufs
    out["dense_same_library_us"] = round(t_dense * 1e6, 1)
    out["dense_same_library_TFLOP/s"] = round(dense_flops / t_dense / 1e12, 1)

    def torch_block(i, bufs=dense_bufs):
        torch.matmul(X, Ws["q"].t(), out=bufs["q"])
        torch.matmul(X, Ws["k"].t(), out=bufs["k"])
        torch.matmul(X, Ws["v"].t(), out=bufs["v"])
        torch.matmul(bufs["q"], Ws["o"].t(), out=bufs["o"])
        torch.matmul(X, Ws["gate"].t(), out=bufs["gate"])
        torch.matmul(X, Ws["up"].t(), out=bufs["up"])
        torch.mul(torch.nn.functional.silu(bufs["gate"]), bufs["up"], out=bufs["h"])
        torch.matmul(bufs["h"], Ws["down"].t(), out=bufs["down"])
    t_torch = time_graph(torch_block, 1, reps)
    out["torch_us"] = round(t_torch * 1e6, 1)
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(the sharding design is described in the design notes); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import tile_gemm_amd as hts
    import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    cfg = wl.config(args.config)
    L = cfg.layers[args.layer]
    M_big = max(cfg.Ms)
    dec_Ms = [m for m in cfg.Ms if m <= 16]
    tdt = torch.bfloat16 if L.dtype == "bf16" else torch.float16

    # ---------------- inputs (seeded, synthetic) ----------------
    W_bits = wl.weight_bits(cfg, L)
    tmap = wl.tile_map(cfg, L)
    X_bits = wl.activation_bits(cfg, L, M_big)
    W = hts.tensor_from_bits(W_bits, L.dtype, dev)
    X = hts.tensor_from_bits(X_bits, L.dtype, dev)
    n_sparse = int(tmap.sum())
    kept = L.N * L.K - n_sparse * L.bn * L.bk // 2

    # pack (timed below as well)
    pw0 = hts.pack(W, tmap, L.bn, L.bk)
    torch.cuda.synchronize()
    packed_bytes = pw0.packed_bytes
    dense_bytes = 2 * L.N * L.K
    n_rot = max(2, -(-ROTATE_BYTES // packed_bytes))
    pws = [pw0] + [hts.PackedWeight(pw0.desc, pw0.index.clone(), pw0.values.clone(), pw0.meta.clone(),
                                    pw0.sizes, pw0.tile_map) for _ in range(n_rot - 1)]
    n_rot_d = max(2, -(-ROTATE_BYTES // dense_bytes))
    Ws = [W] + [W.clone() for _ in range(n_rot_d - 1)]
    # the same weight packed with an all-dense map: the hybrid path's own dense reference (same
    # kernels and storage order; the row-major dense product reads W row by row)
    pd0 = hts.pack(W, np.zeros_like(tmap), L.bn, L.bk)
    pds = [pd0] + [hts.PackedWeight(pd0.desc, pd0.index.clone(), pd0.values.clone(), pd0.meta.clone(),
                                    pd0.sizes, pd0.tile_map) for _ in range(n_rot_d - 1)]
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def time_launches(fn, n, reps=3):
        """Average device time of one launch over n back-to-back launches (HIP events on this stream)."""
        best = None
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(n):
                fn(i)
            e1.record(stream)
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) * 1e-3 / n
            best = t if best is None else min(best, t)
        return best

    def time_graph(fn, per_graph, replays=20):
        """Average device time of one launch, launches captured in a HIP graph (no host overhead)."""
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(per_graph):
                fn(i)                 # warm (outside capture) on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(per_graph):
                fn(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        best = None
        for _ in range(3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(replays):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) * 1e-3 / (replays * per_graph)
            best = t if best is None else min(best, t)
        return best

    results = {}

    # ---------------- decode shapes (HBM-bound) ----------------
    decode = []
    for M in dec_Ms:
        Xm = X[:M].contiguous()
        Ys = [torch.empty((M, L.N), dtype=tdt, device=dev) for _ in range(n_rot)]
        Yd = [torch.empty((M, L.N), dtype=tdt, device=dev) for _ in range(n_rot_d)]
        hyb = lambda i: hts.gemm(Xm, pws[i % n_rot], out=Ys[i % n_rot])
        den = lambda i: hts.dense_gemm(Xm, Ws[i % n_rot_d], out=Yd[i % n_rot_d])
        mm = lambda i: torch.matmul(Xm, Ws[i % n_rot_d].t(), out=Yd[i % n_rot_d])
        dpk = lambda i: hts.gemm(Xm, pds[i % n_rot_d], out=Yd[i % n_rot_d])
        per = 4 if args.quick else 8 * max(n_rot, n_rot_d)
        t_h = time_graph(hyb, per, 2 if args.quick else 25)
        t_d = time_graph(den, per, 2 if args.quick else 25)
        t_dp = time_graph(dpk, per, 2 if args.quick else 25)
        t_t = time_graph(mm, per, 2 if args.quick else 25)
        alg_bytes = packed_bytes + 2 * M * L.K + 2 * M * L.N
        den_bytes = dense_bytes + 2 * M * L.K + 2 * M * L.N
        decode.append({
            "M": M, "us": round(t_h * 1e6, 3),
            "GB/s": round(alg_bytes / t_h / 1e9, 1),
            "frac_hbm": round(alg_bytes / t_h / 1e9 / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": alg_bytes,
            "dense_same_library_us": round(t_d * 1e6, 3),
            "dense_same_library_GB/s": round(den_bytes / t_d / 1e9, 1),
            "speedup_vs_dense": round(t_d / t_h, 3),
            "dense_packed_us": round(t_dp * 1e6, 3),
            "speedup_vs_dense_packed": round(t_dp / t_h, 3),
            "torch_matmul_us": round(t_t * 1e6, 3),
        })

    # ---------------- prefill shape: the timed step ----------------
    M = M_big
    Xm = X
    Ys = [torch.empty((M, L.N), dtype=tdt, device=dev) for _ in range(2)]
    step = lambda i: hts.gemm(Xm, pws[i % n_rot], out=Ys[i % 2])
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_step = e0.elapsed_time(e1) * 1e-3 / args.steps
    alg_flops = 2.0 * M * kept
    dense_flops = 2.0 * M * L.N * L.K
    tflops = alg_flops / t_step / 1e12

    Ydd = [torch.empty((M, L.N), dtype=tdt, device=dev) for _ in range(2)]
    n_pf = 10 if args.quick else 50
    # the hybrid timed like its comparators (best of 3 windows of n_pf launches) for the speed-ups
    t_step_ll = time_launches(step, n_pf)
    t_dense = time_launches(lambda i: hts.dense_gemm(Xm, Ws[i % n_rot_d], out=Ydd[i % 2]), n_pf)
    # (not in profiling runs: it launches the timed step's kernel on another map)
    t_dense_packed = None if args.quick else time_launches(lambda i: hts.gemm(Xm, pds[i % n_rot_d], out=Ydd[i % 2]), n_pf)
    t_torch = time_launches(lambda i: torch.matmul(Xm, Ws[i % n_rot_d].t(), out=Ydd[i % 2]), n_pf)

    # ---------------- pack / unpack ----------------
    vals_tmp = torch.empty_like(pw0.values)
    meta_tmp = torch.empty_like(pw0.meta)
    t_pack = time_launches(lambda i: hts.hts_pack(pw0.desc, pw0.index, Ws[i % n_rot_d], None, vals_tmp, meta_tmp),
                           5 if args.quick else 20)
    Wout = torch.empty_like(W)
    t_unpack = time_launches(lambda i: hts.hts_unpack(pws[i % n_rot].desc, pws[i % n_rot].index,
                                                      pws[i % n_rot].values, pws[i % n_rot].meta, Wout),
                             5 if args.quick else 20)
    pack_bytes = dense_bytes + packed_bytes
    # packing from a given element mask (frozen 2:4 patterns): reads W, the mask inside the 2:4
    # tiles and writes the packed weight
    mask = torch.from_numpy(wl.layer_pair_mask(cfg, L)).to(dev)
    bad = torch.empty(1, dtype=torch.int32, device=dev)
    t_pack_masked = time_launches(lambda i: hts.hts_pack_masked(pw0.desc, pw0.index, Ws[i % n_rot_d], mask, vals_tmp,
                                                                meta_tmp, bad), 5 if args.quick else 20)
    pack_masked_bytes = dense_bytes + n_sparse * L.bn * L.bk + packed_bytes

    if args.calibrate_copy:
        # three plain copies of 256 MiB each (distinct buffers, larger than the Infinity Cache in total)
        n_cp = 256 << 20
        srcs = [torch.empty(n_cp, dtype=torch.uint8, device=dev).fill_(1) for _ in range(3)]
        dsts = [torch.empty(n_cp, dtype=torch.uint8, device=dev) for _ in range(3)]
        torch.cuda.synchronize()
        for a_, b_ in zip(dsts, srcs):
            a_.copy_(b_)
        torch.cuda.synchronize()
        del srcs, dsts

    # ---------------- decoder block: the seven projections of a 7B block ----------------
    block_res = None if args.no_block else run_block(hts, wl, dev, time_graph, args.quick)

    # ---------------- 8-bit E4M3 variant of the same layer ----------------
    fp8_res = None if args.no_fp8 else run_fp8(hts, wl, dev, time_graph, time_launches, args.quick)
    tiles_res = None if args.no_tiles else run_tile_sizes(hts, wl, dev, time_graph, time_launches, args.quick)
    shard_res = None if args.no_shard else run_shard(hts, wl, dev, time_graph, time_launches, args.quick)
    mid_res = None if args.no_mid else run_mid_m(hts, wl, dev, time_graph, args.quick)
    r13 = None if args.no_13b else run_13b(hts, wl, dev, time_graph, time_launches, args.quick)
    sweep_res = None if args.no_sweep else run_sweep(hts, wl, dev, time_graph, time_launches, args.quick)
    dec_res = None if args.no_decompress else run_decompress(hts, wl, dev, time_graph, time_launches, args.quick)
    peaks = None if args.no_peaks else run_peaks(args.quick)

    # ---------------- CPU oracle on the host cores ----------------
    cpu = None
    if not (args.quick or args.no_cpu):
        import oracle
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        # the sample is the whole layer at the step's M (mask + fp64 product), repeated
        reps, t_cpu = 0, []
        while reps < 3 or (sum(t_cpu) < 12.0 and reps < 200):
            t_c0 = time.perf_counter()
            Wm_full = oracle.masked_weights(W_bits, L.dtype, tmap, L.bn, L.bk)
            oracle.gemm_ref(X_bits, Wm_full, L.dtype)
            t_cpu.append(time.perf_counter() - t_c0)
            reps += 1
        t_med = float(np.median(t_cpu))
        cpu = {"value": round(alg_flops / t_med / 1e12, 5), "unit": "TFLOP/s",
               "cores": int(threads), "kind": "oracle",
               "sample": f"whole layer at M={M}: oracle mask + fp64 product, median of {reps} runs "
                         f"({t_med:.2f} s each) on {len(os.sched_getaffinity(0))} visible host cores "
                         f"({platform.processor() or platform.machine()}), BLAS threads {threads}"}

    prefill = {
        "M": M, "us": round(t_step * 1e6, 2),
        "TFLOP/s": round(tflops, 2),
        "dense_equivalent_TFLOP/s": round(dense_flops / t_step / 1e12, 2),
        "frac_mfma": round(tflops / MFMA_PEAK_TFLOPS[L.dtype], 4),
        "us_timed_like_comparators": round(t_step_ll * 1e6, 2),
        "dense_same_library_us": round(t_dense * 1e6, 2),
        "dense_same_library_TFLOP/s": round(dense_flops / t_dense / 1e12, 2),
        "speedup_vs_dense": round(t_dense / t_step_ll, 3),
        "dense_packed_us": None if t_dense_packed is None else round(t_dense_packed * 1e6, 2),
        "speedup_vs_dense_packed": None if t_dense_packed is None else round(t_dense_packed / t_step_ll, 3),
        "torch_matmul_us": round(t_torch * 1e6, 2),
        "torch_matmul_TFLOP/s": round(dense_flops / t_torch / 1e12, 2),
    }
    line = {
        "metric": "hybrid tile-sparse GEMM TFLOP/s & GB/s (% roofline), speedup vs dense, 7B shapes",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": L.dtype,
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: W[{L.N}x{L.K}] {L.dtype}, tile {L.bn}x{L.bk}, "
                               f"{n_sparse}/{L.T} tiles 2:4 ({100.0 * n_sparse * 0.5 / L.T:.1f}% overall sparsity), "
                               f"X[{M}x{L.K}]; step = one hybrid product at M={M}",
                   "M": M, "N": L.N, "K": L.K, "tile": [L.bn, L.bk], "sparse_tiles": n_sparse,
                   "sparse_path": os.environ.get("HTS_SPARSE_PATH", "smfmac")},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_PEAK_TFLOPS[L.dtype],
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_PEAK_TFLOPS[L.dtype], 4),
                     "traffic": recorded_traffic(f"{cfg.name}/{L.name}/M={M}"),
                     "kernel": "gemm_prefill_kernel", "algorithmic_flops_per_launch": alg_flops,
                     "kernel_source_hash": prefill_source_hash()},
        "cpu_baseline": cpu,
        "decode": decode,
        "prefill": prefill,
        "pack": {"us": round(t_pack * 1e6, 2), "GB/s": round(pack_bytes / t_pack / 1e9, 1),
                 "frac_hbm": round(pack_bytes / t_pack / 1e9 / HBM_PEAK_GBS, 4)},
        "unpack": {"us": round(t_unpack * 1e6, 2), "GB/s": round(pack_bytes / t_unpack / 1e9, 1)},
        "pack_masked": {"us": round(t_pack_masked * 1e6, 2), "GB/s": round(pack_masked_bytes / t_pack_masked / 1e9, 1),
                        "frac_hbm": round(pack_masked_bytes / t_pack_masked / 1e9 / HBM_PEAK_GBS, 4)},
        "block": block_res,
        "fp8": fp8_res,
        "tile_sizes": tiles_res,
        "shard": shard_res,
        "mid_m": mid_res,
        "13b": r13,
        "sweep": sweep_res,
        "decompress_fallback": dec_res,
        "measured_peaks": peaks,
        "packed_bytes": packed_bytes,
        "rotation_copies": n_rot,
        "wall_s_timed_region": round(wall, 4),
    }
    if peaks:
        # fractions against the measured denominators beside the published ones
        mp = peaks.get(f"{L.dtype}_dense_TFLOP/s") or peaks.get("bf16_dense_TFLOP/s")
        line["roofline"]["measured_peak"] = mp
        line["roofline"]["frac_of_measured_peak"] = round(tflops / mp, 4) if mp else None
        for d in decode:
            d["frac_of_measured_hbm"] = round(d["GB/s"] / peaks["hbm_stream_read_GB/s"], 4)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

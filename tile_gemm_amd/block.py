"""The linear layers of a LLaMA-style decoder block on hybrid tile-sparse weights.

The pages prune the linear layers of LLaMA-family models and report speed at the level of the
whole model ("PATCH: Learnable Tile-level Hybrid Sparsity for LLMs", section 4, speed).  The
closest weight-free analogue this library can run is one decoder block's seven projections
back to back:

    q = X Wq^T,  k = X Wk^T,  v = X Wv^T,  o = A Wo^T,
    gate = X Wg^T,  up = X Wu^T,  h = silu(gate) * up,  down = h Wd^T

with every W either a packed hybrid weight (hts_gemm) or a row-major dense one
(hts_dense_gemm, the same-library baseline).  Attention itself is not part of this library: the
output projection reads A = q in its place, which keeps the shapes and the data dependence of
the block.  Every call is enqueued on the current stream, so the whole step can be captured in
one HIP graph.
"""
from __future__ import annotations

from typing import Dict

import torch

from . import PackedWeight, dense_gemm, gemm, gemm_silu_mul, silu_mul

PROJECTIONS = ("q", "k", "v", "o", "gate", "up", "down")


def buffers(M: int, weights: Dict[str, object], dtype, device) -> Dict[str, torch.Tensor]:
    """Output buffers of every step for M tokens."""
    def rows(w):
        return w.N if isinstance(w, PackedWeight) else w.shape[0]
    out = {name: torch.empty((M, rows(weights[name])), dtype=dtype, device=device) for name in PROJECTIONS}
    out["h"] = torch.empty_like(out["gate"])
    return out


def _linear(x: torch.Tensor, w, out: torch.Tensor) -> torch.Tensor:
    if isinstance(w, PackedWeight):
        return gemm(x, w, out=out)
    return dense_gemm(x, w, out=out)


def forward(X: torch.Tensor, weights: Dict[str, object], bufs: Dict[str, torch.Tensor],
            fused: bool = False) -> torch.Tensor:
    """One block step on M = X.shape[0] tokens; returns the down-projection output.  fused (packed
    up weight only): the up product writes silu(gate) * up itself (hts_gemm_silu_mul) instead of
    writing up for a separate elementwise pass."""
    fuse = fused and isinstance(weights["up"], PackedWeight)
    for name in ("q", "k", "v", "gate") + (() if fuse else ("up",)):
        _linear(X, weights[name], bufs[name])
    _linear(bufs["q"], weights["o"], bufs["o"])          # attention output stand-in: A = q
    if fuse:
        gemm_silu_mul(X, weights["up"], bufs["gate"], out=bufs["h"])
    else:
        silu_mul(bufs["gate"], bufs["up"], out=bufs["h"])
    return _linear(bufs["h"], weights["down"], bufs["down"])


def kept_flops(M: int, weights: Dict[str, object]) -> float:
    """Algorithmic flops of one step: 2 M (kept weights) over the seven projections."""
    total = 0
    for name in PROJECTIONS:
        w = weights[name]
        if isinstance(w, PackedWeight):
            total += w.N * w.K - w.sizes["n_sparse"] * w.desc.bn * w.desc.bk // 2
        else:
            total += w.shape[0] * w.shape[1]
    return 2.0 * M * total

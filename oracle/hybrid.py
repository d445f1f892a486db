"""CPU oracle for tile-level hybrid (dense / 2:4) sparse linear layers.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this module; only the
tests, the smoke check of the package entry file and the CPU-baseline leg of the
benchmark call it.  It shares no code, table or constant with the GPU path.

What is computed (PATCH page, "PATCH: Learnable Tile-level Hybrid Sparsity for
LLMs", section 2 "core mechanism"): a weight matrix W[N,K] is cut into
rectangular tiles of bn x bk; every tile is either kept dense (0 % sparse) or
made 2:4 sparse (50 % sparse: two of every four weights kept, section 1 and the
lay summary), so that mixing the two tile kinds reaches any overall sparsity
from 0 % to 50 % (section 3).  The layer output is then the plain product of
the activations with the masked weights, Y = X . mask(W)^T.  Section 2
("inference and deployment") says compressed storage is what turns the zeros
into speed; the packed format below is this library's storage of that mask.

Readings where the pages are silent (each also listed in the design notes):
  * 2:4 groups run along K, aligned to k = 0 mod 4 inside each tile.
  * The kept pair of a group is the two largest selection scores; among equal
    scores the lower index wins (a deterministic tie-break).
  * The selection score is |w| (magnitude) or, when a per-column scale c is
    given, fl32(|w| * c_k) -- the Wanda product of weight magnitude and the
    input-activation column norm (Wanda section of the page "SparseGPT vs Wanda:
    one-shot LLM pruning without retraining").
  * Dropped weights of a sparse tile read back as +0.0; kept weights keep their
    exact bits (-0.0 and subnormals included).
  * Products are evaluated in fp64 on the 16-bit inputs widened exactly.

All 16-bit arrays are numpy uint16 bit patterns with a dtype tag "f16" (IEEE
binary16) or "bf16" (bfloat16).  The 8-bit variant (prune, then quantize: the
FAQ of the SparseGPT-vs-Wanda page pairs 2:4 pruning with low-precision
weights) stores numpy uint8 patterns with the tag "fp8": the OCP 8-bit E4M3
format (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, subnormals,
no infinities, 0x7F and 0xFF are NaN).  Every E4M3 value is exact in binary32,
so every rule above applies unchanged to the decoded values.
"""
from __future__ import annotations

import numpy as np

TILE_DENSE = 0
TILE_SPARSE24 = 1

# ----------------------------------------------------------------------------
# 16-bit storage types, widened exactly
# ----------------------------------------------------------------------------

def storage_type(dtype: str):
    """numpy type of the stored bit patterns of a weight / activation dtype."""
    if dtype == "fp8":
        return np.uint8
    if dtype in ("f16", "bf16"):
        return np.uint16
    raise ValueError(f"unknown storage type {dtype!r}")


def e4m3_value(bits: np.ndarray) -> np.ndarray:
    """Exact float64 value of OCP E4M3 bytes: (-1)^s * 2^(e-7) * (1 + m/8) for e > 0,
    (-1)^s * 2^-6 * (m/8) for e = 0; the two all-ones patterns 0x7F / 0xFF are NaN."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    return np.where((b & 0x7F) == 0x7F, np.nan, sign * mag)


def widen_f32(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float32 value of every stored pattern (all three formats embed in binary32)."""
    if dtype == "fp8":
        return e4m3_value(bits).astype(np.float32)
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float32)
    if dtype == "bf16":
        # bfloat16 is the upper half of a binary32 pattern
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    raise ValueError(f"unknown 16-bit type {dtype!r}")


def widen_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    return widen_f32(bits, dtype).astype(np.float64)


# ----------------------------------------------------------------------------
# Tile grid
# ----------------------------------------------------------------------------

def check_grid(N: int, K: int, bn: int, bk: int) -> None:
    assert N > 0 and K > 0, "empty weight"
    assert bn > 0 and bk > 0 and bk % 32 == 0, "a tile row's 2-bit codes must fill whole 32-bit words"
    assert N % bn == 0 and K % bk == 0, "tiles must cover W exactly"


def as_tiles(A: np.ndarray, bn: int, bk: int) -> np.ndarray:
    """View A[N,K] as tiles[T, bn, bk] in row-major tile order t = tn*T_k + tk (a copy)."""
    N, K = A.shape
    return A.reshape(N // bn, bn, K // bk, bk).transpose(0, 2, 1, 3).reshape(-1, bn, bk).copy()


def from_tiles(tiles: np.ndarray, N: int, K: int) -> np.ndarray:
    T, bn, bk = tiles.shape
    return tiles.reshape(N // bn, K // bk, bn, bk).transpose(0, 2, 1, 3).reshape(N, K).copy()


# ----------------------------------------------------------------------------
# Selection: scores and the 2-of-4 choice
# ----------------------------------------------------------------------------

def selection_scores(W_bits: np.ndarray, dtype: str, col_scale: np.ndarray | None = None) -> np.ndarray:
    """float32 score per weight: |w|, or fl32(|w| * c_k) with a per-column scale c (Wanda rule)."""
    a = np.abs(widen_f32(W_bits, dtype))
    if col_scale is None:
        return a
    c = np.asarray(col_scale, dtype=np.float32)
    assert c.shape == (W_bits.shape[1],)
    return np.multiply(a, c[None, :], dtype=np.float32)  # one IEEE binary32 product, RNE


def keep_two_of_four(scores: np.ndarray) -> np.ndarray:
    """Boolean keep-mask over the last axis (length 4): exactly two True per group.

    Weight i of a group is kept when fewer than two of the other weights beat it,
    where j beats i if its score is larger, or equal with a lower index j < i.
    """
    s = np.asarray(scores)
    assert s.shape[-1] == 4
    rank = np.zeros(s.shape, dtype=np.int64)
    for i in range(4):
        for j in range(4):
            if j == i:
                continue
            beats = (s[..., j] > s[..., i]) | ((s[..., j] == s[..., i]) & (j < i))
            rank[..., i] += beats
    return rank < 2


def kept_positions(keep: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """(i0, i1): the lower and the higher kept index of every group (keep has two True per group)."""
    pos = np.arange(4)
    i0 = np.where(keep, pos, 4).min(axis=-1)
    i1 = np.where(keep, pos, -1).max(axis=-1)
    return i0, i1


def sparse_tile_keep(tile_scores: np.ndarray) -> np.ndarray:
    """Keep-mask [bn, bk] of one sparse tile: groups of 4 along K, aligned at the tile start."""
    bn, bk = tile_scores.shape
    return keep_two_of_four(tile_scores.reshape(bn, bk // 4, 4)).reshape(bn, bk)


def masked_weights(W_bits: np.ndarray, dtype: str, tile_map: np.ndarray, bn: int, bk: int,
                   col_scale: np.ndarray | None = None) -> np.ndarray:
    """mask(W): dense tiles unchanged; in sparse tiles the two dropped weights of each group become +0.0."""
    N, K = W_bits.shape
    check_grid(N, K, bn, bk)
    tmap = np.asarray(tile_map, dtype=np.uint8).ravel()
    assert tmap.size == (N // bn) * (K // bk)
    assert np.all(tmap <= 1), "tile map entries must be 0 (dense) or 1 (2:4)"
    tiles = as_tiles(np.asarray(W_bits, dtype=storage_type(dtype)), bn, bk)
    stiles = as_tiles(selection_scores(W_bits, dtype, col_scale), bn, bk)
    for t in np.nonzero(tmap == TILE_SPARSE24)[0]:
        keep = sparse_tile_keep(stiles[t])
        tiles[t][~keep] = 0  # +0.0 in every format
    return from_tiles(tiles, N, K)


# ----------------------------------------------------------------------------
# Packed storage
# ----------------------------------------------------------------------------
# Tiles are stored one after another in row-major tile order t = tn*T_k + tk.
#   dense tile : bn*bk values, row-major inside the tile.
#   sparse tile: bn*bk/2 values; row r, group g holds the kept pair at
#                r*(bk/2) + 2g (lower index) and r*(bk/2) + 2g + 1 (higher index);
#                plus bn*bk/32 metadata words: word r*(bk/32) + g//8 carries the
#                4-bit code  i0 | (i1 << 2)  of group g at bits 4*(g % 8) .. +3.
#   index      : one record per tile {val_off (values), meta_off (words), type, 0}.
# With this code a group's nibble names the two kept positions; the six valid
# codes are exactly the C(4,2) = 6 choices of a 2:4 pattern (PATCH section 2,
# "learnable distributions": six possible patterns).

VALID_NIBBLES = frozenset({0x4, 0x8, 0xC, 0x9, 0xD, 0xE})


def plan(tile_map: np.ndarray, N: int, K: int, bn: int, bk: int, elem_bytes: int = 2):
    """Tile index [T,4] uint32 and buffer sizes for a tile map (sizes in elements/words/bytes;
    elem_bytes is 2 for the 16-bit types, 1 for fp8)."""
    check_grid(N, K, bn, bk)
    tmap = np.asarray(tile_map, dtype=np.uint8).ravel()
    T = (N // bn) * (K // bk)
    assert tmap.size == T and np.all(tmap <= 1)
    index = np.zeros((T, 4), dtype=np.uint32)
    val_off = 0
    meta_off = 0
    for t in range(T):
        index[t] = (val_off, meta_off, tmap[t], 0)
        if tmap[t] == TILE_SPARSE24:
            val_off += bn * bk // 2
            meta_off += bn * bk // 32
        else:
            val_off += bn * bk
    n_sparse = int(tmap.sum())
    sizes = {"values": val_off, "meta": meta_off, "values_bytes": elem_bytes * val_off,
             "meta_bytes": 4 * meta_off, "index_bytes": 16 * T, "n_sparse": n_sparse}
    return index, sizes


# Storage order inside a tile (a format choice of this library, not of the pages): a tile's rows
# (dense: all bk weights; 2:4: the bk/2 kept weights) are cut into 16-row panels -- the whole tile
# when bn is not a multiple of 16 -- and into 16-byte chunks along the row.  Inside a panel the
# chunks are stored column by column, the panel's rows consecutive within a chunk column: chunk c
# of panel row r is at (c * panel_rows + r) chunks from the panel start.  A matrix-core operand
# (one chunk of each of 16 consecutive rows, for four consecutive chunk columns) is then one
# contiguous kilobyte.

def panel_rows(bn: int) -> int:
    return 16 if bn % 16 == 0 else bn


def panel_order(block: np.ndarray, elem_bytes: int) -> np.ndarray:
    """The elements of a row-major [rows, w] block of one tile, flattened in storage order."""
    rows, w = block.shape
    ph, ch = panel_rows(rows), 16 // elem_bytes
    assert w % ch == 0
    return block.reshape(rows // ph, ph, w // ch, ch).transpose(0, 2, 1, 3).ravel()


def panel_unorder(flat: np.ndarray, rows: int, w: int, elem_bytes: int) -> np.ndarray:
    """Inverse of panel_order: the row-major [rows, w] block."""
    ph, ch = panel_rows(rows), 16 // elem_bytes
    return np.asarray(flat).reshape(rows // ph, w // ch, ph, ch).transpose(0, 2, 1, 3).reshape(rows, w)


def pack(W_bits: np.ndarray, dtype: str, tile_map: np.ndarray, bn: int, bk: int,
         col_scale: np.ndarray | None = None, scores: np.ndarray | None = None):
    """(values, meta uint32, index uint32[T,4]) of W under the tile map (values in the storage
    type of dtype: uint16, or uint8 for fp8).

    scores: float32 [N,K] selection scores to use instead of the magnitude / Wanda scores
    (see pack_masked)."""
    N, K = W_bits.shape
    st = storage_type(dtype)
    eb = np.dtype(st).itemsize
    index, sizes = plan(tile_map, N, K, bn, bk)
    tmap = index[:, 2]
    tiles = as_tiles(np.asarray(W_bits, dtype=st), bn, bk)
    if scores is None:
        scores = selection_scores(W_bits, dtype, col_scale)
    stiles = as_tiles(np.asarray(scores, dtype=np.float32), bn, bk)
    values = []
    meta = []
    G = bk // 4
    for t in range(tiles.shape[0]):
        if tmap[t] == TILE_DENSE:
            values.append(panel_order(tiles[t], eb))
            continue
        keep = sparse_tile_keep(stiles[t]).reshape(bn, G, 4)
        i0, i1 = kept_positions(keep)                       # [bn, G]
        groups = tiles[t].reshape(bn, G, 4)
        v0 = np.take_along_axis(groups, i0[..., None], axis=-1)[..., 0]
        v1 = np.take_along_axis(groups, i1[..., None], axis=-1)[..., 0]
        kept = np.stack([v0, v1], axis=-1).reshape(bn, bk // 2)   # row r: (g, lower/higher)
        values.append(panel_order(kept, eb))
        nib = (i0 | (i1 << 2)).astype(np.uint32).reshape(bn, G // 8, 8)
        shifts = (4 * np.arange(8)).astype(np.uint32)
        words = np.bitwise_or.reduce(nib << shifts, axis=-1)  # [bn, bk/32]
        meta.append(words.ravel())
    vals = np.concatenate(values).astype(st) if values else np.zeros(0, st)
    met = np.concatenate(meta).astype(np.uint32) if meta else np.zeros(0, np.uint32)
    assert vals.size == sizes["values"] and met.size == sizes["meta"]
    return vals, met, index


# ----------------------------------------------------------------------------
# Packing from a given element mask
# ----------------------------------------------------------------------------
# PATCH page, section 2 ("variants"): in the PATCH-Tile variant the 2:4 patterns are
# not learned but frozen from a one-shot pruning method, and only the tile choices
# are learned.  The 2:4 selection is then an input: an element mask that keeps two
# of every four weights of each group (along K, aligned as above) in the 2:4 tiles.
# Reading taken for malformed input: the mask is the selection score (1 = marked),
# so a group marking exactly two weights keeps exactly those two; a group marking
# some other number keeps the two the rank rule picks (marked before unmarked, lower
# index first among equals) and is counted as malformed.

def mask_scores(mask: np.ndarray) -> np.ndarray:
    """float32 selection score of every weight from a keep mask: 1 where marked, else 0."""
    return (np.asarray(mask) != 0).astype(np.float32)


def malformed_groups(mask: np.ndarray, tile_map: np.ndarray, bn: int, bk: int) -> int:
    """Number of groups of four in the 2:4 tiles whose mask does not mark exactly two weights."""
    N, K = mask.shape
    check_grid(N, K, bn, bk)
    tmap = np.asarray(tile_map, dtype=np.uint8).ravel()
    m = as_tiles((np.asarray(mask) != 0).astype(np.uint8), bn, bk)[tmap == TILE_SPARSE24]
    counts = m.reshape(m.shape[0], bn, bk // 4, 4).sum(axis=-1)
    return int(np.count_nonzero(counts != 2))


def pack_masked(W_bits: np.ndarray, dtype: str, tile_map: np.ndarray, mask: np.ndarray, bn: int, bk: int):
    """(values, meta, index, malformed) of W packed with the 2:4 pairs the mask marks."""
    vals, met, index = pack(W_bits, dtype, tile_map, bn, bk, scores=mask_scores(mask))
    return vals, met, index, malformed_groups(mask, tile_map, bn, bk)


def masked_weights_from_mask(W_bits: np.ndarray, tile_map: np.ndarray, mask: np.ndarray, bn: int,
                             bk: int) -> np.ndarray:
    """The weight a masked pack stores: dense tiles unchanged; in 2:4 tiles the weights the
    selection drops become +0.0 (for a well-formed mask: exactly the unmarked ones)."""
    N, K = W_bits.shape
    check_grid(N, K, bn, bk)
    tmap = np.asarray(tile_map, dtype=np.uint8).ravel()
    tiles = as_tiles(np.asarray(W_bits), bn, bk)
    stiles = as_tiles(mask_scores(mask), bn, bk)
    for t in np.nonzero(tmap == TILE_SPARSE24)[0]:
        keep = sparse_tile_keep(stiles[t])
        tiles[t][~keep] = 0
    return from_tiles(tiles, N, K)


def unpack(values: np.ndarray, meta: np.ndarray, index: np.ndarray, N: int, K: int,
           bn: int, bk: int) -> np.ndarray:
    """Inverse of pack: W'[N,K] bits (the storage type of values) with +0.0 at dropped
    positions of sparse tiles."""
    check_grid(N, K, bn, bk)
    T = (N // bn) * (K // bk)
    assert index.shape == (T, 4)
    G = bk // 4
    values = np.asarray(values)
    eb = values.dtype.itemsize
    tiles = np.zeros((T, bn, bk), dtype=values.dtype)
    for t in range(T):
        val_off, meta_off, typ, _ = (int(x) for x in index[t])
        if typ == TILE_DENSE:
            tiles[t] = panel_unorder(values[val_off: val_off + bn * bk], bn, bk, eb)
            continue
        pairs = panel_unorder(values[val_off: val_off + bn * bk // 2], bn, bk // 2, eb).reshape(bn, G, 2)
        words = meta[meta_off: meta_off + bn * bk // 32].reshape(bn, G // 8).astype(np.uint32)
        nib = (words[..., None] >> (4 * np.arange(8)).astype(np.uint32)) & np.uint32(0xF)
        nib = nib.reshape(bn, G)
        i0 = (nib & 3).astype(np.int64)
        i1 = (nib >> 2).astype(np.int64)
        groups = np.zeros((bn, G, 4), dtype=values.dtype)
        np.put_along_axis(groups, i0[..., None], pairs[..., 0:1], axis=-1)
        np.put_along_axis(groups, i1[..., None], pairs[..., 1:2], axis=-1)
        tiles[t] = groups.reshape(bn, bk)
    return from_tiles(tiles, N, K)


# ----------------------------------------------------------------------------
# The layer product
# ----------------------------------------------------------------------------

def gemm_ref(X_bits: np.ndarray, Wm_bits: np.ndarray, dtype: str) -> np.ndarray:
    """Y[M,N] = X . Wm^T in float64 on the exactly widened inputs."""
    X = widen_f64(X_bits, dtype)
    W = widen_f64(Wm_bits, dtype)
    assert X.shape[1] == W.shape[1]
    return X @ W.T


def hybrid_ref(X_bits, W_bits, dtype, tile_map, bn, bk, col_scale=None) -> np.ndarray:
    """The whole layer: mask W by the tile map, then the fp64 product."""
    return gemm_ref(X_bits, masked_weights(W_bits, dtype, tile_map, bn, bk, col_scale), dtype)


def within_tolerance(Y: np.ndarray, Y_ref: np.ndarray, rel: float = 5e-3) -> tuple[bool, float]:
    """Acceptance test max|Y - Y_ref| <= rel * max|Y_ref|; returns (ok, max error / max|Y_ref|)."""
    Y = np.asarray(Y, dtype=np.float64)
    scale = float(np.max(np.abs(Y_ref))) if Y_ref.size else 0.0
    err = float(np.max(np.abs(Y - Y_ref))) if Y_ref.size else 0.0
    if scale == 0.0:
        return err == 0.0, err
    return err <= rel * scale, err / scale


# ----------------------------------------------------------------------------
# Wanda-derived tile maps (Wanda section of the SparseGPT-vs-Wanda page:
# weight magnitude times the input activation of its column; the lowest
# products are the ones removed)
# ----------------------------------------------------------------------------

def column_norms(Xcal_bits: np.ndarray, dtype: str) -> np.ndarray:
    """c_k = ||Xcal[:,k]||_2: squares summed in float64 over rows 0,1,2,... in order, sqrt, one rounding to float32."""
    X = widen_f64(Xcal_bits, dtype)
    acc = np.zeros(X.shape[1], dtype=np.float64)
    for r in range(X.shape[0]):
        acc = acc + X[r] * X[r]
    return np.sqrt(acc).astype(np.float32)


def wanda_tile_cost(W_bits: np.ndarray, dtype: str, col_scale: np.ndarray, bn: int, bk: int) -> np.ndarray:
    """Per-tile float64 cost: the Wanda score mass that making the tile 2:4 would drop.

    For each row r of the tile, the two dropped scores of each group g are added
    (lower index first) and accumulated over g = 0,1,2,... in order; the row sums
    are then accumulated over r = 0,1,2,... in order.  All additions in float64.
    """
    N, K = W_bits.shape
    check_grid(N, K, bn, bk)
    stiles = as_tiles(selection_scores(W_bits, dtype, col_scale), bn, bk).astype(np.float64)
    T = stiles.shape[0]
    G = bk // 4
    cost = np.zeros(T, dtype=np.float64)
    for t in range(T):
        s = stiles[t].reshape(bn, G, 4)
        drop = ~keep_two_of_four(s)
        pos = np.arange(4)
        d_lo = np.take_along_axis(s, np.where(drop, pos, 4).min(axis=-1)[..., None], axis=-1)[..., 0]
        d_hi = np.take_along_axis(s, np.where(drop, pos, -1).max(axis=-1)[..., None], axis=-1)[..., 0]
        pair = d_lo + d_hi                                  # [bn, G]
        row = np.zeros(bn, dtype=np.float64)
        for g in range(G):
            row = row + pair[:, g]
        total = 0.0
        for r in range(bn):
            total = total + row[r]
        cost[t] = total
    return cost


def wanda_tile_map(cost: np.ndarray, n_sparse: int) -> np.ndarray:
    """The n_sparse tiles of lowest cost become 2:4 (ties broken by lower tile number)."""
    cost = np.asarray(cost, dtype=np.float64)
    T = cost.size
    assert 0 <= n_sparse <= T
    order = sorted(range(T), key=lambda t: (cost[t], t))
    m = np.zeros(T, dtype=np.uint8)
    m[order[:n_sparse]] = TILE_SPARSE24
    return m


def silu_mul_ref(G_bits: np.ndarray, U_bits: np.ndarray, dtype: str) -> np.ndarray:
    """H = silu(G) * U in float64 on the exactly widened 16-bit inputs, silu(x) = x / (1 + e^-x):
    the gated MLP step between the gate / up projections and the down projection."""
    g = widen_f64(G_bits, dtype)
    u = widen_f64(U_bits, dtype)
    return g / (1.0 + np.exp(-g)) * u


def gated_ref(G_bits: np.ndarray, Y: np.ndarray, dtype: str) -> np.ndarray:
    """silu(G) * Y in float64, G exactly widened from its 16-bit patterns (or taken as float32 when
    dtype is "f32"), Y a float64 product: the gated-MLP step applied to an unrounded product, as
    when it is done in the product's output stage.  With Y the widened 16-bit U it is silu_mul_ref."""
    g = np.asarray(G_bits, np.float32).astype(np.float64) if dtype == "f32" else widen_f64(G_bits, dtype)
    return g / (1.0 + np.exp(-g)) * np.asarray(Y, np.float64)


def wanda_global_maps(costs, n_sparse: int):
    """Global allocation over several layers (PATCH page, section 4, ablations: a sparsity
    target shared by the whole model beats one per layer): the n_sparse tiles of lowest cost
    among all tiles of all the layers become 2:4, ties broken by layer order then tile number.
    Every layer's tiles must hold the same number of weights, so that counting tiles counts
    weights.  Returns one map per layer."""
    costs = [np.asarray(c, dtype=np.float64) for c in costs]
    allc = np.concatenate(costs)
    flat = wanda_tile_map(allc, n_sparse)         # position in the concatenation = (layer, tile) order
    out, o = [], 0
    for c in costs:
        out.append(flat[o: o + c.size].copy())
        o += c.size
    return out


def density(tile_map: np.ndarray) -> float:
    """Fraction of weights kept: 1 - 0.5 * (fraction of 2:4 tiles) (PATCH section 3: 0..50 % sparsity)."""
    tmap = np.asarray(tile_map)
    return 1.0 - 0.5 * float(np.count_nonzero(tmap)) / tmap.size

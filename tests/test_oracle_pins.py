"""Pins of the CPU oracle to facts that do not come from the oracle itself.

* hand-worked fixtures under tests/golden/ (2:4 choices, codes, a packed layer);
* exhaustive brute force with exact rational arithmetic on tiny layers
  (all six 2:4 patterns of every group, a triple-loop product);
* invariants fixed by the method: density, metadata validity, round trips;
* planted mistakes: a wrong variant of an oracle step must fail a pin.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as wl

GOLD = os.path.join(os.path.dirname(__file__), "golden")
DTYPES = ("f16", "bf16")


def _num(v):
    return -0.0 if v == "-0" else float(v)


def _bits(values, dtype):
    return wl.to_bits(np.array([[_num(v) for v in row] for row in values], dtype=np.float32), dtype) \
        if isinstance(values[0], list) else wl.to_bits(np.array([_num(v) for v in values], dtype=np.float32), dtype)


# ---------------------------------------------------------------------------
# brute force (independent of the oracle): exact rationals, all six patterns
# ---------------------------------------------------------------------------

PAIRS = list(itertools.combinations(range(4), 2))   # the six 2:4 patterns, lexicographic


def exact_value(bits16, dtype):
    """Exact rational value of one stored pattern, decoded field by field."""
    b = int(bits16)
    if dtype == "fp8":   # OCP E4M3: s eeee mmm, bias 7, subnormals, 0x7F / 0xFF NaN
        sign = -1 if b >> 7 else 1
        e, m = (b >> 3) & 0xF, b & 0x7
        assert (b & 0x7F) != 0x7F, "finite inputs only"
        if e == 0:
            return sign * Fraction(m, 8) * Fraction(2) ** -6
        return sign * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    sign = -1 if b >> 15 else 1
    if dtype == "f16":
        e, m, bias, mb = (b >> 10) & 0x1F, b & 0x3FF, 15, 10
        emax = 0x1F
    else:
        e, m, bias, mb = (b >> 7) & 0xFF, b & 0x7F, 127, 7
        emax = 0xFF
    assert e != emax, "finite inputs only"
    if e == 0:
        return sign * Fraction(m, 1 << mb) * Fraction(2) ** (1 - bias)
    return sign * (1 + Fraction(m, 1 << mb)) * Fraction(2) ** (e - bias)


def brute_score(bits16, dtype, c=None):
    """|w|, or |w|*c rounded once to binary32 (the double product of two binary32 values is exact)."""
    a = abs(exact_value(bits16, dtype))
    if c is None:
        return a
    return Fraction(float(np.float32(float(a) * float(np.float32(c)))))


def brute_pair(scores):
    """Largest kept-score sum over the six patterns; ties go to the lexicographically smallest pair."""
    best, best_sum = None, None
    for p in PAIRS:
        s = scores[p[0]] + scores[p[1]]
        if best is None or s > best_sum:
            best, best_sum = p, s
    return best


def brute_place(rows, elem_bytes):
    """Storage order of one tile's rows (equal-length lists), element by element: 16-row panels
    (the whole tile when its row count is not a multiple of 16), 16-byte chunks along a row,
    chunk columns one after another with the panel's rows consecutive inside each."""
    n, w = len(rows), len(rows[0])
    ph = 16 if n % 16 == 0 else n
    ch = 16 // elem_bytes
    out = [None] * (n * w)
    for r in range(n):
        for j in range(w):
            panel, rr = divmod(r, ph)
            cc, e = divmod(j, ch)
            out[panel * ph * w + (cc * ph + rr) * ch + e] = rows[r][j]
    return out


def brute_mask_and_pack(Wb, dtype, tmap, bn, bk, c=None):
    """Pure-Python masking and packing, element by element."""
    N, K = Wb.shape
    Tk = K // bk
    eb = 1 if dtype == "fp8" else 2
    Wm = [[int(Wb[n, k]) for k in range(K)] for n in range(N)]
    values, meta, index = [], [], []
    voff = moff = 0
    for tn in range(N // bn):
        for tk in range(Tk):
            t = tn * Tk + tk
            index.append((voff, moff, int(tmap[t]), 0))
            if tmap[t] == 0:
                values += brute_place([[int(Wb[tn * bn + r, tk * bk + cc]) for cc in range(bk)]
                                       for r in range(bn)], eb)
                voff += bn * bk
                continue
            kept_rows = []
            for r in range(bn):
                n = tn * bn + r
                word, nword = 0, 0
                kept = []
                for g in range(bk // 4):
                    ks = [tk * bk + 4 * g + i for i in range(4)]
                    sc = [brute_score(Wb[n, k], dtype, None if c is None else c[k]) for k in ks]
                    i0, i1 = brute_pair(sc)
                    kept += [int(Wb[n, ks[i0]]), int(Wb[n, ks[i1]])]
                    for i in range(4):
                        if i not in (i0, i1):
                            Wm[n][ks[i]] = 0
                    word |= (i0 | (i1 << 2)) << (4 * (g % 8))
                    if g % 8 == 7:
                        meta.append(word)
                        word, nword = 0, nword + 1
                kept_rows.append(kept)
            values += brute_place(kept_rows, eb)
            voff += bn * bk // 2
            moff += bn * bk // 32
    st = np.uint8 if dtype == "fp8" else np.uint16
    return (np.array(Wm, dtype=st), np.array(values, dtype=st),
            np.array(meta, dtype=np.uint32), np.array(index, dtype=np.uint32).reshape(-1, 4))


def tie_heavy_bits(shape, dtype, g):
    """Small integers and halves with many equal magnitudes, signed zeros, and a few subnormals."""
    choices = np.array([0.0, -0.0, 0.5, -0.5, 1.0, -1.0, 2.0, -2.0, 3.0, 0.25], dtype=np.float32)
    x = choices[g.integers(0, len(choices), size=shape)]
    b = wl.to_bits(x, dtype)
    sub = b.dtype.type(0x0001)   # smallest positive subnormal of each format
    flip = g.random(shape) < 0.03
    b[flip] = sub
    return b


# ---------------------------------------------------------------------------
# golden fixtures
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", DTYPES)
def test_golden_two_of_four_groups(dtype):
    gold = json.load(open(os.path.join(GOLD, "two_of_four_groups.json")))
    for case in gold["groups"]:
        s = oracle.selection_scores(_bits([case["w"]], dtype), dtype)
        keep = oracle.keep_two_of_four(s)[0]
        assert sorted(np.nonzero(keep)[0].tolist()) == case["keep"], case
        i0, i1 = oracle.kept_positions(keep)
        assert int(i0 | (i1 << 2)) == case["nibble"], case
    for case in gold["scaled_groups"]:
        c = np.array(case["c"], dtype=np.float32)
        s = oracle.selection_scores(_bits([case["w"]], dtype), dtype, c)
        keep = oracle.keep_two_of_four(s)[0]
        assert sorted(np.nonzero(keep)[0].tolist()) == case["keep"], case


@pytest.mark.parametrize("dtype", DTYPES)
def test_golden_pack_layer(dtype):
    gold = json.load(open(os.path.join(GOLD, "pack_2x64.json")))
    W = _bits(gold["W"], dtype)
    tmap = np.array(gold["tile_map"], dtype=np.uint8)
    vals, meta, index = oracle.pack(W, dtype, tmap, gold["bn"], gold["bk"])
    assert np.array_equal(vals, _bits(gold["values"], dtype))
    assert [f"{int(w):08X}" for w in meta] == gold["meta_hex"]
    assert index.tolist() == gold["index"]
    Wm = oracle.masked_weights(W, dtype, tmap, gold["bn"], gold["bk"])
    assert np.array_equal(Wm[:, :32], _bits(gold["masked_W_tile0"], dtype))
    assert np.array_equal(Wm[:, 32:], W[:, 32:])
    Y = oracle.gemm_ref(_bits([[1.0] * 64], dtype), Wm, dtype)
    assert Y.tolist() == [gold["masked_row_sums"]]
    assert np.array_equal(oracle.unpack(vals, meta, index, 2, 64, 2, 32), Wm)


# ---------------------------------------------------------------------------
# brute force on tiny layers
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("scaled", [False, True])
def test_brute_force_mask_and_pack(dtype, seed, scaled):
    g = np.random.default_rng(1000 + seed)
    N, K, bn, bk = 8, 64, 4, 32
    W = tie_heavy_bits((N, K), dtype, g) if seed % 2 == 0 else wl.gaussian_bits((N, K), 0.02, dtype, g)
    tmap = (g.random((N // bn) * (K // bk)) < 0.6).astype(np.uint8)
    c = None
    if scaled:
        c = np.array(g.choice([0.0, 0.5, 1.0, 2.0, 3.0, 1.5], size=K), dtype=np.float32)
    Wm_b, vals_b, meta_b, idx_b = brute_mask_and_pack(W, dtype, tmap, bn, bk, c)
    vals, meta, idx = oracle.pack(W, dtype, tmap, bn, bk, c)
    assert np.array_equal(oracle.masked_weights(W, dtype, tmap, bn, bk, c), Wm_b)
    assert np.array_equal(vals, vals_b)
    assert np.array_equal(meta, meta_b)
    assert np.array_equal(idx, idx_b)


def test_brute_force_selection_many_ties():
    g = np.random.default_rng(7)
    s = g.integers(0, 3, size=(4000, 4)).astype(np.float32)   # scores in {0,1,2}: ties everywhere
    keep = oracle.keep_two_of_four(s)
    for row, k in zip(s, keep):
        p = brute_pair([Fraction(float(v)) for v in row])
        assert sorted(np.nonzero(k)[0].tolist()) == list(p)


@pytest.mark.parametrize("dtype", DTYPES)
def test_brute_force_product(dtype):
    g = np.random.default_rng(3)
    M, N, K, bn, bk = 3, 8, 64, 4, 32
    X = wl.gaussian_bits((M, K), 1.0, dtype, g)
    W = wl.gaussian_bits((N, K), 0.02, dtype, g)
    tmap = np.array([1, 0, 0, 1], dtype=np.uint8)
    Wm_b, *_ = brute_mask_and_pack(W, dtype, tmap, bn, bk)
    Y = oracle.hybrid_ref(X, W, dtype, tmap, bn, bk)
    for m in range(M):
        for n in range(N):
            exact = sum(exact_value(X[m, k], dtype) * exact_value(Wm_b[n, k], dtype) for k in range(K))
            mag = sum(abs(exact_value(X[m, k], dtype) * exact_value(Wm_b[n, k], dtype)) for k in range(K))
            assert abs(Fraction(Y[m, n]) - exact) <= K * Fraction(2) ** -52 * mag


def test_exact_value_decoder_matches_numpy():
    # the brute force's own field decoder against numpy's binary16 (and the bf16 embedding in binary32)
    allb = np.arange(0, 1 << 16, 97, dtype=np.uint16)
    f16 = allb[(allb & 0x7C00) != 0x7C00]
    assert all(float(exact_value(b, "f16")) == float(v) for b, v in zip(f16, f16.view(np.float16)))
    bf = allb[(allb & 0x7F80) != 0x7F80]
    assert all(float(exact_value(b, "bf16")) == float(np.uint32(int(b) << 16).view(np.float32)) for b in bf)


# ---------------------------------------------------------------------------
# invariants fixed by the method
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", DTYPES)
def test_all_dense_map_is_plain_product(dtype):
    g = np.random.default_rng(11)
    W = wl.gaussian_bits((128, 256), 0.02, dtype, g)
    X = wl.gaussian_bits((5, 256), 1.0, dtype, g)
    tmap = np.zeros(2 * 4, dtype=np.uint8)
    assert np.array_equal(oracle.masked_weights(W, dtype, tmap, 64, 64), W)
    vals, meta, idx = oracle.pack(W, dtype, tmap, 64, 64)
    assert meta.size == 0 and vals.size == W.size
    assert oracle.density(tmap) == 1.0


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("bn,bk", [(64, 64), (128, 128), (32, 96)])
def test_sparse_invariants(dtype, bn, bk):
    g = np.random.default_rng(bn + bk)
    N, K = 2 * bn, 3 * bk
    W = wl.gaussian_bits((N, K), 0.02, dtype, g)
    W[0, :8] = 0                                           # all-zero groups
    W[1, 4:8] = wl.to_bits(np.array([-0.0, -0.0, 1.0, -0.0], np.float32), dtype)
    tmap = np.array([1, 0, 1, 1, 1, 0], dtype=np.uint8)
    Wm = oracle.masked_weights(W, dtype, tmap, bn, bk)
    vals, meta, idx = oracle.pack(W, dtype, tmap, bn, bk)
    T = tmap.size
    n_s = int(tmap.sum())
    # closed-form sizes and monotone offsets
    assert vals.size == N * K - n_s * bn * bk // 2
    assert meta.size * 4 == n_s * bn * bk // 8
    assert idx.shape == (T, 4) and np.all(np.diff(idx[:, 0].astype(np.int64)) > 0)
    assert np.all(idx[:, 3] == 0) and np.array_equal(idx[:, 2], tmap)
    # density = 1 - 0.5 * sparse fraction, counted on the kept positions
    tiles = oracle.as_tiles(Wm, bn, bk)
    kept = 0
    for t in range(T):
        if tmap[t]:
            groups = tiles[t].reshape(bn, bk // 4, 4)
            nz = (groups & 0x7FFF) != 0
            assert np.all(nz.sum(-1) <= 2)                 # at most two non-zeros per group
            kept += bn * bk // 2
        else:
            kept += bn * bk
    assert Fraction(kept, N * K) == 1 - Fraction(n_s, 2 * T)
    assert math.isclose(oracle.density(tmap), kept / (N * K), rel_tol=1e-15)
    # every code is one of the six patterns; every group has exactly two kept slots
    nibs = (meta[:, None] >> (4 * np.arange(8)).astype(np.uint32)) & 0xF
    assert set(np.unique(nibs).tolist()) <= oracle.VALID_NIBBLES
    # unpack(pack(W)) == mask(W), bit for bit (signed zeros included)
    assert np.array_equal(oracle.unpack(vals, meta, idx, N, K, bn, bk), Wm)
    # -0.0 kept at position 0 of the second group of row 1 survives as 0x8000 when kept
    assert Wm[1, 6] == W[1, 6]


def test_all_sparse_map_equals_uniform_two_of_four():
    g = np.random.default_rng(5)
    W = wl.gaussian_bits((64, 128), 0.02, "bf16", g)
    tmap = np.ones(2, dtype=np.uint8)
    Wm = oracle.masked_weights(W, "bf16", tmap, 64, 64)
    # a whole-matrix 2:4 by magnitude (no tiles at all) gives the same mask
    s = np.abs(oracle.widen_f32(W, "bf16")).reshape(64, 32, 4)
    keep = np.zeros_like(s, dtype=bool)
    order = np.argsort(-s, axis=-1, kind="stable")          # descending, lower index first on ties
    np.put_along_axis(keep, order[..., :2], True, axis=-1)
    ref = np.where(keep.reshape(64, 128), W, np.uint16(0))
    assert np.array_equal(Wm, ref)
    assert oracle.density(tmap) == 0.5


def test_linearity_in_x():
    g = np.random.default_rng(9)
    W = wl.gaussian_bits((64, 64), 0.02, "f16", g)
    tmap = np.array([1], np.uint8)
    X1 = wl.gaussian_bits((2, 64), 1.0, "f16", g)
    X2 = wl.gaussian_bits((2, 64), 1.0, "f16", g)
    Y1 = oracle.hybrid_ref(X1, W, "f16", tmap, 64, 64)
    Y2 = oracle.hybrid_ref(X2, W, "f16", tmap, 64, 64)
    Xs = np.concatenate([X1, X2])
    assert np.allclose(oracle.hybrid_ref(Xs, W, "f16", tmap, 64, 64), np.concatenate([Y1, Y2]), rtol=0, atol=0)


def test_tolerance_rule():
    Yr = np.array([[1.0, -2.0], [0.5, 4.0]])
    assert oracle.within_tolerance(Yr + 0.019, Yr)[0]
    assert not oracle.within_tolerance(Yr + 0.021, Yr)[0]


# ---------------------------------------------------------------------------
# Wanda-derived maps
# ---------------------------------------------------------------------------

def test_column_norms_exact():
    g = np.random.default_rng(21)
    X = wl.gaussian_bits((16, 40), 1.0, "bf16", g)
    c = oracle.column_norms(X, "bf16")
    for k in range(40):
        ss = sum(exact_value(X[r, k], "bf16") ** 2 for r in range(16))
        exact = math.sqrt(ss)                       # float sqrt of a float-rounded rational: within 1 ulp64
        assert abs(float(c[k]) - exact) <= float(np.spacing(np.float32(exact)))


def test_wanda_cost_and_map_brute_force():
    g = np.random.default_rng(31)
    N, K, bn, bk = 8, 64, 4, 32
    W = wl.gaussian_bits((N, K), 0.02, "bf16", g)
    c = np.abs(g.standard_normal(K)).astype(np.float32) * np.float32(3)
    cost = oracle.wanda_tile_cost(W, "bf16", c, bn, bk)
    Tk = K // bk
    for t in range(cost.size):
        tn, tk = divmod(t, Tk)
        exact = Fraction(0)
        for r in range(bn):
            for gi in range(bk // 4):
                ks = [tk * bk + 4 * gi + i for i in range(4)]
                sc = [brute_score(W[tn * bn + r, k], "bf16", c[k]) for k in ks]
                p = brute_pair(sc)
                exact += sum(sc[i] for i in range(4) if i not in p)
        assert abs(Fraction(cost[t]) - exact) <= Fraction(2) ** -40 * exact
    for n_s in (0, 1, 3, cost.size):
        m = oracle.wanda_tile_map(cost, n_s)
        assert int(m.sum()) == n_s
        sel, rest = np.nonzero(m)[0], np.nonzero(m == 0)[0]
        for a in sel:
            for b in rest:
                assert (cost[a], a) < (cost[b], b)


# ---------------------------------------------------------------------------
# planted mistakes: a wrong variant of an oracle step must fail a pin
# ---------------------------------------------------------------------------

def test_planted_mistakes_are_caught(monkeypatch):
    gold = json.load(open(os.path.join(GOLD, "pack_2x64.json")))
    W = _bits(gold["W"], "bf16")
    tmap = np.array(gold["tile_map"], dtype=np.uint8)

    def golden_ok():
        vals, meta, index = oracle.pack(W, "bf16", tmap, 2, 32)
        return (np.array_equal(vals, _bits(gold["values"], "bf16"))
                and [f"{int(w):08X}" for w in meta] == gold["meta_hex"])

    assert golden_ok()
    # (1) tie-break toward the higher index
    real_keep = oracle.hybrid.keep_two_of_four

    def keep_high_ties(scores):
        return real_keep(np.asarray(scores)[..., ::-1])[..., ::-1]
    monkeypatch.setattr(oracle.hybrid, "keep_two_of_four", keep_high_ties)
    assert not golden_ok()
    monkeypatch.setattr(oracle.hybrid, "keep_two_of_four", real_keep)
    # (2) kept pair stored higher index first (swapped code fields)
    real_pos = oracle.hybrid.kept_positions
    monkeypatch.setattr(oracle.hybrid, "kept_positions", lambda k: real_pos(k)[::-1])
    assert not golden_ok()
    monkeypatch.setattr(oracle.hybrid, "kept_positions", real_pos)
    # (3) signed score (forgetting the magnitude)
    real_scores = oracle.hybrid.selection_scores
    monkeypatch.setattr(oracle.hybrid, "selection_scores",
                        lambda Wb, dt, c=None: oracle.widen_f32(Wb, dt))
    assert not golden_ok()
    monkeypatch.setattr(oracle.hybrid, "selection_scores", real_scores)
    assert golden_ok()


# ---------------------------------------------------------------------------
# packing from a given element mask
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", DTYPES)
def test_golden_pack_from_mask(dtype):
    gold = json.load(open(os.path.join(GOLD, "pack_masked_2x64.json")))
    N, K, bn, bk = gold["N"], gold["K"], gold["bn"], gold["bk"]
    W = _bits([[c + 1 for c in range(K)], [-(c + 1) for c in range(K)]], dtype)
    mask = np.zeros((N, K), np.uint8)
    mask[:, 32:] = np.arange(32) % 3 == 0          # ignored: the tile is dense
    for r, key in enumerate(("mask_pairs_row0", "mask_pairs_row1")):
        for g, (i0, i1) in enumerate(gold[key]):
            mask[r, 4 * g + i0] = mask[r, 4 * g + i1] = 1
    tmap = np.array(gold["tile_map"], np.uint8)
    vals, meta, index, bad = oracle.pack_masked(W, dtype, tmap, mask, bn, bk)
    assert bad == 0
    assert [f"{int(w):08X}" for w in meta] == gold["meta_hex"]
    assert np.array_equal(vals[:32], _bits(gold["values_tile0"], dtype))
    # the dense tile: chunks of 8 values, chunk column by chunk column, the two rows consecutive
    assert np.array_equal(vals[32:], np.concatenate([W[r, 32 + 8 * c: 40 + 8 * c] for c in range(4) for r in range(2)]))


def _random_pair_mask(N, K, g):
    mask = np.zeros((N, K // 4, 4), np.uint8)
    pick = g.integers(0, 6, size=(N, K // 4))
    for n in range(6):
        i0, i1 = PAIRS[n]
        sel = pick == n
        mask[sel, i0] = 1
        mask[sel, i1] = 1
    return mask.reshape(N, K)


@pytest.mark.parametrize("dtype", DTYPES)
def test_pack_from_well_formed_mask_brute_force(dtype):
    g = np.random.default_rng(41)
    N, K, bn, bk = 8, 128, 4, 32
    W = wl.gaussian_bits((N, K), 0.02, dtype, g)
    mask = _random_pair_mask(N, K, g)
    tmap = (g.random((N // bn) * (K // bk)) < 0.5).astype(np.uint8)
    vals, meta, index, bad = oracle.pack_masked(W, dtype, tmap, mask, bn, bk)
    assert bad == 0
    back = oracle.unpack(vals, meta, index, N, K, bn, bk)
    # the expected value of the GPU masked unpack and of the product over a mask-packed weight
    Wm = oracle.masked_weights_from_mask(W, tmap, mask, bn, bk)
    Tk = K // bk
    for n in range(N):
        for k in range(K):
            sparse = tmap[(n // bn) * Tk + k // bk] == 1
            want = W[n, k] if (not sparse or mask[n, k]) else 0
            assert back[n, k] == want
            assert Wm[n, k] == want
    # codes name the marked positions (found here group by group with np.nonzero)
    for t in np.nonzero(tmap)[0]:
        vo, mo, _, _ = index[t]
        tn, tk = divmod(int(t), Tk)
        for r in range(bn):
            for gi in range(bk // 4):
                pos = np.nonzero(mask[tn * bn + r, tk * bk + 4 * gi: tk * bk + 4 * gi + 4])[0]
                word = int(meta[mo + r * (bk // 32) + gi // 8])
                assert (word >> (4 * (gi % 8))) & 0xF == int(pos[0]) | (int(pos[1]) << 2)


def _malformed_case(seed=43):
    """A 2:4 layer whose mask marks any number of weights per group, with marked entries of
    arbitrary nonzero value (nonzero = keep), and the pair each group must keep."""
    g = np.random.default_rng(seed)
    N, K, bn, bk = 4, 64, 4, 32
    W = wl.gaussian_bits((N, K), 0.02, "bf16", g)
    marked = g.random((N, K)) < 0.5                  # any number marked per group
    mask = np.where(marked, g.integers(1, 256, size=(N, K)), 0).astype(np.uint8)
    tmap = np.array([1, 1], np.uint8)
    want = np.zeros((N, K // 4, 4), np.uint16)
    groups = marked.reshape(N, K // 4, 4)
    for n in range(N):
        for gi in range(K // 4):
            order = [i for i in range(4) if groups[n, gi, i]] + [i for i in range(4) if not groups[n, gi, i]]
            kept = sorted(order[:2])              # marked first, lower index first among equals
            want[n, gi, kept] = W[n, 4 * gi + np.array(kept)]
    return W, mask, tmap, (N, K, bn, bk), groups, want.reshape(N, K)


def test_pack_from_malformed_mask_brute_force():
    W, mask, tmap, (N, K, bn, bk), groups, want = _malformed_case()
    vals, meta, index, bad = oracle.pack_masked(W, "bf16", tmap, mask, bn, bk)
    assert bad == int(np.count_nonzero(groups.sum(axis=-1) != 2))
    assert np.array_equal(oracle.unpack(vals, meta, index, N, K, bn, bk), want)
    assert np.array_equal(oracle.masked_weights_from_mask(W, tmap, mask, bn, bk), want)


def test_planted_mask_mistakes_are_caught(monkeypatch):
    # masked_weights_from_mask must fail the brute-force pin when its selection is wrong
    W, mask, tmap, (N, K, bn, bk), _, want = _malformed_case()

    def pin_ok():
        return np.array_equal(oracle.masked_weights_from_mask(W, tmap, mask, bn, bk), want)

    assert pin_ok()
    real = oracle.hybrid.mask_scores
    # (1) the mask's raw byte values used as the score instead of marked / unmarked
    monkeypatch.setattr(oracle.hybrid, "mask_scores", lambda m: np.asarray(m).astype(np.float32))
    assert not pin_ok()
    # (2) marked and unmarked swapped (the mask read as a drop mask)
    monkeypatch.setattr(oracle.hybrid, "mask_scores", lambda m: (np.asarray(m) == 0).astype(np.float32))
    assert not pin_ok()
    monkeypatch.setattr(oracle.hybrid, "mask_scores", real)
    # (3) ties among marked weights to the higher index
    real_keep = oracle.hybrid.keep_two_of_four
    monkeypatch.setattr(oracle.hybrid, "keep_two_of_four", lambda s: real_keep(np.asarray(s)[..., ::-1])[..., ::-1])
    assert not pin_ok()
    monkeypatch.setattr(oracle.hybrid, "keep_two_of_four", real_keep)
    assert pin_ok()


@pytest.mark.parametrize("dtype", DTYPES)
def test_pack_from_magnitude_mask_equals_magnitude_pack(dtype):
    # the keep mask of a magnitude pack (read back from its codes), given as the mask, packs the same
    g = np.random.default_rng(47)
    N, K, bn, bk = 64, 256, 32, 64
    W = wl.gaussian_bits((N, K), 0.02, dtype, g)
    tmap = (g.random((N // bn) * (K // bk)) < 0.5).astype(np.uint8)
    _, m, idx = oracle.pack(W, dtype, np.ones_like(tmap), bn, bk)   # magnitude 2:4 in every tile
    mask = np.zeros((N, K), np.uint8)
    for t in range(idx.shape[0]):
        tn, tk = divmod(t, K // bk)
        words = m[idx[t, 1]: idx[t, 1] + bn * bk // 32].reshape(bn, bk // 32)
        for r in range(bn):
            for gi in range(bk // 4):
                code = (int(words[r, gi // 8]) >> (4 * (gi % 8))) & 0xF
                mask[tn * bn + r, tk * bk + 4 * gi + (code & 3)] = 1
                mask[tn * bn + r, tk * bk + 4 * gi + (code >> 2)] = 1
    a = oracle.pack(W, dtype, tmap, bn, bk)
    b = oracle.pack_masked(W, dtype, tmap, mask, bn, bk)
    assert b[3] == 0
    assert all(np.array_equal(x, y) for x, y in zip(a, b[:3]))


# ---------------------------------------------------------------------------
# global (cross-layer) Wanda allocation
# ---------------------------------------------------------------------------

def test_wanda_global_allocation_brute_force():
    g = np.random.default_rng(53)
    sizes = [12, 30, 7]
    costs = [np.round(g.random(n) * 8) / 4 for n in sizes]      # many exact ties, across layers too
    for n_s in (0, 1, 9, 25, sum(sizes)):
        maps = oracle.wanda_global_maps(costs, n_s)
        assert [m.size for m in maps] == sizes
        assert sum(int(m.sum()) for m in maps) == n_s
        keyed = [(float(costs[l][t]), l, t, int(maps[l][t])) for l in range(3) for t in range(sizes[l])]
        sparse = [k[:3] for k in keyed if k[3] == 1]
        dense = [k[:3] for k in keyed if k[3] == 0]
        assert all(a < b for a in sparse for b in dense)        # (cost, layer, tile) order
    # one layer: the global allocation is the per-layer one
    assert np.array_equal(oracle.wanda_global_maps([costs[1]], 11)[0], oracle.wanda_tile_map(costs[1], 11))


def test_silu_mul_closed_forms():
    # silu(x) = x * sigmoid(x).  Pins that are not the formula: tabulated logistic values
    # (sigmoid(1) = 0.7310585786300049, sigmoid(2) = 0.8807970779778823, sigmoid(-1) = 0.2689414213699951),
    # the odd-part identity silu(x) - silu(-x) = x, the asymptotes, and linearity in U.
    xs = np.array([1.0, 2.0, -1.0, 16.0, -16.0], np.float32)
    one = wl.to_bits(np.ones_like(xs), "f16")
    h = oracle.silu_mul_ref(wl.to_bits(xs, "f16"), one, "f16")
    assert np.allclose(h[:3], [0.7310585786300049, 2 * 0.8807970779778823, -0.2689414213699951], rtol=1e-15, atol=0)
    assert abs(h[3] - 16.0) < 2e-6 and abs(h[4]) < 2e-6
    g = np.random.default_rng(59)
    x = wl.gaussian_bits((256,), 3.0, "bf16", g)
    negx = x ^ np.uint16(0x8000)                           # exact negation of the bit pattern
    ones = wl.to_bits(np.ones(256, np.float32), "bf16")
    d = oracle.silu_mul_ref(x, ones, "bf16") - oracle.silu_mul_ref(negx, ones, "bf16")
    assert np.allclose(d, oracle.widen_f64(x, "bf16"), rtol=1e-14, atol=1e-300)
    assert oracle.silu_mul_ref(wl.to_bits(np.zeros(3, np.float32), "bf16"), ones[:3], "bf16").tolist() == [0.0] * 3
    three = wl.to_bits(np.full(256, 3.0, np.float32), "bf16")
    assert np.allclose(oracle.silu_mul_ref(x, three, "bf16"), 3.0 * oracle.silu_mul_ref(x, ones, "bf16"),
                       rtol=1e-15, atol=0)


def test_gated_ref_reduces_to_silu_mul():
    # the gated output stage on an unrounded product: with the product equal to a 16-bit U it is the
    # elementwise step exactly; a product of 1.0 gives the tabulated logistic values; fp32 G (y_dtype
    # f32) is taken as is
    g = np.random.default_rng(61)
    G = wl.gaussian_bits((64, 48), 2.0, "bf16", g)
    U = wl.gaussian_bits((64, 48), 1.0, "bf16", g)
    assert np.array_equal(oracle.gated_ref(G, oracle.widen_f64(U, "bf16"), "bf16"), oracle.silu_mul_ref(G, U, "bf16"))
    one = np.ones(3)
    assert np.allclose(oracle.gated_ref(np.array([1.0, 2.0, -1.0], np.float32), one, "f32"),
                       [0.7310585786300049, 2 * 0.8807970779778823, -0.2689414213699951], rtol=1e-15, atol=0)


# ---------------------------------------------------------------------------
# the 8-bit (OCP E4M3) variant
# ---------------------------------------------------------------------------

def test_e4m3_values_from_the_format_definition():
    # hand-derived from the field layout s eeee mmm, bias 7
    table = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x30: 0.5, 0x38: 1.0,
             0x3C: 1.5, 0x40: 2.0, 0x44: 3.0, 0x48: 4.0, 0x77: 240.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
    got = oracle.e4m3_value(np.array(list(table), dtype=np.uint8))
    assert np.array_equal(got, np.array(list(table.values())))
    z = oracle.e4m3_value(np.array([0x80], dtype=np.uint8))
    assert z[0] == 0.0 and np.signbit(z[0])
    assert np.all(np.isnan(oracle.e4m3_value(np.array([0x7F, 0xFF], dtype=np.uint8))))


def test_e4m3_decode_matches_torch_for_every_byte():
    torch = pytest.importorskip("torch")
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_value(b)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    # and the brute force's own field decoder agrees with torch on every finite byte
    assert all(float(exact_value(int(x), "fp8")) == float(r) for x, r in zip(b[~nan], ref[~nan]))


def test_e4m3_rounding_of_the_input_generator_is_nearest():
    # the generator's rounding picks, for every input, a representable value at the least distance
    g = np.random.default_rng(5)
    x = (g.standard_normal(20000) * np.exp(g.uniform(-10, 6, 20000))).astype(np.float32)
    vals = oracle.e4m3_value(np.arange(256, dtype=np.uint8))
    finite = np.sort(np.unique(vals[~np.isnan(vals)]))
    q = oracle.e4m3_value(wl.to_bits(x, "fp8"))
    xs = np.clip(x.astype(np.float64), -448.0, 448.0)
    best = np.min(np.abs(finite[None, :] - xs[:, None]), axis=1)
    assert np.array_equal(np.abs(q - xs), best)


def fp8_tie_heavy(shape, g):
    choices = np.array([0.0, -0.0, 0.5, -0.5, 1.0, -1.0, 2.0, -2.0, 3.0, 0.25, 448.0, 2.0 ** -9], dtype=np.float32)
    return wl.to_bits(choices[g.integers(0, len(choices), size=shape)], "fp8")


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("scaled", [False, True])
def test_brute_force_mask_and_pack_fp8(seed, scaled):
    g = np.random.default_rng(2000 + seed)
    N, K, bn, bk = 8, 64, 4, 32
    W = fp8_tie_heavy((N, K), g) if seed % 2 == 0 else wl.gaussian_bits((N, K), 1.0, "fp8", g)
    tmap = (g.random((N // bn) * (K // bk)) < 0.6).astype(np.uint8)
    c = np.array(g.choice([0.0, 0.5, 1.0, 2.0, 3.0, 1.5], size=K), dtype=np.float32) if scaled else None
    Wm_b, vals_b, meta_b, idx_b = brute_mask_and_pack(W, "fp8", tmap, bn, bk, c)
    vals, meta, idx = oracle.pack(W, "fp8", tmap, bn, bk, c)
    assert vals.dtype == np.uint8
    assert np.array_equal(oracle.masked_weights(W, "fp8", tmap, bn, bk, c), Wm_b)
    assert np.array_equal(vals, vals_b)
    assert np.array_equal(meta, meta_b)
    assert np.array_equal(idx, idx_b)
    assert np.array_equal(oracle.unpack(vals, meta, idx, N, K, bn, bk), Wm_b)


def test_brute_force_product_fp8():
    g = np.random.default_rng(4)
    M, N, K, bn, bk = 3, 8, 64, 4, 32
    X = wl.gaussian_bits((M, K), 1.0, "fp8", g)
    W = wl.gaussian_bits((N, K), 1.0, "fp8", g)
    tmap = np.array([0, 1, 1, 0], dtype=np.uint8)
    Wm_b, *_ = brute_mask_and_pack(W, "fp8", tmap, bn, bk)
    Y = oracle.hybrid_ref(X, W, "fp8", tmap, bn, bk)
    for m in range(M):
        for n in range(N):
            # products of two E4M3 values have at most 8 significant bits: the fp64 sum is exact
            exact = sum(exact_value(X[m, k], "fp8") * exact_value(Wm_b[n, k], "fp8") for k in range(K))
            assert Fraction(Y[m, n]) == exact


def test_fp8_packed_sizes_and_invariants():
    g = np.random.default_rng(9)
    N, K, bn, bk = 256, 384, 128, 128
    W = wl.gaussian_bits((N, K), 1.0, "fp8", g)
    tmap = np.array([1, 0, 1, 1, 0, 0], dtype=np.uint8)
    vals, meta, idx = oracle.pack(W, "fp8", tmap, bn, bk)
    _, sizes = oracle.plan(tmap, N, K, bn, bk, elem_bytes=1)
    assert vals.size == sizes["values"] == sizes["values_bytes"] == 3 * bn * bk // 2 + 3 * bn * bk
    assert meta.size == 3 * bn * bk // 32
    nib = (meta[:, None] >> (4 * np.arange(8, dtype=np.uint32))) & np.uint32(0xF)
    assert set(np.unique(nib).tolist()) <= set(oracle.VALID_NIBBLES)
    Wm = oracle.masked_weights(W, "fp8", tmap, bn, bk)
    assert np.array_equal(oracle.unpack(vals, meta, idx, N, K, bn, bk), Wm)
    t = oracle.as_tiles(Wm, bn, bk)
    nz = (oracle.e4m3_value(t) != 0).reshape(t.shape[0], bn, bk // 4, 4).sum(-1)
    assert np.all(nz[tmap == 1] <= 2)

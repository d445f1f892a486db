"""Seeded synthetic inputs for the hybrid tile-sparse (dense / 2:4) linear layer.

This module holds NO arithmetic of the method itself: it only draws random
numbers, rounds them to the storage type (16-bit, or 8-bit E4M3), and draws
tile maps.  Both the
CPU oracle (through the tests) and the GPU library (through the tests, the
benchmark and the smoke check) take their inputs from here, so neither side
ever supplies inputs to the other.

Workload shapes follow the layers of LLaMA-2 7B / 13B, the models the PATCH
page ("PATCH: Learnable Tile-level Hybrid Sparsity for LLMs", section 4,
experimental results) evaluates on; trained weights and evaluation datasets are
not available, so Gaussian layers of the same shapes stand in for them
(weights ~ N(0, 0.02), activations ~ N(0, 1), calibration activations with 1 %
outlier columns scaled by 20).

Seeds: every buffer is drawn from ``SeedSequence([cfg_id, layer_id, tag])``
with tag X=0, W=1, MAP=2, CALIB=3, OUTLIER=4.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import numpy as np

TAG_X, TAG_W, TAG_MAP, TAG_CALIB, TAG_OUTLIER = 0, 1, 2, 3, 4

F16, BF16, FP8 = "f16", "bf16", "fp8"


def rng(cfg_id: int, layer_id: int, tag: int, extra: Sequence[int] = ()) -> np.random.Generator:
    """PCG64 generator seeded by SeedSequence([cfg_id, layer_id, tag, *extra])."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg_id, layer_id, tag, *extra])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE binary16 (numpy's RNE cast, subnormals kept); returns uint16 bits."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to OCP E4M3 (round to nearest, ties to even; magnitudes past
    448, the largest finite value, saturate to 448); returns uint8 bits."""
    a64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    neg = np.signbit(a64)
    a = np.minimum(np.abs(a64), 448.0)
    _, ex = np.frexp(np.maximum(a, 2.0 ** -6))            # a = f * 2^ex with f in [0.5, 1)
    q = np.ldexp(1.0, ex - 1 - 3)                          # spacing of the 3-bit mantissa at a
    r = np.minimum(np.round(a / q) * q, 448.0)             # numpy rounds halves to even
    _, er = np.frexp(np.maximum(r, 2.0 ** -6))
    e = er - 1                                             # exponent of r (at least -6)
    sub = r < 2.0 ** -6
    m = np.where(sub, r * 2.0 ** 9, (np.ldexp(r, -e) - 1.0) * 8.0)
    ebits = np.where(sub, 0, e + 7)
    bits = (neg.astype(np.int64) << 7) | (ebits.astype(np.int64) << 3) | np.round(m).astype(np.int64)
    return bits.astype(np.uint8)


def to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == BF16:
        return f32_to_bf16_bits(x)
    if dtype == F16:
        return f32_to_f16_bits(x)
    if dtype == FP8:
        return f32_to_e4m3_bits(x)
    raise ValueError(dtype)


def gaussian_bits(shape: Tuple[int, ...], sigma: float, dtype: str, g: np.random.Generator) -> np.ndarray:
    """N(0, sigma^2) drawn in float32 and rounded to the storage type (uint16 or uint8 bits)."""
    x = g.standard_normal(size=shape, dtype=np.float32) * np.float32(sigma)
    return to_bits(x, dtype)


def bernoulli_map(n_tiles: int, p: float, g: np.random.Generator) -> np.ndarray:
    """Each tile independently sparse (1) with probability p."""
    return (g.random(n_tiles) < p).astype(np.uint8)


def exact_map(n_tiles: int, n_sparse: int, g: np.random.Generator) -> np.ndarray:
    """Exactly n_sparse tiles marked sparse (1), positions from a seeded permutation."""
    m = np.zeros(n_tiles, dtype=np.uint8)
    m[g.permutation(n_tiles)[:n_sparse]] = 1
    return m


TAG_MASK = 5


def pair_mask(N: int, K: int, g: np.random.Generator) -> np.ndarray:
    """uint8 keep mask [N,K] marking, in every group of four along K, one of the six pairs
    (uniformly at random): a stand-in for a frozen 2:4 pattern from a one-shot pruning method."""
    pairs = np.array([[1, 1, 0, 0], [1, 0, 1, 0], [1, 0, 0, 1], [0, 1, 1, 0], [0, 1, 0, 1], [0, 0, 1, 1]], np.uint8)
    return pairs[g.integers(0, 6, size=(N, K // 4))].reshape(N, K)


def layer_pair_mask(cfg: "Config", layer: "Layer") -> np.ndarray:
    """The seeded pair mask of a named layer."""
    return pair_mask(layer.N, layer.K, rng(cfg.cfg_id, layer.layer_id, TAG_MASK))


def calib_bits(rows: int, K: int, dtype: str, cfg_id: int, layer_id: int,
               outlier_frac: float = 0.01, outlier_scale: float = 20.0) -> np.ndarray:
    """Calibration activations [rows, K] ~ N(0,1) with round(outlier_frac*K) columns scaled by outlier_scale."""
    x = rng(cfg_id, layer_id, TAG_CALIB).standard_normal(size=(rows, K), dtype=np.float32)
    n_out = int(round(outlier_frac * K))
    cols = rng(cfg_id, layer_id, TAG_OUTLIER).choice(K, size=n_out, replace=False)
    x[:, cols] *= np.float32(outlier_scale)
    return to_bits(x, dtype)


@dataclasses.dataclass(frozen=True)
class Layer:
    """One linear layer Y[M,N] = X[M,K] . W[N,K]^T with its tile map recipe."""
    name: str
    N: int
    K: int
    dtype: str
    bn: int
    bk: int
    map_kind: str            # "bernoulli" | "exact" | "wanda"
    p: float                 # bernoulli probability, exact sparse-tile fraction, or wanda overall sparsity
    layer_id: int = 0
    calib_id: int = 0        # which calibration input (layers sharing an input share it)

    @property
    def T_n(self) -> int:
        return self.N // self.bn

    @property
    def T_k(self) -> int:
        return self.K // self.bk

    @property
    def T(self) -> int:
        return self.T_n * self.T_k

    @property
    def n_sparse_target(self) -> int:
        if self.map_kind == "exact":
            return int(round(self.p * self.T))
        if self.map_kind == "wanda":
            # overall sparsity rho = 0.5 * (sparse-tile fraction)  =>  n_s = round(2 rho T)
            return int(round(2.0 * self.p * self.T))
        raise ValueError("bernoulli maps have no fixed sparse count")


@dataclasses.dataclass(frozen=True)
class Config:
    cfg_id: int
    name: str
    layers: Tuple[Layer, ...]
    Ms: Tuple[int, ...]
    x_sigma: float = 1.0
    w_sigma: float = 0.02
    calib_rows: int = 128


def _sweep_layers() -> Tuple[Layer, ...]:
    return tuple(Layer(f"sweep_p{p:g}", 4096, 4096, F16, 128, 128, "exact", p, layer_id=i)
                 for i, p in enumerate((0.0, 0.25, 0.5, 0.75, 1.0)))


def _block_layers() -> Tuple[Layer, ...]:
    d, f = 4096, 11008
    spec = [("q", d, d, 0), ("k", d, d, 0), ("v", d, d, 0), ("o", d, d, 1),
            ("gate", f, d, 2), ("up", f, d, 2), ("down", d, f, 3)]
    return tuple(Layer(n, N, K, BF16, 128, 128, "wanda", 0.30, layer_id=i, calib_id=c)
                 for i, (n, N, K, c) in enumerate(spec))


CONFIGS: Tuple[Config, ...] = (
    Config(1, "tiny", (Layer("tiny", 256, 256, F16, 64, 64, "bernoulli", 0.5),), (8,)),
    Config(2, "7b_up", (Layer("up_proj", 11008, 4096, BF16, 128, 128, "exact", 0.25),), (1, 16, 2048)),
    Config(3, "13b", (Layer("sq_5120", 5120, 5120, BF16, 128, 128, "exact", 0.5, layer_id=0),
                      Layer("up_13824", 13824, 5120, BF16, 128, 128, "exact", 0.5, layer_id=1)), (1, 16, 4096)),
    Config(4, "sweep", _sweep_layers(), (1, 2048)),
    Config(5, "7b_block", _block_layers(), (2048,)),
    # prune then quantize: the 7B up-projection with 8-bit E4M3 weights and activations, drawn at
    # unit scale (a per-tensor scale would sit outside the product)
    Config(6, "7b_up_fp8", (Layer("up_proj_fp8", 11008, 4096, FP8, 128, 128, "exact", 0.25),), (1, 16, 2048),
           x_sigma=1.0, w_sigma=1.0),
)


def config(name_or_id) -> Config:
    for c in CONFIGS:
        if c.name == name_or_id or c.cfg_id == name_or_id:
            return c
    raise KeyError(name_or_id)


def weight_bits(cfg: Config, layer: Layer) -> np.ndarray:
    """W[N,K] as uint16 bits of the layer's 16-bit type, ~ N(0, w_sigma^2)."""
    return gaussian_bits((layer.N, layer.K), cfg.w_sigma, layer.dtype, rng(cfg.cfg_id, layer.layer_id, TAG_W))


def activation_bits(cfg: Config, layer: Layer, M: int, M_max: Optional[int] = None) -> np.ndarray:
    """X[M,K] as uint16 bits: the first M rows of one [M_max,K] draw, so every M of a layer shares rows."""
    M_max = max(cfg.Ms) if M_max is None else M_max
    if M > M_max:
        raise ValueError("M larger than the configured maximum")
    x = gaussian_bits((M_max, layer.K), cfg.x_sigma, layer.dtype, rng(cfg.cfg_id, layer.layer_id, TAG_X))
    return np.ascontiguousarray(x[:M])


def tile_map(cfg: Config, layer: Layer) -> np.ndarray:
    """uint8[T] tile map in row-major tile order (1 = 2:4 sparse, 0 = dense) for bernoulli/exact layers."""
    g = rng(cfg.cfg_id, layer.layer_id, TAG_MAP)
    if layer.map_kind == "bernoulli":
        return bernoulli_map(layer.T, layer.p, g)
    if layer.map_kind == "exact":
        return exact_map(layer.T, layer.n_sparse_target, g)
    raise ValueError("wanda maps are derived from the weights and calibration data, not drawn")


def layer_calib_bits(cfg: Config, layer: Layer) -> np.ndarray:
    """Calibration activations [calib_rows, K] shared by every layer with the same calib_id."""
    return calib_bits(cfg.calib_rows, layer.K, layer.dtype, cfg.cfg_id, 100 + layer.calib_id)


def small_layer(N: int, K: int, dtype: str, bn: int, bk: int, seed: int) -> Tuple[np.ndarray, np.ndarray]:
    """Ad-hoc (W bits, generator) pair for parity cases off the named configurations."""
    g = rng(9000 + seed, 0, TAG_W)
    return gaussian_bits((N, K), 0.02, dtype, g), g


def numpy_of_bits(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float32 view of 16-bit patterns (for inspection and for feeding float APIs; 8-bit
    patterns go to torch as float8_e4m3fn instead)."""
    if dtype == F16:
        return bits.view(np.float16).astype(np.float32)
    if dtype == BF16:
        return (bits.astype(np.uint32) << 16).view(np.float32)
    raise ValueError(dtype)


def list_parity_cases() -> List[Tuple[Config, Layer, int]]:
    """Every (config, layer, M) triple of the named workloads."""
    return [(c, l, M) for c in CONFIGS for l in c.layers for M in c.Ms]

"""Seeded synthetic inputs shared by the HIP path's tests, the oracle's tests
and the benchmark.

This module draws random numbers and rounds them to the storage type; it
holds none of the attention arithmetic.  Every array is float32 whose values
are exactly representable in the requested storage type, so the GPU receives
them losslessly (bfloat16 bits) and the oracle widens the same values
exactly to float64.

Distributions (standard for these layers, stated once here): activations
q_nope, q_pe, c_kv, k_pe ~ N(0, 1); weights W_UK [H, n, r] and W_UV [H, r, v]
~ N(0, 1/r); scale = 1/sqrt(n + rope).  Draw order from one PCG64 stream:
(per-sequence lengths, when drawn), q_nope, q_pe, c_kv, k_pe, W_UK, W_UV.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16 (ties to even), as float32."""
    return bf16_to_f32(bf16_bits(x))


@dataclass(frozen=True)
class Workload:
    """One MLA attention workload: geometry, batch and storage type."""
    name: str
    r: int
    n: int
    v: int
    rope: int
    heads: int
    batch: int
    L: int
    kv: int | None = None              # fixed Kv per sequence (None: drawn)
    kv_range: tuple[int, int] | None = None  # inclusive uniform range for drawn Kv
    dtype: str = "bf16"                # "f32" or "bf16"
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.n + self.rope)


# Workloads (geometry r/n/v/rope, heads, batch, cached Kv, query rows L, storage):
WORKLOADS = {
    # DeepSeek-V3 MLA geometry, 16 heads, one sequence of 512, 4 rows, float32.
    "dsv3_h16_kv512_l4_f32": Workload("dsv3_h16_kv512_l4_f32", 512, 128, 128, 64, 16, 1, 4,
                                      kv=512, dtype="f32", seed=1),
    # DeepSeek-V3 geometry, 128 heads, one sequence of 8192, 8 rows, bfloat16.
    "dsv3_h128_kv8192_l8_bf16": Workload("dsv3_h128_kv8192_l8_bf16", 512, 128, 128, 64, 128, 1, 8,
                                         kv=8192, dtype="bf16", seed=2),
    # GLM-4.7-Flash-like geometry 512/192/256, 32 heads, cache 8192 (rows L swept).
    "glm47_h32_kv8192_bf16": Workload("glm47_h32_kv8192_bf16", 512, 192, 256, 64, 32, 1, 8,
                                      kv=8192, dtype="bf16", seed=3),
    # GLM-5.3-Flash-like geometry 512/256/256, 64 heads, cache 32768, 16 rows.
    "glm53_h64_kv32768_l16_bf16": Workload("glm53_h64_kv32768_l16_bf16", 512, 256, 256, 64, 64, 1, 16,
                                           kv=32768, dtype="bf16", seed=4),
    # DeepSeek-V3 geometry, 128 heads, 32 sequences with Kv ~ U[1024, 32768], 8 rows each.
    "dsv3_h128_b32_varlen_l8_bf16": Workload("dsv3_h128_b32_varlen_l8_bf16", 512, 128, 128, 64, 128, 32, 8,
                                             kv_range=(1024, 32768), dtype="bf16", seed=5),
    # 16-head shares of the two DeepSeek-V3 workloads above (one GPU's heads when 8 GPUs
    # split the 128 heads): the latent cache is the same size, the rows 8x fewer, so HBM
    # rather than MFMA bounds the attention.  Same seeds, so the batch draws the same lengths.
    "dsv3_h16_kv8192_l8_bf16": Workload("dsv3_h16_kv8192_l8_bf16", 512, 128, 128, 64, 16, 1, 8,
                                        kv=8192, dtype="bf16", seed=2),
    "dsv3_h16_b32_varlen_l8_bf16": Workload("dsv3_h16_b32_varlen_l8_bf16", 512, 128, 128, 64, 16, 32, 8,
                                            kv_range=(1024, 32768), dtype="bf16", seed=5),
}

# Query-row counts of the forced-path sweep on the GLM-4.7-Flash-like workload.
SWEEP_L = (1, 2, 8, 64, 379, 398, 512, 2048)


@dataclass
class Inputs:
    w: Workload
    L: int
    offsets: np.ndarray                     # int64 [B+1]
    q_nope: np.ndarray                      # [B, L, H, n]
    q_pe: np.ndarray                        # [B, L, H, rope]
    c_kv: np.ndarray                        # [sumKv, r]
    k_pe: np.ndarray                        # [sumKv, rope]
    w_uk: np.ndarray                        # [H, n, r]
    w_uv: np.ndarray                        # [H, r, v]
    extra: dict = field(default_factory=dict)

    @property
    def kv_lens(self) -> np.ndarray:
        return np.diff(self.offsets)

    @property
    def scale(self) -> float:
        return self.w.scale


def _draw(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if dtype == "bf16":
        x = round_bf16(x)
    return x


def make_inputs(w: Workload, L: int | None = None, kv: int | None = None, batch: int | None = None,
                seed: int | None = None) -> Inputs:
    """Draw one seeded input set for workload ``w`` (optionally overriding L, Kv, batch, seed)."""
    L = w.L if L is None else int(L)
    B = w.batch if batch is None else int(batch)
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    if kv is not None:
        lens = np.full(B, int(kv), dtype=np.int64)
    elif w.kv is not None:
        lens = np.full(B, int(w.kv), dtype=np.int64)
    else:
        lo, hi = w.kv_range
        lens = rng.integers(lo, hi, size=B, endpoint=True).astype(np.int64)
    lens = np.maximum(lens, L)
    offsets = np.zeros(B + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(lens)
    T = int(offsets[-1])
    H = w.heads
    q_nope = _draw(rng, (B, L, H, w.n), 1.0, w.dtype)
    q_pe = _draw(rng, (B, L, H, w.rope), 1.0, w.dtype)
    c_kv = _draw(rng, (T, w.r), 1.0, w.dtype)
    k_pe = _draw(rng, (T, w.rope), 1.0, w.dtype)
    w_uk = _draw(rng, (H, w.n, w.r), 1.0 / math.sqrt(w.r), w.dtype)
    w_uv = _draw(rng, (H, w.r, w.v), 1.0 / math.sqrt(w.r), w.dtype)
    return Inputs(w, L, offsets, q_nope, q_pe, c_kv, k_pe, w_uk, w_uv)


def draw_like(shape, std: float, dtype: str, seed: int) -> np.ndarray:
    """A stand-alone seeded N(0, std^2) tensor in the storage type (e.g. a
    synthetic folded query q_lat, or synthetic per-head K / V)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return _draw(rng, shape, std, dtype)


# Pooled-indexer workload: one sequence of 131072 cached positions (the longest
# context the pages measure the indexer at), a verify step of 8 new positions,
# keys = the bf16 latent rows (width 512), top-2048 budget.
INDEXER_WORKLOAD = dict(name="indexer_kv131072_s8_d512_top2048", kv=131072, S=8, d=512, budget=2048, seed=6)


@dataclass
class IndexerInputs:
    offsets: np.ndarray                     # int64 [B+1], cache lengths after the step
    keys: np.ndarray                        # [sumKv, d] bf16-exact float32 ~ N(0, 1)
    q: np.ndarray                           # [B, d] float32 ~ N(0, 1/d): the indexer query of the step


def indexer_inputs(lengths, d: int, seed: int) -> IndexerInputs:
    """Seeded keys and queries for the pooled indexer (draw order: keys, q)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = np.asarray(lengths, dtype=np.int64)
    offsets = np.zeros(lens.size + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(lens)
    keys = _draw(rng, (int(offsets[-1]), d), 1.0, "bf16")
    q = _draw(rng, (lens.size, d), 1.0 / math.sqrt(d), "f32")
    return IndexerInputs(offsets, keys, q)


def custom(r: int, n: int, v: int, rope: int, heads: int, batch: int, L: int, kv: int | None = None,
           kv_range: tuple[int, int] | None = None, dtype: str = "bf16", seed: int = 0,
           name: str = "custom") -> Workload:
    return Workload(name, r, n, v, rope, heads, batch, L, kv=kv, kv_range=kv_range, dtype=dtype, seed=seed)

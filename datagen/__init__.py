"""Seeded synthetic inputs for C = relu(A·B).

This module draws the input matrices and nothing else: it holds none of the
method's arithmetic (no products, sums or activation). Both sides of every
parity check (the fp64 oracle and the gfx950 library) consume exactly the
arrays produced here, so a result difference can only come from the two
implementations of relu(A·B) themselves.

Generator: SplitMix64 in its counter form. Output i of stream ``seed`` is
``mix64(seed + (i + 1) * 0x9E3779B97F4A7C15)`` with the published SplitMix64
finaliser (Steele, Lea, Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014). Being counter based, any element can be drawn
without the ones before it, and the stream does not depend on numpy's or
torch's RNG implementations.

Distributions (workload shapes from the lecture pages' matmul section and
the five configurations below):
  * U(-1,1): 2u - 1 with u = top 53 bits / 2^53, rounded once to fp32.
  * N(0,1)/sqrt(K): Box-Muller cosine branch on the pair (u_2i, u_2i+1),
    times 1/sqrt(K), all in fp64, rounded once to fp32.
  * bf16 inputs: the fp32 value rounded to bf16 (round to nearest, ties to
    even), kept as uint16 bit patterns.
  * small integers in [lo, hi]: floor(u * (hi - lo + 1)) + lo, exact in fp32
    and bf16, used where every summation order must give the same result.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

GOLDEN_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 16


def _mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 finaliser, in place on a uint64 array (wrapping arithmetic)."""
    t = z >> np.uint64(30)
    z ^= t
    z *= _M1
    np.right_shift(z, np.uint64(27), out=t)
    z ^= t
    z *= _M2
    np.right_shift(z, np.uint64(31), out=t)
    z ^= t
    return z


def splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Outputs start .. start+count-1 of the SplitMix64 stream ``seed``."""
    z = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    z *= GOLDEN_GAMMA
    z += np.uint64(seed & 0xFFFFFFFFFFFFFFFF)
    return _mix64(z)


def uniform01(seed: int, start: int, count: int) -> np.ndarray:
    """Doubles in [0, 1) from the top 53 bits of each SplitMix64 output."""
    z = splitmix64(seed, start, count)
    z >>= np.uint64(11)
    u = z.view(np.int64).astype(np.float64)
    u *= 2.0 ** -53
    return u


def _fill(n: int, fn) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        out[s:e] = fn(s, e - s)
    return out


def uniform_pm1_f32(seed: int, rows: int, cols: int) -> np.ndarray:
    """rows x cols fp32 matrix, entries i.i.d. U(-1, 1)."""
    return _fill(rows * cols, lambda s, n: 2.0 * uniform01(seed, s, n) - 1.0).reshape(rows, cols)


def normal_f32(seed: int, rows: int, cols: int, scale: float = 1.0) -> np.ndarray:
    """rows x cols fp32 matrix, entries i.i.d. N(0,1) * scale (scale applied in fp64)."""
    def chunk(s, n):
        u = uniform01(seed, 2 * s, 2 * n)
        u1, u2 = u[0::2], u[1::2]
        r = np.sqrt(-2.0 * np.log1p(-u1))  # 1 - u1 lies in (0, 1]
        return r * np.cos(2.0 * math.pi * u2) * scale
    return _fill(rows * cols, chunk).reshape(rows, cols)


def small_int_f32(seed: int, rows: int, cols: int, lo: int = -4, hi: int = 4) -> np.ndarray:
    """rows x cols fp32 matrix of integers drawn uniformly from [lo, hi]."""
    span = hi - lo + 1
    return _fill(rows * cols, lambda s, n: np.floor(uniform01(seed, s, n) * span) + lo).reshape(rows, cols)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bit patterns.
    Inputs must be finite (the generators above only produce finite values)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    return ((b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def pad_rows(x: np.ndarray, ld: int, fill=0) -> np.ndarray:
    """Copy a rows x cols matrix into a rows x ld buffer (leading dimension ld >= cols)."""
    rows, cols = x.shape
    if ld < cols:
        raise ValueError("leading dimension smaller than the row length")
    if ld == cols:
        return np.ascontiguousarray(x)
    out = np.full((rows, ld), fill, dtype=x.dtype)
    out[:, :cols] = x
    return out


@dataclasses.dataclass(frozen=True)
class Config:
    """One workload of relu(A·B): shapes, leading dimensions (elements), dtype, distribution."""
    ident: int
    name: str
    dtype: str          # "f32" or "bf16"
    M: int
    N: int
    K: int
    lda: int
    ldb: int
    ldc: int
    dist: str           # "normal_over_sqrtk", "uniform_pm1", "small_int" or "zeros"

    @property
    def seed_a(self) -> int:
        return 1000 + self.ident

    @property
    def seed_b(self) -> int:
        return 2000 + self.ident

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


# The five workloads: three square fp32 sizes along the pages' square-matmul
# scaling sweep (256 .. 8192), one ragged fp32 shape that no tile size divides,
# and the large bf16 shape.
CONFIGS = {
    1: Config(1, "f32_256", "f32", 256, 256, 256, 256, 256, 256, "normal_over_sqrtk"),
    2: Config(2, "f32_1024", "f32", 1024, 1024, 1024, 1024, 1024, 1024, "normal_over_sqrtk"),
    3: Config(3, "f32_4096", "f32", 4096, 4096, 4096, 4096, 4096, 4096, "uniform_pm1"),
    4: Config(4, "f32_4097x3001x2049", "f32", 4097, 3001, 2049, 2049, 3001, 3001, "normal_over_sqrtk"),
    5: Config(5, "bf16_8192", "bf16", 8192, 8192, 8192, 8192, 8192, 8192, "normal_over_sqrtk"),
}


def draw(dist: str, seed: int, rows: int, cols: int, K: int) -> np.ndarray:
    if dist == "normal_over_sqrtk":
        return normal_f32(seed, rows, cols, 1.0 / math.sqrt(K))
    if dist == "uniform_pm1":
        return uniform_pm1_f32(seed, rows, cols)
    if dist == "small_int":
        return small_int_f32(seed, rows, cols)
    if dist == "zeros":
        return np.zeros((rows, cols), dtype=np.float32)
    raise ValueError(f"unknown distribution {dist!r}")


def make_inputs(cfg: Config):
    """Host arrays (A, B) for a config, laid out with its leading dimensions.
    fp32 configs give float32 arrays; bf16 configs give uint16 bf16 bit patterns."""
    a = draw(cfg.dist, cfg.seed_a, cfg.M, cfg.K, cfg.K)
    b = draw(cfg.dist, cfg.seed_b, cfg.K, cfg.N, cfg.K)
    if cfg.dtype == "bf16":
        a, b = f32_to_bf16_bits(a), f32_to_bf16_bits(b)
    return pad_rows(a, cfg.lda), pad_rows(b, cfg.ldb)

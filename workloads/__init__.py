"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only *makes inputs*: random matrices with the value distribution of
momentum matrices (N(0, std) drawn in fp32, rounded to bf16 with
round-to-nearest-even when the storage type is bf16), the shape lists of the
matrix sets that are measured, and row splits of those matrices over S shard
buffers. It holds none of the method's arithmetic (no cost, no assignment, no
offsets, no Newton-Schulz), so the oracle and the HIP path can both be fed
from it without sharing any of their own code.

Every matrix is reproducible on its own from ``(seed, index)``, so a test can
regenerate one matrix of a large set for the oracle without rebuilding the set.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# Coefficients of the quintic and cubic iterations used by the measured sets.
QUINTIC = (3.4445, -4.7750, 2.0315)
CUBIC = (1.5, -0.5, 0.0)
DEFAULT_EPS = 1e-7


# ----------------------------------------------------------------------------
# bf16 storage (bit patterns held in uint16 arrays)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 with round-to-nearest-even; return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    rounded = np.where(nan, (u >> 16) | 0x40, rounded)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 values (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
# matrices
# ----------------------------------------------------------------------------

def host_matrix(seed: int, index: int, shape, std: float = 0.02, dtype: str = "bf16") -> np.ndarray:
    """One seeded matrix on the host.

    Values are N(0, std) drawn in fp32 from ``numpy.random.default_rng([seed, index])``.
    Returns uint16 bf16 bits for ``dtype == "bf16"``, float32 values for ``"f32"``.
    """
    rng = np.random.default_rng([int(seed), int(index)])
    x = rng.standard_normal(tuple(shape), dtype=np.float32)
    if std != 1.0:
        x = x * np.float32(std)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f32":
        return x
    raise ValueError(f"unknown dtype {dtype!r}")


def device_matrix(seed: int, index: int, shape, std: float = 0.02, dtype: str = "bf16",
                  device: str = "cuda"):
    """One seeded matrix made by torch's generator on ``device`` (for large sets).

    Used where host generation of a multi-GiB set would dominate a run. The
    values differ from :func:`host_matrix` for the same seed; a test that checks
    such a matrix copies it back to the host for the oracle.
    """
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) * 1_000_003 + int(index))
    x = torch.randn(tuple(shape), generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    if dtype == "f32":
        return x
    raise ValueError(f"unknown dtype {dtype!r}")


# ----------------------------------------------------------------------------
# row splits over S shard buffers
# ----------------------------------------------------------------------------

def orthogonal_rows_bits(m: int, n: int, seed: int) -> np.ndarray:
    """bf16 bits (uint16, m x n) of a +-1 matrix whose rows are orthogonal with
    equal norms sqrt(n): the m x m Sylvester-Hadamard matrix tiled n / m times
    along the columns, each column then multiplied by a seeded random sign.
    m must be a power of two and n a multiple of m."""
    if m & (m - 1) or n % m:
        raise ValueError("m must be a power of two and n a multiple of m")
    h = np.ones((1, 1), dtype=np.int8)
    while h.shape[0] < m:
        h = np.block([[h, h], [h, -h]])
    signs = np.where(np.random.default_rng(seed).integers(0, 2, size=n) > 0, 1, -1).astype(np.int8)
    neg = (np.tile(h, (1, n // m)) * signs[None, :]) < 0
    return np.where(neg, np.uint16(0xBF80), np.uint16(0x3F80))   # -1.0 / +1.0 in bf16


def even_split_rows(rows: int, num_shards: int) -> list[int]:
    """Split ``rows`` over shards the ``torch.tensor_split`` way: the first
    ``rows % S`` shards get one extra row."""
    q, r = divmod(rows, num_shards)
    return [q + (1 if s < r else 0) for s in range(num_shards)]


def row_cut_split_rows(row_counts: list[int], cuts: list[int]) -> list[list[int]]:
    """Split a set of matrices whose rows are laid end to end in one buffer.

    ``cuts`` are the S+1 row boundaries ``[0, c1, ..., total]`` of the shards;
    shard s holds global rows ``[cuts[s], cuts[s+1])``. Returns split_rows[i][s]
    = how many rows of matrix i fall in shard s. This mirrors a flat buffer that
    is cut into contiguous per-rank ranges at row granularity.
    """
    S = len(cuts) - 1
    out = []
    start = 0
    for rows in row_counts:
        end = start + rows
        out.append([max(0, min(end, cuts[s + 1]) - max(start, cuts[s])) for s in range(S)])
        start = end
    return out


# ----------------------------------------------------------------------------
# the measured sets
# ----------------------------------------------------------------------------

@dataclass
class MatrixSet:
    name: str
    shapes: list
    dtype: str = "bf16"
    std: float = 0.02
    seed: int = 0
    steps: int = 5
    coeffs: tuple = QUINTIC
    description: str = ""
    split_rows: list | None = None      # [n][S] or None
    num_shards: int = 1
    homes_hint: list | None = field(default=None)

    @property
    def n(self) -> int:
        return len(self.shapes)


def single_fp32() -> MatrixSet:
    """One fp32 64x128 matrix, entries N(0, 1), seed 0."""
    return MatrixSet("fp32-64x128", [(64, 128)], dtype="f32", std=1.0, seed=0,
                     description="one fp32 64x128 matrix, N(0,1)")


def square_batch() -> MatrixSet:
    """16 bf16 1024x1024 matrices, N(0, 0.02), seed 1: one shape bucket."""
    return MatrixSet("16x1024x1024-bf16", [(1024, 1024)] * 16, seed=1,
                     description="16 bf16 1024x1024 matrices, N(0,0.02)")


def dense_transformer(layers: int = 32, hidden: int = 4096, ffn: int = 14336,
                      kv: int = 1024) -> MatrixSet:
    """Per layer: q, k, v, o, gate, up, down in layer-major order (224 matrices at 32 layers)."""
    per_layer = [(hidden, hidden), (kv, hidden), (kv, hidden), (hidden, hidden),
                 (ffn, hidden), (ffn, hidden), (hidden, ffn)]
    return MatrixSet(f"dense-transformer-{layers}L-h{hidden}-f{ffn}", per_layer * layers, seed=3,
                     description=f"{layers} layers x [q,k,v,o,gate,up,down], hidden {hidden}, ffn {ffn}")


def routed_square_batch(uneven: bool = True) -> MatrixSet:
    """The 16 x 1024^2 set stored as S = 4 row shards.

    even: every matrix is cut into four 256-row shards.
    uneven: the 16 x 1024 rows are laid end to end and cut at rows
    [0, 6000, 11500, 16384, 16384]; matrix 5 and 11 straddle two shards, the
    others sit whole in one shard, and the fourth shard holds nothing.
    """
    base = square_batch()
    if uneven:
        splits = row_cut_split_rows([s[0] for s in base.shapes], [0, 6000, 11500, 16384, 16384])
        name = "16x1024x1024-bf16-S4-uneven"
    else:
        splits = [even_split_rows(s[0], 4) for s in base.shapes]
        name = "16x1024x1024-bf16-S4-even"
    return MatrixSet(name, base.shapes, seed=base.seed, split_rows=splits, num_shards=4,
                     description=base.description + (" in 4 uneven row shards" if uneven
                                                     else " in 4 even row shards"))


def many_small(num_random: int = 3000, experts: int = 64, seed_shapes: int = 5,
               seed_values: int = 6) -> MatrixSet:
    """3000 matrices with rows, cols each round(exp(U(ln 64, ln 4096))), plus
    MoE experts x {2048x7168, 7168x2048, 2048x7168}."""
    rng = np.random.default_rng(seed_shapes)
    lo, hi = math.log(64), math.log(4096)
    dims = np.rint(np.exp(rng.uniform(lo, hi, size=(num_random, 2)))).astype(np.int64)
    shapes = [(int(r), int(c)) for r, c in dims]
    shapes += [(2048, 7168), (7168, 2048), (2048, 7168)] * experts
    return MatrixSet(f"many-small-{num_random}+moe{experts}", shapes, seed=seed_values,
                     description=f"{num_random} log-uniform [64,4096]^2 + {experts} experts x 3")


SETS = {
    "fp32-64x128": single_fp32,
    "square": square_batch,
    "routed-uneven": lambda: routed_square_batch(True),
    "routed-even": lambda: routed_square_batch(False),
    "dense-transformer": dense_transformer,
    "many-small": many_small,
}

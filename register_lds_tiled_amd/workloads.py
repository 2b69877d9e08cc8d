"""Seeded synthetic inputs for the row-major SGEMM workloads.

This module is shared by the tests, the benchmark and the CPU oracle's
callers.  It only draws and lays out input matrices; it holds none of the
product's arithmetic.

Workloads (all fp32, row-major, tight leading dimensions):

* ``micro``   4x4x1024 -- the first page's worked example ("Micro Kernel
  입문하기", teach-meaning.tistory.com/1544, section 2 and walkthrough section
  6): A (4xK) holds (i % 7) * 0.1f and B (Kx4) holds (i % 5) * 0.2f over the
  flat row-major index i, each product taken in fp32 as the page's host code
  does.
* ``sq1024``  1024^3, A and B i.i.d. Uniform(-1, 1)  (the tiled page's first
  measured shape, "gemm_tiled_test", teach-meaning.tistory.com/1542, section 7;
  the pages do not state a distribution; Uniform(-1, 1) is the reading taken).
* ``sq2048``  2048^3, Uniform(-1, 1)  (the tiled page's second shape).
* ``ragged``  M=1000, N=1500, K=777, Uniform(-1, 1): no dimension is a
  multiple of any tile, and A's rows (777 floats) are only 4-byte aligned.
* ``sq8192``  8192^3, A and B i.i.d. Normal(0, 1): the large compute-bound
  case.

Random draws use numpy's PCG64 with a per-workload seed, A first, then B,
from one generator; Uniform(-1, 1) is drawn in float64 and rounded to float32,
Normal(0, 1) is drawn directly in float32.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    dist: str          # "worked", "uniform" or "normal"
    seed: int | None

    @property
    def flops(self) -> float:
        """2*M*N*K: one multiply and one add per term of every output sum."""
        return 2.0 * self.M * self.N * self.K

    def describe(self) -> str:
        d = {"worked": "worked-example init", "uniform": "U(-1,1)", "normal": "N(0,1)"}[self.dist]
        return f"sgemm {self.M}x{self.N}x{self.K} fp32 row-major {d}" + (
            f" seed {self.seed}" if self.seed is not None else "")


WORKLOADS = {
    "micro": Workload("micro", 4, 4, 1024, "worked", None),
    "sq1024": Workload("sq1024", 1024, 1024, 1024, "uniform", 1002),
    "sq2048": Workload("sq2048", 2048, 2048, 2048, "uniform", 1003),
    "ragged": Workload("ragged", 1000, 1500, 777, "uniform", 1004),
    "sq8192": Workload("sq8192", 8192, 8192, 8192, "normal", 1005),
}

# Skinny shapes, bound by HBM (one operand streamed once): a row vector
# times a matrix, a matrix times a column vector, 8 and 16 rows of A, 4
# columns of B.
SKINNY = {
    "row1": Workload("row1", 1, 8192, 8192, "uniform", 1006),
    "col1": Workload("col1", 8192, 1, 8192, "uniform", 1007),
    "rows8": Workload("rows8", 8, 65536, 8192, "uniform", 1008),
    "cols4": Workload("cols4", 65536, 4, 8192, "uniform", 1009),
    "rows16": Workload("rows16", 16, 65536, 8192, "uniform", 1010),
}


def workload(name: str) -> Workload:
    """A named workload of either table."""
    return WORKLOADS[name] if name in WORKLOADS else SKINNY[name]


def worked_example(K: int = 1024):
    """A (4xK) = (i % 7) * 0.1f and B (Kx4) = (i % 5) * 0.2f, fp32 products."""
    ia = np.arange(4 * K, dtype=np.int64)
    ib = np.arange(K * 4, dtype=np.int64)
    A = ((ia % 7).astype(np.float32) * np.float32(0.1)).reshape(4, K)
    B = ((ib % 5).astype(np.float32) * np.float32(0.2)).reshape(K, 4)
    return A, B


def random_inputs(M: int, N: int, K: int, seed: int, dist: str = "uniform"):
    """Draw A (MxK) then B (KxN) from one PCG64 generator."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if dist == "uniform":
        A = rng.uniform(-1.0, 1.0, (M, K)).astype(np.float32)
        B = rng.uniform(-1.0, 1.0, (K, N)).astype(np.float32)
    elif dist == "normal":
        A = rng.standard_normal((M, K), dtype=np.float32)
        B = rng.standard_normal((K, N), dtype=np.float32)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return A, B


def integer_inputs(M: int, N: int, K: int, seed: int, lo: int = -3, hi: int = 3):
    """Integer-valued fp32 inputs drawn uniformly from {lo..hi}.  With
    |values| <= 3 every partial sum is an integer below 2^24 in magnitude for
    K <= 1.8M, so every summation order gives the same exact result."""
    rng = np.random.Generator(np.random.PCG64(seed))
    A = rng.integers(lo, hi + 1, (M, K)).astype(np.float32)
    B = rng.integers(lo, hi + 1, (K, N)).astype(np.float32)
    return A, B


def epilogue_inputs(M: int, N: int, seed: int, scale: float = 1.0, integer: bool = False):
    """Operands of the fused epilogue: the C read when beta != 0 (MxN) and a
    per-column bias (N), from one PCG64 generator, C first.  Uniform(-scale,
    scale) rounded to float32, or, with integer=True, integers in
    [-scale, scale] (exact in every fp32 operation of a small epilogue)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if integer:
        s = int(scale)
        C = rng.integers(-s, s + 1, (M, N)).astype(np.float32)
        bias = rng.integers(-s, s + 1, N).astype(np.float32)
    else:
        C = rng.uniform(-scale, scale, (M, N)).astype(np.float32)
        bias = rng.uniform(-scale, scale, N).astype(np.float32)
    return C, bias


def to_bf16_storage(X: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 storage (uint16), rounding to nearest even: the
    input encoding of the 16-bit workloads (finite inputs only)."""
    u = np.ascontiguousarray(X, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def to_f16_storage(X: np.ndarray) -> np.ndarray:
    """float32 -> IEEE binary16 storage (uint16), numpy's round to nearest."""
    return np.ascontiguousarray(X, dtype=np.float32).astype(np.float16).view(np.uint16)


def lowp_inputs(M: int, N: int, K: int, seed: int, fmt: str, dist: str = "uniform",
                integer: bool = False):
    """A (MxK) and B (KxN) as 16-bit storage (uint16) in format fmt ("bf16"
    or "f16"): the float32 draws of random_inputs (or integer_inputs, which
    both formats hold exactly), encoded."""
    A, B = integer_inputs(M, N, K, seed) if integer else random_inputs(M, N, K, seed, dist)
    enc = {"bf16": to_bf16_storage, "f16": to_f16_storage}[fmt]
    return enc(A), enc(B)


def tile_samples(M: int, N: int, seed: int, band: int = 128, tile: int = 64):
    """Indices of outputs that reach every tile of an M x N result (for
    sampled checks of products too large to compare whole): one row in each
    `band`-row band and one column in each `band`-column band, each at an
    offset inside its band drawn afresh per band, and one entry in each
    `tile` x `tile` tile, ragged last bands and tiles included.  Returns
    (rows, cols, er, ec) as int64 arrays."""
    rng = np.random.Generator(np.random.PCG64(seed))

    def one_per(n, size):
        starts = np.arange(0, n, size)
        return starts + rng.integers(0, np.minimum(size, n - starts))

    rows, cols = one_per(M, band), one_per(N, band)
    nr, nc = -(-M // tile), -(-N // tile)
    er = np.repeat(np.arange(0, M, tile), nc)
    ec = np.tile(np.arange(0, N, tile), nr)
    er = er + rng.integers(0, np.minimum(tile, M - er))
    ec = ec + rng.integers(0, np.minimum(tile, N - ec))
    return rows, cols, er, ec


def inputs_for(w: Workload):
    if w.dist == "worked":
        return worked_example(w.K)
    return random_inputs(w.M, w.N, w.K, w.seed, w.dist)

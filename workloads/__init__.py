"""Seeded synthetic inputs for the FP32 GEMM workloads.

This module only draws numbers and lays them out in storage order; it holds
none of the product's arithmetic, and it is the one piece shared by the tests,
the benchmark, the oracle's callers and the HIP path's callers.

Workloads (shapes and value distributions of the linear-layer and square
matrix products the pages discuss: "GEMM 性能优化", opening paragraph — FFN,
QKV projections and linear layers are GEMMs; "PMPP Chapter 06", section 1 —
A and C row-major, B row-major or column-major for corner turning):

========  =====================  ======  =======================  ====
name      M x N x K              B       values                   seed
========  =====================  ======  =======================  ====
sq256     256 x 256 x 256        row     uniform[-1, 1]           0
sq4096    4096 x 4096 x 4096     row     uniform[-1, 1]           1
sq4096t   4096 x 4096 x 4096     col     normal(0, 1)             2
ragged    5003 x 4097 x 2049     row     uniform[-1, 1]           3
ffn       8192 x 14336 x 4096    row     normal(0, 0.02)          4
skinny    16 x 4096 x 4096       row     normal(0, 0.02)          4
longk     1024 x 1024 x 8192     row     uniform[-1, 1]           5
========  =====================  ======  =======================  ====

Recipe: ``numpy.random.default_rng(seed)`` (PCG64); A is drawn first, then B,
each in storage order (a column-major B is drawn as its N x K storage buffer),
in float64 and cast to float32.  ``normal(0, 0.02)`` means standard deviation
0.02.  The integer-valued variant of every workload draws integers uniformly
from {-8, ..., 8} with ``seed + 1000``; every partial sum then stays below
2**24 in magnitude, so any summation order is exact in float32.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

ROW_MAJOR = 0
COL_MAJOR = 1


@dataclass(frozen=True)
class Workload:
    name: str
    m: int
    n: int
    k: int
    layout_b: int
    dist: str          # "uniform", "normal1", "normal002"
    seed: int
    note: str = ""


WORKLOADS = {
    w.name: w
    for w in (
        Workload("sq256", 256, 256, 256, ROW_MAJOR, "uniform", 0, "small square case"),
        Workload("sq4096", 4096, 4096, 4096, ROW_MAJOR, "uniform", 1, "large square, compute-bound"),
        Workload("sq4096t", 4096, 4096, 4096, COL_MAJOR, "normal1", 2, "B column-major (corner turning)"),
        Workload("ragged", 5003, 4097, 2049, ROW_MAJOR, "uniform", 3, "boundary tiles, odd strides"),
        Workload("ffn", 8192, 14336, 4096, ROW_MAJOR, "normal002", 4, "FFN linear layer"),
        Workload("skinny", 16, 4096, 4096, ROW_MAJOR, "normal002", 4, "memory-bound, few rows"),
        Workload("longk", 1024, 1024, 8192, ROW_MAJOR, "uniform", 5, "few tiles, long k (stream-K)"),
        Workload("gemv_t", 1, 4096, 4096, COL_MAJOR, "normal002", 6, "one row, B column-major (y = W x)"),
        Workload("decode4_t", 4, 14336, 4096, COL_MAJOR, "normal002", 7, "four rows, B column-major, FFN-sized"),
        Workload("fewcol8", 8192, 8, 8192, ROW_MAJOR, "normal002", 8, "few columns: A streamed once"),
    )
}


def _draw(rng: np.random.Generator, dist: str, size: int) -> np.ndarray:
    if dist == "uniform":
        x = rng.uniform(-1.0, 1.0, size)
    elif dist == "normal1":
        x = rng.normal(0.0, 1.0, size)
    elif dist == "normal002":
        x = rng.normal(0.0, 0.02, size)
    elif dist == "int8range":
        x = rng.integers(-8, 9, size).astype(np.float64)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return x.astype(np.float32)


def b_storage_shape(k: int, n: int, layout_b: int, ldb: int | None = None):
    """(rows, row stride) of B's storage buffer."""
    if layout_b == ROW_MAJOR:
        return k, (n if ldb is None else ldb)
    return n, (k if ldb is None else ldb)


def a_storage_shape(m: int, k: int, layout_a: int, lda: int | None = None):
    """(rows, row stride) of A's storage buffer."""
    if layout_a == ROW_MAJOR:
        return m, (k if lda is None else lda)
    return k, (m if lda is None else lda)


def random_operands(m: int, n: int, k: int, layout_b: int, dist: str, seed: int,
                    lda: int | None = None, ldb: int | None = None, pad_value: float = np.nan,
                    layout_a: int = ROW_MAJOR):
    """Draw A (M x K) and B (K x N), each in the given layout, as storage arrays.

    The logical entries are drawn in storage order with packed strides (a
    column-major A as its K x M storage buffer); when a leading dimension
    larger than the minimum is asked for, the packed values are placed into a
    wider buffer whose padding holds ``pad_value`` (NaN by default, so that
    any use of padding shows up in the result)."""
    rng = np.random.default_rng(seed)
    a_rows, a_cols = a_storage_shape(m, k, layout_a)
    a = _draw(rng, dist, a_rows * a_cols).reshape(a_rows, a_cols)
    b_rows, b_cols = b_storage_shape(k, n, layout_b)
    b = _draw(rng, dist, b_rows * b_cols).reshape(b_rows, b_cols)
    return _pad(a, lda, pad_value), _pad(b, ldb, pad_value)


def _pad(x: np.ndarray, ld: int | None, pad_value: float) -> np.ndarray:
    if ld is None or ld == x.shape[1]:
        return np.ascontiguousarray(x)
    if ld < x.shape[1]:
        raise ValueError("leading dimension smaller than the row length")
    out = np.full((x.shape[0], ld), pad_value, dtype=np.float32)
    out[:, : x.shape[1]] = x
    return out


def epilogue_operands(m: int, n: int, seed: int):
    """C_in (M x N, row-major) and bias (N) for the linear-layer epilogue,
    normal(0, 1), drawn C_in first then bias."""
    rng = np.random.default_rng(seed)
    c_in = _draw(rng, "normal1", m * n).reshape(m, n)
    bias = _draw(rng, "normal1", n)
    return np.ascontiguousarray(c_in), bias


def workload_operands(w: Workload | str, integer: bool = False):
    """Operands of a named workload (packed strides).  ``integer=True`` gives the
    integer-valued variant (values in {-8..8}, seed + 1000)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    if integer:
        return random_operands(w.m, w.n, w.k, w.layout_b, "int8range", w.seed + 1000)
    return random_operands(w.m, w.n, w.k, w.layout_b, w.dist, w.seed)


def mod_pattern_operands(m: int, n: int, k: int, layout_b: int):
    """Structured integer operands with a closed-form product.

    A[i][k]  = ((i mod 7) - 3) * ((k mod 3) - 1)
    B(k, j)  = ((k mod 3) - 1) * ((j mod 5) - 2)
    The k-dependence makes any misalignment between the A and B k-indices
    visible.  Returned in storage order for the given B layout."""
    i = np.arange(m)[:, None]
    kk_a = np.arange(k)[None, :]
    a = (((i % 7) - 3) * ((kk_a % 3) - 1)).astype(np.float32)
    kk = np.arange(k)[:, None]
    j = np.arange(n)[None, :]
    b_logical = (((kk % 3) - 1) * ((j % 5) - 2)).astype(np.float32)  # K x N
    b = b_logical if layout_b == ROW_MAJOR else np.ascontiguousarray(b_logical.T)
    return np.ascontiguousarray(a), np.ascontiguousarray(b)


def int_storage(rows: int, cols: int, seed: int) -> np.ndarray:
    """A (rows x cols) float32 storage buffer of integers uniform in [-8, 8],
    drawn as int8 so that operands of a few GiB stay cheap to make."""
    rng = np.random.default_rng(seed)
    return rng.integers(-8, 9, (rows, cols), dtype=np.int8).astype(np.float32)


def permutation(n: int, seed: int) -> np.ndarray:
    """A seeded permutation of range(n)."""
    return np.random.default_rng(seed).permutation(n)


def sample_indices(m: int, n: int, count: int, seed: int):
    """Seeded element sample that always includes the four corners and the
    last row/column (boundary tiles), plus ``count`` uniform draws."""
    rng = np.random.default_rng(seed)
    rows = list(rng.integers(0, m, count))
    cols = list(rng.integers(0, n, count))
    edge_r = [0, 0, m - 1, m - 1] + [m - 1] * 16 + list(rng.integers(0, m, 16))
    edge_c = [0, n - 1, 0, n - 1] + list(rng.integers(0, n, 16)) + [n - 1] * 16
    return (np.array(rows + edge_r, dtype=np.int64), np.array(cols + edge_c, dtype=np.int64))

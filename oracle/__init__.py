"""CPU oracle for C = A.B (float32 inputs, float64 sequential accumulation).

TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers allowed; the product library never
imports, links or runs anything here, and nothing here imports the product
package.  The arithmetic lives in ``gemm_oracle.c`` (plain C, built by gcc with
``-ffp-contract=off``); this module only marshals numpy arrays into it.

Definition followed (pages "GEMM 性能优化", section 指标与目标 and 台阶 1;
"PMPP Chapter 06: Performance considerations", section 1 and its
corner-turning example):

    C[i, j] = sum_{k < K} A[i, k] * B(k, j)
    S[i, j] = sum_{k < K} |A[i, k] * B(k, j)|

with ``A[i, k] = A_store[i*lda + k]`` (``layout_a == 0``, row-major) or
``A_store[k*lda + i]`` (``layout_a == 1``, column-major), and
``B(k, j) = B_store[k*ldb + j]`` (``layout_b == 0``, row-major) or
``B_store[j*ldb + k]`` (``layout_b == 1``, column-major).  Each element is
summed in double in k order 0..K-1.

``epilogue_f64`` adds the linear-layer epilogue on top of that product:
``act(alpha * C + beta * C_in + bias[j])`` with ``act`` the identity, ReLU
``max(x, 0)`` or GELU ``x * Phi(x) = x/2 * (1 + erf(x / sqrt(2)))`` (their
textbook definitions), evaluated in float64.

Pins: every function here is pinned by the CPU tests in ``tests/test_oracle.py``
(exact rational brute force, block-matrix identity along K, M/N-split and
layout/transpose identities, identity and permutation products, closed forms at
the full workload shapes).  No function is left "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gemm_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_gemm.so")

# -O3 lets gcc vectorise the inner j loop of the row-major routine; that runs
# different output elements side by side and leaves every element's own k-order
# sum untouched.  -ffp-contract=off forbids fused multiply-adds.
CFLAGS = ["-O3", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c11"]

_lib = None


def build(verbose: bool = False) -> str:
    """Compile gemm_oracle.c into liboracle_gemm.so (always recompiles)."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64, f32p, f64p, i64p = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    lib.oracle_gemm_f64_ex.argtypes = [i64, i64, i64, ctypes.c_int, ctypes.c_int, f32p, i64, f32p, i64,
                                       f64p, f64p, i64]
    lib.oracle_gemm_f64_ex.restype = ctypes.c_int
    lib.oracle_gemm_f64_sampled_ex.argtypes = [i64, i64, i64, ctypes.c_int, ctypes.c_int, f32p, i64, f32p, i64,
                                               i64, i64p, i64p, f64p, f64p]
    lib.oracle_gemm_f64_sampled_ex.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _check_operands(A, B, m, n, k, layout_b, lda, ldb, layout_a=0):
    if layout_a not in (0, 1):
        raise ValueError("layout_a must be 0 (row-major) or 1 (column-major)")
    if layout_b not in (0, 1):
        raise ValueError("layout_b must be 0 (row-major) or 1 (column-major)")
    for name, arr in (("A", A), ("B", B)):
        if not isinstance(arr, np.ndarray) or arr.dtype != np.float32 or not arr.flags.c_contiguous:
            raise TypeError(f"{name} must be a C-contiguous float32 numpy array")
    if min(m, n, k) < 0:
        raise ValueError("negative dimension")
    if lda < (k if layout_a == 0 else m) or ldb < (n if layout_b == 0 else k):
        raise ValueError("leading dimension too small")
    if layout_a == 0:
        need_a = (m - 1) * lda + k if m > 0 and k > 0 else 0
    else:
        need_a = (k - 1) * lda + m if m > 0 and k > 0 else 0
    if layout_b == 0:
        need_b = (k - 1) * ldb + n if k > 0 and n > 0 else 0
    else:
        need_b = (n - 1) * ldb + k if k > 0 and n > 0 else 0
    if A.size < need_a or B.size < need_b:
        raise ValueError("operand storage smaller than its extent")


def _default_ld(m, n, k, layout_a, layout_b, lda, ldb):
    lda = (k if layout_a == 0 else m) if lda is None else lda
    ldb = (n if layout_b == 0 else k) if ldb is None else ldb
    return lda, ldb


def gemm_f64(A: np.ndarray, B: np.ndarray, m: int, n: int, k: int, layout_b: int,
             lda: int | None = None, ldb: int | None = None, layout_a: int = 0):
    """Full product.  ``A``/``B`` are the float32 storage buffers (any shape,
    C-contiguous; they are read flat).  Returns ``(C, S)`` as (m, n) float64."""
    lda, ldb = _default_ld(m, n, k, layout_a, layout_b, lda, ldb)
    _check_operands(A, B, m, n, k, layout_b, lda, ldb, layout_a)
    C = np.empty((m, n), dtype=np.float64)
    S = np.empty((m, n), dtype=np.float64)
    if m == 0 or n == 0:
        return C, S
    rc = _load().oracle_gemm_f64_ex(m, n, k, layout_a, layout_b, A.ctypes.data, lda, B.ctypes.data, ldb,
                                    C.ctypes.data, S.ctypes.data, n)
    if rc != 0:
        raise ValueError(f"oracle_gemm_f64_ex rejected its arguments (code {rc})")
    return C, S


def gemm_f64_sampled(A: np.ndarray, B: np.ndarray, m: int, n: int, k: int, layout_b: int,
                     rows, cols, lda: int | None = None, ldb: int | None = None, layout_a: int = 0):
    """The same sums for the elements (rows[t], cols[t]).  Returns ``(c, s)``."""
    lda, ldb = _default_ld(m, n, k, layout_a, layout_b, lda, ldb)
    _check_operands(A, B, m, n, k, layout_b, lda, ldb, layout_a)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape or rows.ndim != 1:
        raise ValueError("rows and cols must be 1-D of equal length")
    c = np.empty(rows.size, dtype=np.float64)
    s = np.empty(rows.size, dtype=np.float64)
    rc = _load().oracle_gemm_f64_sampled_ex(m, n, k, layout_a, layout_b, A.ctypes.data, lda, B.ctypes.data,
                                            ldb, rows.size, rows.ctypes.data, cols.ctypes.data,
                                            c.ctypes.data, s.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_gemm_f64_sampled_ex rejected its arguments (code {rc})")
    return c, s


ACT_NONE, ACT_RELU, ACT_GELU = 0, 1, 2


def epilogue_f64(ab, s_ab, c_in=None, alpha: float = 1.0, beta: float = 0.0, bias=None, act: int = ACT_NONE):
    """Linear-layer epilogue on an oracle product ``ab`` (float64, (m, n) or
    sampled 1-D with ``bias`` already gathered per element):

        x = alpha * ab + beta * c_in + bias[j];   out = act(x)

    ``c_in`` is read only when beta != 0.  Returns ``(out, scale)`` with the
    error scale ``|alpha| * S + |beta * c_in| + |bias|`` (the magnitudes the
    float32 evaluation rounds), for ``within_tolerance``."""
    from scipy.special import erf

    ab = np.asarray(ab, dtype=np.float64)
    x = alpha * ab
    scale = abs(alpha) * np.asarray(s_ab, dtype=np.float64)
    if beta != 0.0:
        cin = np.asarray(c_in, dtype=np.float64)
        x = x + beta * cin
        scale = scale + np.abs(beta * cin)
    if bias is not None:
        b = np.asarray(bias, dtype=np.float64)
        x = x + b
        scale = scale + np.abs(b)
    if act == ACT_NONE:
        out = x
    elif act == ACT_RELU:
        out = np.maximum(x, 0.0)
    elif act == ACT_GELU:
        out = 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))
    else:
        raise ValueError("act must be 0 (none), 1 (ReLU) or 2 (GELU)")
    return out, scale


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_num_threads())


def set_num_threads(threads: int) -> int:
    """Thread count of later oracle calls; returns the previous one."""
    return int(_load().oracle_set_num_threads(threads))


def within_tolerance(c_test, c_ref, s_ref, rel: float = 1e-5, abs_: float = 1e-6):
    """Per-element acceptance |c - c_ref| <= rel*S + abs_, evaluated in float64.

    Returns ``(ok, max_ratio)`` where max_ratio is the largest
    |c - c_ref| / (rel*S + abs_) over the elements (<= 1 means within)."""
    c_test = np.asarray(c_test, dtype=np.float64)
    err = np.abs(c_test - c_ref)
    bound = rel * np.asarray(s_ref, dtype=np.float64) + abs_
    ratio = err / bound
    finite = np.isfinite(c_test).all()
    max_ratio = float(ratio.max()) if ratio.size else 0.0
    return bool(finite and max_ratio <= 1.0), max_ratio

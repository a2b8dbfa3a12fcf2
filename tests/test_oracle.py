"""Pins for the CPU oracle: checks against things other than the oracle itself.

Every check below compares the oracle with something the pages or plain
mathematics fix: exact rational arithmetic on tiny inputs, the block-matrix
identity along K ("GEMM 性能优化", 台阶 1), M/N splits, the row-/column-major
storage of the same B ("PMPP Chapter 06", section 1, corner turning), the
transpose identity, identity and permutation products, and closed-form
integer products at the full workload shapes.  ``test_pins_catch_planted_mistakes``
plants plausible mistakes in a wrapped oracle and requires each to trip a pin.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from workloads import (COL_MAJOR, ROW_MAJOR, WORKLOADS, mod_pattern_operands, permutation,
                       random_operands, sample_indices)

U64 = 2.0 ** -53  # unit roundoff of double


def gamma(n):
    """Higham's gamma_n = n u / (1 - n u): bound factor for n roundings."""
    return n * U64 / (1.0 - n * U64)


def exact_rational(A, B, m, n, k, layout_b, lda, ldb):
    """Exact C and S by rational arithmetic (tiny sizes only)."""
    a = A.reshape(-1)
    b = B.reshape(-1)
    C = [[Fraction(0)] * n for _ in range(m)]
    S = [[Fraction(0)] * n for _ in range(m)]
    for i in range(m):
        for j in range(n):
            acc = Fraction(0)
            acc_abs = Fraction(0)
            for kk in range(k):
                bv = b[kk * ldb + j] if layout_b == ROW_MAJOR else b[j * ldb + kk]
                p = Fraction(float(a[i * lda + kk])) * Fraction(float(bv))
                acc += p
                acc_abs += abs(p)
            C[i][j] = acc
            S[i][j] = acc_abs
    return C, S


# ----------------------------------------------------------------------------
# Pin checks.  Each takes the oracle's full-product function as ``gemm`` and
# returns True when the pin holds.
# ----------------------------------------------------------------------------

TINY_SHAPES = [(1, 1, 1), (2, 3, 5), (3, 2, 7), (5, 7, 3), (7, 5, 17), (17, 3, 2), (1, 17, 5)]


def pin_exact_rational(gemm, m, n, k, layout_b, padded, seed, integer=False):
    lda = k + 3 if padded else k
    ldb_min = n if layout_b == ROW_MAJOR else k
    ldb = ldb_min + 2 if padded else ldb_min
    dist = "int8range" if integer else "normal1"
    A, B = random_operands(m, n, k, layout_b, dist, seed, lda=lda, ldb=ldb)
    C, S = gemm(A, B, m, n, k, layout_b, lda, ldb)
    Ce, Se = exact_rational(A, B, m, n, k, layout_b, lda, ldb)
    for i in range(m):
        for j in range(n):
            if integer:
                if Fraction(C[i, j]) != Ce[i][j] or Fraction(S[i, j]) != Se[i][j]:
                    return False
            else:
                bound = gamma(k) * float(Se[i][j])
                if not abs(Fraction(C[i, j]) - Ce[i][j]) <= Fraction(bound):
                    return False
                if not abs(Fraction(S[i, j]) - Se[i][j]) <= Fraction(bound):
                    return False
    return True


def _slice_k(A, B, m, n, k, layout_b, k0, k1):
    """Operands restricted to k in [k0, k1), packed."""
    A2 = np.ascontiguousarray(A.reshape(m, -1)[:, k0:k1])
    if layout_b == ROW_MAJOR:
        B2 = np.ascontiguousarray(B.reshape(k, -1)[k0:k1, :n])
    else:
        B2 = np.ascontiguousarray(B.reshape(n, -1)[:, k0:k1])
    return A2, B2


def pin_k_split(gemm, m, n, k, layout_b, seed, integer=False):
    A, B = random_operands(m, n, k, layout_b, "int8range" if integer else "uniform", seed)
    C, S = gemm(A, B, m, n, k, layout_b, k, n if layout_b == ROW_MAJOR else k)
    for k1 in sorted({1, k // 2, k - 1}):
        if not 0 < k1 < k:
            continue
        A1, B1 = _slice_k(A, B, m, n, k, layout_b, 0, k1)
        A2, B2 = _slice_k(A, B, m, n, k, layout_b, k1, k)
        C1, S1 = gemm(A1, B1, m, n, k1, layout_b, k1, n if layout_b == ROW_MAJOR else k1)
        C2, S2 = gemm(A2, B2, m, n, k - k1, layout_b, k - k1, n if layout_b == ROW_MAJOR else k - k1)
        if integer:
            if not (np.array_equal(C, C1 + C2) and np.array_equal(S, S1 + S2)):
                return False
        else:
            tol = 2 * gamma(k) * S + 1e-300
            if not (np.all(np.abs(C - (C1 + C2)) <= tol) and np.all(np.abs(S - (S1 + S2)) <= tol)):
                return False
    return True


def pin_mn_split(gemm, m, n, k, layout_b, seed):
    A, B = random_operands(m, n, k, layout_b, "normal1", seed)
    ldb = n if layout_b == ROW_MAJOR else k
    C, S = gemm(A, B, m, n, k, layout_b, k, ldb)
    r0, r1 = m // 3, m - m // 4
    Cr, _ = gemm(np.ascontiguousarray(A.reshape(m, k)[r0:r1]), B, r1 - r0, n, k, layout_b, k, ldb)
    c0, c1 = n // 4, n - n // 3
    if layout_b == ROW_MAJOR:
        Bc = np.ascontiguousarray(B.reshape(k, n)[:, c0:c1])
        Cc, _ = gemm(A, Bc, m, c1 - c0, k, layout_b, k, c1 - c0)
    else:
        Bc = np.ascontiguousarray(B.reshape(n, k)[c0:c1, :])
        Cc, _ = gemm(A, Bc, m, c1 - c0, k, layout_b, k, k)
    return np.array_equal(Cr, C[r0:r1]) and np.array_equal(Cc, C[:, c0:c1])


def pin_layout_equivalence(gemm, m, n, k, seed):
    A, Brow = random_operands(m, n, k, ROW_MAJOR, "normal1", seed)
    Bcol = np.ascontiguousarray(Brow.reshape(k, n).T)   # same logical B, column-major storage
    C1, S1 = gemm(A, Brow, m, n, k, ROW_MAJOR, k, n)
    C2, S2 = gemm(A, Bcol, m, n, k, COL_MAJOR, k, k)
    return np.array_equal(C1, C2) and np.array_equal(S1, S2)


def pin_transpose(gemm, m, n, k, seed):
    """(A.B)^T = B^T.A^T, with the operands' roles swapped: B^T is the
    column-major B's storage read row-major, A^T is A's storage read
    column-major.  Products commute exactly, so the result is bitwise equal."""
    A, Bcol = random_operands(m, n, k, COL_MAJOR, "normal1", seed)
    C, _ = gemm(A, Bcol, m, n, k, COL_MAJOR, k, k)
    Ct, _ = gemm(Bcol, A, n, m, k, COL_MAJOR, k, k)
    return np.array_equal(C.T, Ct)


def pin_identity_permutation(gemm, m, n, k, layout_b, seed):
    A, B = random_operands(m, n, k, layout_b, "normal1", seed)
    ldb = n if layout_b == ROW_MAJOR else k
    Bl = (B.reshape(k, n) if layout_b == ROW_MAJOR else B.reshape(n, k).T).astype(np.float64)
    Al = A.reshape(m, k).astype(np.float64)

    def store_b(logical):  # K x N logical -> storage for layout_b
        x = np.asarray(logical, dtype=np.float32)
        return np.ascontiguousarray(x if layout_b == ROW_MAJOR else x.T)

    ok = True
    # A . I_k = A
    C, _ = gemm(A, store_b(np.eye(k)), m, k, k, layout_b, k, k)
    ok &= np.array_equal(C, Al)
    # I_k . B = B  (A operand = identity, K x K)
    C, _ = gemm(np.eye(k, dtype=np.float32), B, k, n, k, layout_b, k, ldb)
    ok &= np.array_equal(C, Bl)
    # A . P with P[kk][j] = 1 iff kk == p[j]  ->  (A.P)[i][j] = A[i][p[j]]
    p = permutation(k, seed + 7)
    P = np.zeros((k, k), dtype=np.float32)
    P[p, np.arange(k)] = 1.0
    C, _ = gemm(A, store_b(P), m, k, k, layout_b, k, k)
    ok &= np.array_equal(C, Al[:, p])
    # P . B with P[i][kk] = 1 iff kk == q[i]  ->  (P.B)[i][j] = B[q[i]][j]
    q = permutation(k, seed + 11)
    Q = np.zeros((k, k), dtype=np.float32)
    Q[np.arange(k), q] = 1.0
    C, _ = gemm(Q, B, k, n, k, layout_b, k, ldb)
    ok &= np.array_equal(C, Bl[q, :])
    return bool(ok)


def closed_form(rows, cols, k):
    """C and S of the mod-pattern operands, from the sum of ((k mod 3) - 1)^2
    over k < K, which counts the k with k mod 3 != 1: K - floor((K + 1) / 3)."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    count = k - (k + 1) // 3
    a = (rows % 7) - 3
    b = (cols % 5) - 2
    return (a * b * count).astype(np.float64), (np.abs(a) * np.abs(b) * count).astype(np.float64)


def pin_closed_form_full(gemm, m, n, k, layout_b):
    A, B = mod_pattern_operands(m, n, k, layout_b)
    C, S = gemm(A, B, m, n, k, layout_b, k, n if layout_b == ROW_MAJOR else k)
    Ce, Se = closed_form(np.arange(m)[:, None], np.arange(n)[None, :], k)
    return np.array_equal(C, Ce) and np.array_equal(S, Se)


def pin_all_ones(gemm, m, n, k, layout_b):
    A = np.ones((m, k), dtype=np.float32)
    B = np.ones((k, n) if layout_b == ROW_MAJOR else (n, k), dtype=np.float32)
    C, S = gemm(A, B, m, n, k, layout_b, k, n if layout_b == ROW_MAJOR else k)
    return bool(np.all(C == k) and np.all(S == k))


def pin_numpy_crosscheck(gemm, m, n, k, layout_b, seed):
    """An independent summation (numpy's float64 matmul) agrees within the
    rounding bound of two different orders."""
    A, B = random_operands(m, n, k, layout_b, "normal1", seed)
    C, S = gemm(A, B, m, n, k, layout_b, k, n if layout_b == ROW_MAJOR else k)
    Bl = (B.reshape(k, n) if layout_b == ROW_MAJOR else B.reshape(n, k).T).astype(np.float64)
    ref = A.reshape(m, k).astype(np.float64) @ Bl
    return bool(np.all(np.abs(C - ref) <= 2 * gamma(k) * S + 1e-300))


def gemm_real(A, B, m, n, k, layout_b, lda, ldb):
    return oracle.gemm_f64(A, B, m, n, k, layout_b, lda, ldb)


# ----------------------------------------------------------------------------
# The pins, applied to the real oracle
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("shape", TINY_SHAPES)
@pytest.mark.parametrize("layout_b", [ROW_MAJOR, COL_MAJOR])
@pytest.mark.parametrize("padded", [False, True])
def test_exact_rational_random(shape, layout_b, padded):
    m, n, k = shape
    assert pin_exact_rational(gemm_real, m, n, k, layout_b, padded, seed=100 + m * 7 + n * 3 + k)


@pytest.mark.parametrize("shape", TINY_SHAPES)
@pytest.mark.parametrize("layout_b", [ROW_MAJOR, COL_MAJOR])
def test_exact_rational_integer(shape, layout_b):
    m, n, k = shape
    assert pin_exact_rational(gemm_real, m, n, k, layout_b, True, seed=5, integer=True)


@pytest.mark.parametrize("layout_b", [ROW_MAJOR, COL_MAJOR])
@pytest.mark.parametrize("integer", [False, True])
def test_block_identity_along_k(layout_b, integer):
    assert pin_k_split(gemm_real, 37, 29, 101, layout_b, seed=21, integer=integer)


@pytest.mark.parametrize("layout_b", [ROW_MAJOR, COL_MAJOR])
def test_mn_split_bitwise(layout_b):
    assert pin_mn_split(gemm_real, 45, 38, 77, layout_b, seed=22)


def test_layout_equivalence_bitwise():
    assert pin_layout_equivalence(gemm_real, 33, 41, 65, seed=23)


def test_transpose_identity_bitwise():
    assert pin_transpose(gemm_real, 19, 27, 53, seed=24)


@pytest.mark.parametrize("layout_b", [ROW_MAJOR, COL_MAJOR])
def test_identity_and_permutation_bitwise(layout_b):
    assert pin_identity_permutation(gemm_real, 23, 31, 40, layout_b, seed=25)


@pytest.mark.parametrize("shape", [(1, 1, 1), (67, 129, 300), (130, 67, 2), (5, 3, 1000)])
@pytest.mark.parametrize("layout_b", [ROW_MAJOR, COL_MAJOR])
def test_closed_form_full_product(shape, layout_b):
    assert pin_closed_form_full(gemm_real, *shape, layout_b)


@pytest.mark.parametrize("layout_b", [ROW_MAJOR, COL_MAJOR])
def test_all_ones(layout_b):
    assert pin_all_ones(gemm_real, 9, 13, 257, layout_b)


@pytest.mark.parametrize("layout_b", [ROW_MAJOR, COL_MAJOR])
def test_numpy_float64_crosscheck(layout_b):
    assert pin_numpy_crosscheck(gemm_real, 64, 80, 96, layout_b, seed=26)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_closed_form_at_workload_shapes_sampled(name):
    """The sampled oracle at every workload's full shape against the closed form."""
    w = WORKLOADS[name]
    A, B = mod_pattern_operands(w.m, w.n, w.k, w.layout_b)
    rows, cols = sample_indices(w.m, w.n, 400, seed=31)
    c, s = oracle.gemm_f64_sampled(A, B, w.m, w.n, w.k, w.layout_b, rows, cols)
    ce, se = closed_form(rows, cols, w.k)
    assert np.array_equal(c, ce) and np.array_equal(s, se)


@pytest.mark.parametrize("layout_b", [ROW_MAJOR, COL_MAJOR])
def test_sampled_equals_full_bitwise(layout_b):
    m, n, k = 57, 83, 129
    A, B = random_operands(m, n, k, layout_b, "normal1", 27, lda=k + 1,
                           ldb=(n if layout_b == ROW_MAJOR else k) + 5)
    ldb = (n if layout_b == ROW_MAJOR else k) + 5
    C, S = oracle.gemm_f64(A, B, m, n, k, layout_b, k + 1, ldb)
    rows, cols = sample_indices(m, n, 300, seed=28)
    c, s = oracle.gemm_f64_sampled(A, B, m, n, k, layout_b, rows, cols, k + 1, ldb)
    assert np.array_equal(c, C[rows, cols]) and np.array_equal(s, S[rows, cols])


def test_rejects_bad_arguments():
    A = np.zeros((4, 4), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.gemm_f64(A, A, 4, 4, 4, 2)
    with pytest.raises(ValueError):
        oracle.gemm_f64(A, A, 4, 4, 5, 0)            # storage too small / lda < k
    with pytest.raises(TypeError):
        oracle.gemm_f64(A.astype(np.float64), A, 4, 4, 4, 0)
    with pytest.raises(ValueError):
        oracle.gemm_f64_sampled(A, A, 4, 4, 4, 0, [4], [0])


def test_tolerance_helper():
    ref = np.array([1.0, -2.0, 0.0])
    s = np.array([10.0, 10.0, 0.0])
    ok, r = oracle.within_tolerance(ref + np.array([1e-4, -1e-4, 1e-6]), ref, s)
    assert ok and r <= 1.0
    ok, r = oracle.within_tolerance(ref + np.array([2e-4, 0, 0]), ref, s)
    assert not ok and r > 1.0
    ok, _ = oracle.within_tolerance(np.array([np.nan, -2.0, 0.0]), ref, s)
    assert not ok


# ----------------------------------------------------------------------------
# Planted mistakes: each wrapped oracle below carries one plausible bug; the
# pin suite must catch every one of them.
# ----------------------------------------------------------------------------

def _mutant_drop_last_term(A, B, m, n, k, layout_b, lda, ldb):
    return oracle.gemm_f64(A, B, m, n, max(k - 1, 0), layout_b, lda, ldb)


def _mutant_wrong_layout(A, B, m, n, k, layout_b, lda, ldb):
    """Reads B with the other layout's index whenever the strides allow it."""
    try:
        return oracle.gemm_f64(A, B, m, n, k, 1 - layout_b, lda, ldb)
    except ValueError:
        return oracle.gemm_f64(A, B, m, n, k, layout_b, lda, ldb)


def _mutant_sign(A, B, m, n, k, layout_b, lda, ldb):
    C, S = oracle.gemm_f64(A, B, m, n, k, layout_b, lda, ldb)
    C = C.copy()
    C[-1, -1] = -C[-1, -1]
    return C, S


def _mutant_row_shift(A, B, m, n, k, layout_b, lda, ldb):
    C, S = oracle.gemm_f64(A, B, m, n, k, layout_b, lda, ldb)
    return np.roll(C, 1, axis=0), np.roll(S, 1, axis=0)


def _mutant_k_misaligned(A, B, m, n, k, layout_b, lda, ldb):
    """B's k index off by one (reads B(k+1, j), zero past the end)."""
    if layout_b == ROW_MAJOR:
        Bl = B.reshape(-1)[: k * ldb].reshape(k, ldb)
        Bs = np.zeros_like(Bl)
        Bs[:-1] = Bl[1:]
    else:
        Bl = B.reshape(-1)[: n * ldb].reshape(n, ldb)
        Bs = np.zeros_like(Bl)
        Bs[:, : k - 1] = Bl[:, 1:k]
    return oracle.gemm_f64(A, np.ascontiguousarray(Bs), m, n, k, layout_b, lda, ldb)


def _mutant_float32_accumulate(A, B, m, n, k, layout_b, lda, ldb):
    """Accumulates in float32 instead of float64."""
    C, S = oracle.gemm_f64(A, B, m, n, k, layout_b, lda, ldb)
    a = A.reshape(-1)
    b = B.reshape(-1)
    C = C.copy()
    for i in range(m):
        for j in range(n):
            acc = np.float32(0)
            for kk in range(k):
                bv = b[kk * ldb + j] if layout_b == ROW_MAJOR else b[j * ldb + kk]
                acc = np.float32(acc + np.float32(a[i * lda + kk]) * np.float32(bv))
            C[i, j] = acc
    return C, S


def _pin_suite(gemm):
    """Returns the names of the pins that fail for ``gemm`` (small sizes)."""
    failed = []
    checks = {
        "exact_rational": lambda: all(pin_exact_rational(gemm, m, n, k, lb, True, 7)
                                      for (m, n, k) in [(2, 3, 5), (7, 5, 17)] for lb in (0, 1)),
        "exact_integer": lambda: all(pin_exact_rational(gemm, 5, 7, 3, lb, False, 8, integer=True)
                                     for lb in (0, 1)),
        "k_split": lambda: all(pin_k_split(gemm, 9, 7, 23, lb, 9) for lb in (0, 1)),
        "mn_split": lambda: all(pin_mn_split(gemm, 12, 10, 9, lb, 10) for lb in (0, 1)),
        "layout": lambda: pin_layout_equivalence(gemm, 6, 9, 11, 11),
        "transpose": lambda: pin_transpose(gemm, 5, 8, 7, 12),
        "identity_perm": lambda: all(pin_identity_permutation(gemm, 6, 7, 8, lb, 13) for lb in (0, 1)),
        "closed_form": lambda: all(pin_closed_form_full(gemm, 11, 13, 17, lb) for lb in (0, 1)),
        "all_ones": lambda: all(pin_all_ones(gemm, 3, 4, 5, lb) for lb in (0, 1)),
    }
    for name, fn in checks.items():
        try:
            ok = fn()
        except Exception:
            ok = False
        if not ok:
            failed.append(name)
    return failed


def test_pin_suite_passes_on_real_oracle():
    assert _pin_suite(gemm_real) == []


@pytest.mark.parametrize("mutant", [_mutant_drop_last_term, _mutant_wrong_layout, _mutant_sign,
                                    _mutant_row_shift, _mutant_k_misaligned,
                                    _mutant_float32_accumulate])
def test_pins_catch_planted_mistakes(mutant):
    assert _pin_suite(mutant), f"no pin caught {mutant.__name__}"

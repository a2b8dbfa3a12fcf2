"""Pins for the oracle's column-major A and linear-layer epilogue.

Column-major A (``A[i][k] = A_store[k*lda + i]``, the pages' column-major
convention of "PMPP Chapter 06", section 1, applied to the first operand) is
checked against exact rational arithmetic on tiny inputs and against the same
values stored row-major.  The epilogue ``act(alpha*AB + beta*C_in + bias[j])``
is checked against what its definitions fix: special cases (alpha = 0,
beta = 0, no bias), the textbook values of the normal distribution function
Phi behind GELU (x * Phi(x)), the identity GELU(x) - GELU(-x) = x, and ReLU's
definition.  ``test_pins_catch_planted_mistakes_ex`` requires each planted
mistake to trip one of these pins.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from workloads import COL_MAJOR, ROW_MAJOR, epilogue_operands, random_operands

U64 = 2.0 ** -53


def exact_rational_ex(A, B, m, n, k, layout_a, layout_b, lda, ldb):
    a = A.reshape(-1)
    b = B.reshape(-1)
    C = [[Fraction(0)] * n for _ in range(m)]
    for i in range(m):
        for j in range(n):
            acc = Fraction(0)
            for kk in range(k):
                av = a[i * lda + kk] if layout_a == ROW_MAJOR else a[kk * lda + i]
                bv = b[kk * ldb + j] if layout_b == ROW_MAJOR else b[j * ldb + kk]
                acc += Fraction(float(av)) * Fraction(float(bv))
            C[i][j] = acc
    return C


def real_gemm(A, B, m, n, k, layout_a, layout_b, lda, ldb):
    return oracle.gemm_f64(A, B, m, n, k, layout_b, lda, ldb, layout_a=layout_a)


# ---- pins (each takes the functions under test and returns True if it holds)

def pin_col_a_exact(gemm, m, n, k, layout_b, padded, seed):
    lda = m + 2 if padded else m
    ldb = (n if layout_b == ROW_MAJOR else k) + (3 if padded else 0)
    A, B = random_operands(m, n, k, layout_b, "normal1", seed, lda=lda, ldb=ldb, layout_a=COL_MAJOR)
    C, S = gemm(A, B, m, n, k, COL_MAJOR, layout_b, lda, ldb)
    E = exact_rational_ex(A, B, m, n, k, COL_MAJOR, layout_b, lda, ldb)
    g = k * U64 / (1 - k * U64)
    return all(abs(Fraction(C[i, j]) - E[i][j]) <= Fraction(g * S[i, j]) + Fraction(1, 10 ** 300)
               for i in range(m) for j in range(n)) and np.isfinite(C).all()


def pin_col_a_equals_row_a(gemm, m, n, k, layout_b, seed):
    A_row, B = random_operands(m, n, k, layout_b, "normal1", seed)
    A_col = np.ascontiguousarray(A_row.T)
    C1, S1 = gemm(A_row, B, m, n, k, ROW_MAJOR, layout_b, k, None)
    C2, S2 = gemm(A_col, B, m, n, k, COL_MAJOR, layout_b, m, None)
    return np.array_equal(C1, C2) and np.array_equal(S1, S2)


PHI_1 = 0.8413447460685429     # Phi(1), textbook value
PHI_2 = 0.9772498680518208     # Phi(2)


def pin_epilogue(epi):
    ab = np.array([[1.0, -1.0, 2.0], [0.0, 3.0, -2.0]])
    s = np.abs(ab) + 1.0
    cin = np.array([[0.5, 0.25, -4.0], [1.0, -1.0, 2.0]])
    bias = np.array([10.0, -20.0, 30.0])
    ok = True
    # alpha = 0, beta = 0: only the bias, broadcast along rows (bias[j]).
    out, sc = epi(ab, s, None, 0.0, 0.0, bias, oracle.ACT_NONE)
    ok &= np.array_equal(out, np.broadcast_to(bias, ab.shape)) and np.array_equal(sc, np.broadcast_to(np.abs(bias), ab.shape))
    # alpha only: a scaling, exact in float64 for these values.
    out, sc = epi(ab, s, None, 2.0, 0.0, None, oracle.ACT_NONE)
    ok &= np.array_equal(out, 2.0 * ab) and np.array_equal(sc, 2.0 * s)
    # beta: C_in enters as beta * C_in; beta = 0 ignores C_in even if NaN.
    out, _ = epi(ab, s, cin, 1.0, -2.0, None, oracle.ACT_NONE)
    ok &= np.array_equal(out, ab - 2.0 * cin)
    out, _ = epi(ab, s, np.full(ab.shape, np.nan), 1.0, 0.0, None, oracle.ACT_NONE)
    ok &= np.array_equal(out, ab)
    # ReLU.
    out, _ = epi(ab, s, None, 1.0, 0.0, None, oracle.ACT_RELU)
    ok &= np.array_equal(out, np.where(ab > 0, ab, 0.0))
    # GELU = x * Phi(x): textbook values and the odd identity.
    out, _ = epi(ab, s, None, 1.0, 0.0, None, oracle.ACT_GELU)
    ok &= abs(out[0, 0] - PHI_1) < 1e-15 and abs(out[0, 1] + (1 - PHI_1)) < 1e-15
    ok &= abs(out[0, 2] - 2 * PHI_2) < 1e-15 and out[1, 0] == 0.0
    x = np.linspace(-6, 6, 97)[None, :]
    gp, _ = epi(x, np.abs(x), None, 1.0, 0.0, None, oracle.ACT_GELU)
    gm, _ = epi(-x, np.abs(x), None, 1.0, 0.0, None, oracle.ACT_GELU)
    ok &= np.allclose(gp - gm, x, rtol=0, atol=1e-14)
    return bool(ok)


@pytest.mark.parametrize("shape", [(1, 1, 1), (2, 3, 5), (5, 7, 3), (7, 5, 17), (17, 3, 2)])
@pytest.mark.parametrize("layout_b", [ROW_MAJOR, COL_MAJOR])
@pytest.mark.parametrize("padded", [False, True])
def test_col_a_exact_rational(shape, layout_b, padded):
    assert pin_col_a_exact(real_gemm, *shape, layout_b, padded, seed=7 + sum(shape))


@pytest.mark.parametrize("layout_b", [ROW_MAJOR, COL_MAJOR])
def test_col_a_equals_row_a_bitwise(layout_b):
    assert pin_col_a_equals_row_a(real_gemm, 37, 29, 53, layout_b, seed=11)


def test_col_a_sampled_equals_full():
    m, n, k = 23, 31, 47
    A, B = random_operands(m, n, k, ROW_MAJOR, "normal1", 12, layout_a=COL_MAJOR)
    C, S = oracle.gemm_f64(A, B, m, n, k, ROW_MAJOR, layout_a=COL_MAJOR)
    rows, cols = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
    c, s = oracle.gemm_f64_sampled(A, B, m, n, k, ROW_MAJOR, rows.ravel(), cols.ravel(), layout_a=COL_MAJOR)
    assert np.array_equal(c, C.ravel()) and np.array_equal(s, S.ravel())


def test_epilogue_pins():
    assert pin_epilogue(oracle.epilogue_f64)


def test_epilogue_operands_shapes():
    c_in, bias = epilogue_operands(5, 7, 3)
    assert c_in.shape == (5, 7) and bias.shape == (7,) and c_in.dtype == np.float32


# ---- planted mistakes

def _gemm_col_a_read_row(A, B, m, n, k, layout_a, layout_b, lda, ldb):
    # column-major A read as if row-major with the same stride
    if layout_a == COL_MAJOR:
        A2 = np.full(m * max(lda, k) + k, 0, dtype=np.float32)
        flat = A.reshape(-1)
        for i in range(m):
            for kk in range(k):
                A2[i * lda + kk] = flat[i * lda + kk] if i * lda + kk < flat.size else 0.0
        return oracle.gemm_f64(A2, B, m, n, k, layout_b, max(lda, k), ldb)
    return real_gemm(A, B, m, n, k, layout_a, layout_b, lda, ldb)


def _gemm_col_a_transposed_wrong(A, B, m, n, k, layout_a, layout_b, lda, ldb):
    C, S = real_gemm(A, B, m, n, k, layout_a, layout_b, lda, ldb)
    if layout_a == COL_MAJOR and m > 1:
        C = C[::-1].copy()
    return C, S


def _epi_gelu_wrong_scale(ab, s, cin, alpha, beta, bias, act):
    if act == oracle.ACT_GELU:
        from scipy.special import erf
        x = alpha * np.asarray(ab, dtype=np.float64)
        return 0.5 * x * (1.0 + erf(x)), abs(alpha) * s
    return oracle.epilogue_f64(ab, s, cin, alpha, beta, bias, act)


def _epi_bias_by_row(ab, s, cin, alpha, beta, bias, act):
    if bias is not None:
        ab = np.asarray(ab, dtype=np.float64)
        b = np.asarray(bias)[: ab.shape[0], None] if ab.ndim == 2 and ab.shape[0] <= len(bias) else bias
        out, sc = oracle.epilogue_f64(ab, s, cin, alpha, beta, None, act)
        return out + b, sc + np.abs(b)
    return oracle.epilogue_f64(ab, s, cin, alpha, beta, bias, act)


def _epi_beta_on_product(ab, s, cin, alpha, beta, bias, act):
    if beta != 0.0:
        return oracle.epilogue_f64(np.asarray(ab) * (alpha + beta), s, None, 1.0, 0.0, bias, act)
    return oracle.epilogue_f64(ab, s, cin, alpha, beta, bias, act)


def _epi_relu_leaky(ab, s, cin, alpha, beta, bias, act):
    out, sc = oracle.epilogue_f64(ab, s, cin, alpha, beta, bias, oracle.ACT_NONE if act == oracle.ACT_RELU else act)
    if act == oracle.ACT_RELU:
        out = np.where(out > 0, out, 0.01 * out)
    return out, sc


def test_ex_pins_pass_on_real_oracle():
    assert pin_col_a_exact(real_gemm, 5, 7, 3, ROW_MAJOR, True, 1)
    assert pin_col_a_equals_row_a(real_gemm, 9, 4, 6, COL_MAJOR, 2)
    assert pin_epilogue(oracle.epilogue_f64)


@pytest.mark.parametrize("mutant", [_gemm_col_a_read_row, _gemm_col_a_transposed_wrong])
def test_pins_catch_planted_gemm_mistakes_ex(mutant):
    caught = (not pin_col_a_exact(mutant, 5, 7, 3, ROW_MAJOR, True, 1)
              or not pin_col_a_equals_row_a(mutant, 9, 4, 6, COL_MAJOR, 2))
    assert caught


@pytest.mark.parametrize("mutant", [_epi_gelu_wrong_scale, _epi_bias_by_row, _epi_beta_on_product, _epi_relu_leaky])
def test_pins_catch_planted_epilogue_mistakes(mutant):
    assert not pin_epilogue(mutant)

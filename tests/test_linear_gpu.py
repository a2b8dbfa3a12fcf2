"""Linear-layer layouts and epilogue on the GPU, through the C ABI.

C = act(alpha * A.B + beta * C_in + bias[j]) with A row- or column-major,
against the oracle's product and epilogue (float64).  Tolerance: the
product's |err| <= 1e-5 * S + 1e-6 carries through alpha; the float32
epilogue adds a few roundings of |alpha|*S + |beta*C_in| + |bias| (the scale
S' the oracle returns), ReLU is 1-Lipschitz, GELU at most 1.13-Lipschitz with
an erf approximation error below 1e-7 * |x| <= 1e-7 * S'; so
|err| <= 1.2e-5 * S' + 1.2e-6.  Integer-valued operands, C_in and bias with
alpha = beta = 1 and no GELU are exact in float32 and must match bitwise.
"""
import numpy as np
import pytest
import torch

import dense_gemm_optimisation_fp32_amd as g
import oracle
from tests.gpu_helpers import device, to_dev
from workloads import (COL_MAJOR, ROW_MAJOR, WORKLOADS, epilogue_operands, random_operands,
                       sample_indices)

pytestmark = pytest.mark.gpu

REL, ABS = 1.2e-5, 1.2e-6
EX_VARIANTS = ["dma_256x256x16_w4x2_s4", "dma_256x256x16_w2x2_s4", "dma_256x128x16_w2x2_s3",
               "dma_128x128x16_w2x2_s3", "dma_64x128x16_w2x2_s2", "dma_64x64x16_w2x2_s2", "dma_64x64x16_w2x2_s3"]
ACTS = [g.GEMM_F32_ACT_NONE, g.GEMM_F32_ACT_RELU, g.GEMM_F32_ACT_GELU]


def variant_index(name):
    for v in range(g.gemm_f32_num_variants()):
        if g.gemm_f32_variant_info(v)["name"] == name:
            return v
    raise KeyError(name)


def run_ex(A, B, m, n, k, layout_a, layout_b, lda=None, ldb=None, ldc=None, epilogue=0, alpha=1.0, beta=0.0,
           c_in=None, bias=None, act=0, c_fill=0.0, repeat=1):
    lda = (k if layout_a == ROW_MAJOR else m) if lda is None else lda
    ldb = (n if layout_b == ROW_MAJOR else k) if ldb is None else ldb
    ldc = n if ldc is None else ldc
    dA, dB = to_dev(A), to_dev(B)
    C0 = np.full((m, ldc), np.float32(c_fill), dtype=np.float32)
    if c_in is not None:
        C0[:, :n] = c_in
    dbias = to_dev(bias) if bias is not None else None
    plan = g.gemm_f32_create_ex(m, n, k, layout_a, layout_b, lda, ldb, ldc, epilogue)
    outs = []
    try:
        info = g.gemm_f32_describe(plan)
        stream = torch.cuda.current_stream().cuda_stream
        for _ in range(repeat):
            dC = to_dev(C0.reshape(-1)[: (m - 1) * ldc + n])
            g.gemm_f32_run_ex(plan, dA.data_ptr(), dB.data_ptr(), dC.data_ptr(), alpha, beta,
                              dbias.data_ptr() if dbias is not None else None, act, stream)
            torch.cuda.synchronize()
            full = C0.copy().reshape(-1)
            full[: (m - 1) * ldc + n] = dC.cpu().numpy()
            outs.append(full.reshape(m, ldc))
    finally:
        g.gemm_f32_destroy(plan)
    return outs[-1], info, outs


def check(C, ref, scale, what):
    ok, ratio = oracle.within_tolerance(C, ref, scale, REL, ABS)
    assert ok, f"{what}: max error ratio {ratio:.3g}"
    return ratio


SHAPES = [(300, 520, 77), (513, 257, 1000), (129, 131, 33), (1, 300, 17), (37, 1, 5), (64, 64, 4096)]


@pytest.mark.parametrize("vname", EX_VARIANTS)
@pytest.mark.parametrize("layout_a", [ROW_MAJOR, COL_MAJOR])
@pytest.mark.parametrize("layout_b", [ROW_MAJOR, COL_MAJOR])
def test_layouts_plain_product(vname, layout_a, layout_b, monkeypatch):
    monkeypatch.setenv("GEMM_F32_VARIANT", str(variant_index(vname)))
    for (m, n, k) in SHAPES:
        print(f"\n[case] {vname} layout_a={layout_a} layout_b={layout_b} shape={(m, n, k)}", flush=True)
        A, B = random_operands(m, n, k, layout_b, "normal1", seed=100 + m + k, layout_a=layout_a)
        C, info, _ = run_ex(A, B, m, n, k, layout_a, layout_b)
        assert info["name"] == vname and info["layout_a"] == layout_a
        Cref, S = oracle.gemm_f64(A, B, m, n, k, layout_b, layout_a=layout_a)
        ok, ratio = oracle.within_tolerance(C, Cref, S)
        assert ok, f"{vname} {(m, n, k)}: ratio {ratio:.3g}"


@pytest.mark.parametrize("vname", EX_VARIANTS)
@pytest.mark.parametrize("layout_a", [ROW_MAJOR, COL_MAJOR])
@pytest.mark.parametrize("act", ACTS)
def test_epilogue_vs_oracle(vname, layout_a, act, monkeypatch):
    monkeypatch.setenv("GEMM_F32_VARIANT", str(variant_index(vname)))
    for (m, n, k), layout_b in [((300, 520, 77), ROW_MAJOR), ((513, 257, 1000), COL_MAJOR),
                                ((129, 131, 33), ROW_MAJOR)]:
        print(f"\n[case] epilogue {vname} layout_a={layout_a} act={act} shape={(m, n, k)}", flush=True)
        A, B = random_operands(m, n, k, layout_b, "normal1", seed=200 + m, layout_a=layout_a)
        c_in, bias = epilogue_operands(m, n, seed=300 + m)
        AB, S = oracle.gemm_f64(A, B, m, n, k, layout_b, layout_a=layout_a)
        for alpha, beta, with_bias in [(0.5, -1.5, True), (1.0, 0.0, True), (2.0, 0.25, False)]:
            C, info, outs = run_ex(A, B, m, n, k, layout_a, layout_b, epilogue=1, alpha=alpha, beta=beta,
                                   c_in=c_in, bias=bias if with_bias else None, act=act, repeat=2)
            assert info["epilogue"] == 1
            ref, scale = oracle.epilogue_f64(AB, S, c_in, alpha, beta, bias if with_bias else None, act)
            check(C[:, :n], ref, scale, f"{vname} alpha={alpha} beta={beta} bias={with_bias} act={act}")
            assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("vname", EX_VARIANTS)
def test_epilogue_integer_bitexact_and_c_untouched(vname, monkeypatch):
    """Integer operands, C_in and bias, alpha = beta = 1: exact.  beta = 0
    leaves C unread (NaN there does not leak), and C's row padding is never
    written."""
    monkeypatch.setenv("GEMM_F32_VARIANT", str(variant_index(vname)))
    m, n, k = 300, 520, 77
    ldc = n + 5
    for layout_a in (ROW_MAJOR, COL_MAJOR):
        A, B = random_operands(m, n, k, ROW_MAJOR, "int8range", seed=400, layout_a=layout_a)
        rng = np.random.default_rng(401)
        c_in = rng.integers(-50, 51, (m, n)).astype(np.float32)
        bias = rng.integers(-9, 10, n).astype(np.float32)
        AB, S = oracle.gemm_f64(A, B, m, n, k, ROW_MAJOR, layout_a=layout_a)
        for act in (g.GEMM_F32_ACT_NONE, g.GEMM_F32_ACT_RELU):
            C, _, _ = run_ex(A, B, m, n, k, layout_a, ROW_MAJOR, ldc=ldc, epilogue=1, alpha=1.0, beta=1.0,
                             c_in=c_in, bias=bias, act=act, c_fill=-3.5)
            ref, _ = oracle.epilogue_f64(AB, S, c_in, 1.0, 1.0, bias, act)
            assert np.array_equal(C[:, :n].astype(np.float64), ref)
            assert np.all(C[:-1, n:] == np.float32(-3.5))
        C, _, _ = run_ex(A, B, m, n, k, layout_a, ROW_MAJOR, ldc=ldc, epilogue=1, alpha=1.0, beta=0.0,
                         c_in=np.full((m, n), np.nan, dtype=np.float32), bias=bias, act=g.GEMM_F32_ACT_NONE)
        ref, _ = oracle.epilogue_f64(AB, S, None, 1.0, 0.0, bias, g.GEMM_F32_ACT_NONE)
        assert np.array_equal(C[:, :n].astype(np.float64), ref)


@pytest.mark.parametrize("layout_a", [ROW_MAJOR, COL_MAJOR])
def test_padded_column_major_a(layout_a):
    """lda above its minimum with NaN in A's padding: the padding never reaches C."""
    m, n, k = 200, 190, 70
    lda = (k if layout_a == ROW_MAJOR else m) + 7
    A, B = random_operands(m, n, k, ROW_MAJOR, "uniform", seed=500, lda=lda, layout_a=layout_a)
    C, _, _ = run_ex(A, B, m, n, k, layout_a, ROW_MAJOR, lda=lda)
    Cref, S = oracle.gemm_f64(A, B, m, n, k, ROW_MAJOR, lda=lda, layout_a=layout_a)
    ok, ratio = oracle.within_tolerance(C, Cref, S)
    assert ok, ratio


def test_run_ex_rejects_epilogue_on_plain_plan():
    m, n, k = 64, 64, 64
    plan = g.gemm_f32_create_ex(m, n, k, COL_MAJOR, ROW_MAJOR, m, n, n, 0)
    try:
        dA = torch.zeros(m * k, device=device())
        with pytest.raises(g.GemmF32Error):
            g.gemm_f32_run_ex(plan, dA.data_ptr(), dA.data_ptr(), dA.data_ptr(), 2.0, 0.0, None, 0,
                              torch.cuda.current_stream().cuda_stream)
        with pytest.raises(g.GemmF32Error):
            g.gemm_f32_run_ex(plan, dA.data_ptr(), dA.data_ptr(), dA.data_ptr(), 1.0, 0.0, None, 7,
                              torch.cuda.current_stream().cuda_stream)
    finally:
        g.gemm_f32_destroy(plan)


@pytest.mark.parametrize("act", ["relu", "gelu"])
def test_ffn_linear_full_size_every_element(act):
    """The FFN shape as a linear layer: act(X.W + bias), X 8192 x 4096,
    W 4096 x 14336 stored as the usual (14336, 4096) weight (column-major B);
    every element against the oracle's product and epilogue."""
    w = WORKLOADS["ffn"]
    m, n, k = w.m, w.n, w.k
    print(f"\n[case] ffn linear act={act}", flush=True)
    A, B = random_operands(m, n, k, COL_MAJOR, w.dist, w.seed)
    _, bias = epilogue_operands(1, n, seed=600)
    X = torch.from_numpy(A).to(device())
    W = torch.from_numpy(B).to(device())               # (n, k) row-major = column-major B
    b = torch.from_numpy(bias).to(device())
    Y = g.linear(X, W.t(), b, activation=act)
    torch.cuda.synchronize()
    out = Y.cpu().numpy()
    del X, W, Y
    ab, s = oracle.gemm_f64(A, B, m, n, k, COL_MAJOR)
    ref, scale = oracle.epilogue_f64(ab, s, None, 1.0, 0.0, bias[None, :],
                                     oracle.ACT_RELU if act == "relu" else oracle.ACT_GELU)
    del ab, s
    ratio = check(out, ref, scale, f"ffn {act}")
    print(f"\n[parity] ffn linear bias+{act}: max error ratio {ratio:.3g}", flush=True)


def test_binding_linear_column_major_a_and_beta():
    m, n, k = 250, 270, 190
    A, B = random_operands(m, n, k, ROW_MAJOR, "normal1", seed=700, layout_a=COL_MAJOR)
    c_in, bias = epilogue_operands(m, n, seed=701)
    At = torch.from_numpy(A).to(device()).t()           # logical (m, k), column-major
    Bt = torch.from_numpy(B).to(device())
    out = torch.from_numpy(c_in).to(device()).clone()
    Y = g.linear(At, Bt, torch.from_numpy(bias).to(device()), activation="gelu", alpha=0.75, beta=0.5, out=out)
    AB, S = oracle.gemm_f64(A, B, m, n, k, ROW_MAJOR, layout_a=COL_MAJOR)
    ref, scale = oracle.epilogue_f64(AB, S, c_in, 0.75, 0.5, bias, oracle.ACT_GELU)
    check(Y.cpu().numpy(), ref, scale, "linear")
    M = g.matmul(At, Bt)
    ok, ratio = oracle.within_tolerance(M.cpu().numpy(), AB, S)
    assert ok, ratio


def test_linear_dispatch_choice():
    """Column-major A, the fused epilogue and column-major B all take the
    eight-wavefront 256x256 tile on whole-wave shapes, where it measured
    fastest (on a 256-CU MI355X); a shape of 2.25 waves of it keeps 128x128."""
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the choice was measured on a 256-CU MI355X")
    m = n = k = 4096
    info = g.Plan(m, n, k, ROW_MAJOR, m, n, n, layout_a=COL_MAJOR).info
    assert info["name"] == "dma_256x256x16_w4x2_s4" and info["stream_k"] == 0
    m, n, k = 8192, 14336, 4096
    info = g.Plan(m, n, k, ROW_MAJOR, k, n, n, epilogue=1).info
    assert info["name"] == "dma_256x256x16_w4x2_s4" and info["stream_k"] == 0
    info = g.Plan(m, n, k, ROW_MAJOR, m, n, n, layout_a=COL_MAJOR).info
    assert info["name"] == "dma_256x256x16_w4x2_s4"
    info = g.Plan(4096, 4096, 4096, COL_MAJOR, 4096, 4096, 4096, layout_a=COL_MAJOR).info
    assert info["name"] == "dma_256x256x16_w4x2_s4"
    info = g.Plan(6144, 6144, 6144, COL_MAJOR, 6144, 6144, 6144, epilogue=1).info
    assert info["name"] == "dma_128x128x16_w2x2_s3"


def test_group_m_default_per_tile():
    """The 256x256 tile rasterises in groups of 4 tile-rows, the others in 8."""
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the choice was measured on a 256-CU MI355X")
    assert g.Plan(4096, 4096, 4096, ROW_MAJOR, 4096, 4096, 4096).info["group_m"] == 4
    assert g.Plan(4096, 4096, 4096, COL_MAJOR, 4096, 4096, 4096).info["group_m"] == 4
    assert g.Plan(6144, 6144, 6144, ROW_MAJOR, 6144, 6144, 6144).info["group_m"] == 8


# Few rows (few tiles, few columns) with the epilogue: the few-row kernel applies it
# where it writes C (one k split, or the last split of a tile to finish), the transposed
# few-column plans (up to four rows, column-major B) and the few-column
# kernels (N <= 8) where they store C's element.  (shape, B layout,
# plan name, k splits.)
FEW_ROW_EX = [((16, 4096, 4096), ROW_MAJOR, "skinny_16x64_w16_d4", 4),
              ((16, 4096, 4096), COL_MAJOR, "skinny_16x64_w16_d4", 4),
              ((2, 4096, 4096), COL_MAJOR, "skinny_16x32_w16_d4", 2),
              ((24, 2048, 3000), COL_MAJOR, "skinny_32x64_w8_d4", 8),
              ((5, 2050, 777), ROW_MAJOR, "skinny_16x32_w16_d4", 3),
              ((1, 300, 17), ROW_MAJOR, "skinny_16x64_w16_d4", 1),
              ((1, 4096, 4096), COL_MAJOR, "fewcol_8x1_k2048_w8", 1),
              ((1, 3001, 2049), COL_MAJOR, "fewcol_8x1_k2048_w8", 1),
              ((3, 8192, 3000), COL_MAJOR, "fewcol_8x4_k1024", 1),
              ((6, 11008, 3000), COL_MAJOR, "fewcol_8x8_k1024_w8", 1),
              ((256, 256, 4096), ROW_MAJOR, "skinny_16x64_w16_d4", 4),
              ((300, 700, 1500), COL_MAJOR, "skinny_16x64_w8_d4", 1),
              ((1000, 1, 4096), ROW_MAJOR, "fewcol_8x1_k2048", 1),
              ((777, 3, 2500), COL_MAJOR, "fewcol_8x4_k1024", 1),
              ((700, 4, 9000), ROW_MAJOR, "fewcol_8x4_k2048", 1),
              ((513, 7, 1000), COL_MAJOR, "fewcol_8x8_k1024", 1)]


@pytest.mark.parametrize("shape,layout_b,name,split", FEW_ROW_EX)
def test_few_rows_epilogue(shape, layout_b, name, split):
    """The fused epilogue on the few-row plans against the oracle's epilogue,
    runs repeating bit for bit; integer operands with alpha = beta = 1 exact,
    and C's row padding never written."""
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the plans were chosen for a 256-CU MI355X")
    m, n, k = shape
    A, B = random_operands(m, n, k, layout_b, "normal1", seed=500 + m + n)
    c_in, bias = epilogue_operands(m, n, seed=600 + m)
    AB, S = oracle.gemm_f64(A, B, m, n, k, layout_b)
    for act in ACTS:
        for alpha, beta, with_bias in [(0.5, -1.5, True), (1.0, 0.0, False)]:
            print(f"\n[case] few-row epilogue {shape} layout_b={layout_b} act={act} alpha={alpha} beta={beta}",
                  flush=True)
            C, info, outs = run_ex(A, B, m, n, k, ROW_MAJOR, layout_b, epilogue=1, alpha=alpha, beta=beta,
                                   c_in=c_in, bias=bias if with_bias else None, act=act, repeat=2)
            assert info["name"] == name and info["epilogue"] == 1 and info["split_k"] == split
            assert info["transposed"] == (1 if name.startswith("fewcol") and n > 8 else 0)
            ref, scale = oracle.epilogue_f64(AB, S, c_in, alpha, beta, bias if with_bias else None, act)
            check(C[:, :n], ref, scale, f"{name} {shape} act={act} alpha={alpha} beta={beta}")
            assert np.array_equal(outs[0], outs[1])
    A, B = random_operands(m, n, k, layout_b, "int8range", seed=700 + m)
    rng = np.random.default_rng(701)
    c_in = rng.integers(-50, 51, (m, n)).astype(np.float32)
    bias = rng.integers(-9, 10, n).astype(np.float32)
    AB, S = oracle.gemm_f64(A, B, m, n, k, layout_b)
    for act in (g.GEMM_F32_ACT_NONE, g.GEMM_F32_ACT_RELU):
        C, _, _ = run_ex(A, B, m, n, k, ROW_MAJOR, layout_b, ldc=n + 3, epilogue=1, alpha=1.0, beta=1.0,
                         c_in=c_in, bias=bias, act=act, c_fill=-3.5)
        ref, _ = oracle.epilogue_f64(AB, S, c_in, 1.0, 1.0, bias, act)
        assert np.array_equal(C[:, :n].astype(np.float64), ref)
        assert np.all(C[:, n:] == np.float32(-3.5))


# Column-major A on the few-row kernel (16 rows of a column per 64-byte
# read), plain and with the epilogue: (shape, B layout, plan name, k splits
# or None).
COL_A_FEW = [((16, 4096, 4096), ROW_MAJOR, "skinny_16x64_w16_d4", 4),
             ((24, 2048, 3000), COL_MAJOR, "skinny_32x64_w8_d4", 8),
             ((16, 1000, 700), ROW_MAJOR, "skinny_16x64_w16_d4", None),
             ((5, 2050, 777), COL_MAJOR, "skinny_16x32_w16_d4", 3),
             ((200, 190, 70), ROW_MAJOR, "skinny_16x16_w4_d4", 1)]


@pytest.mark.parametrize("shape,layout_b,name,split", COL_A_FEW)
def test_few_rows_column_major_a(shape, layout_b, name, split):
    """Column-major A (lda padded, NaN in the padding) on the few-row plans:
    the plain product (integer operands bit for bit) and the epilogue against
    the oracle."""
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the plans were chosen for a 256-CU MI355X")
    m, n, k = shape
    lda = m + 3
    print(f"\n[case] few rows, column-major A {shape} layout_b={layout_b}", flush=True)
    A, B = random_operands(m, n, k, layout_b, "int8range", seed=820 + m, layout_a=COL_MAJOR, lda=lda)
    C, info, outs = run_ex(A, B, m, n, k, COL_MAJOR, layout_b, lda=lda, repeat=2)
    assert info["name"] == name and info["layout_a"] == COL_MAJOR
    if split is not None:
        assert info["split_k"] == split
    Cref, _ = oracle.gemm_f64(A, B, m, n, k, layout_b, lda=lda, layout_a=COL_MAJOR)
    assert np.array_equal(C[:, :n].astype(np.float64), Cref)
    assert np.array_equal(outs[0], outs[1])
    A, B = random_operands(m, n, k, layout_b, "normal1", seed=830 + m, layout_a=COL_MAJOR, lda=lda)
    c_in, bias = epilogue_operands(m, n, seed=831)
    C, info, _ = run_ex(A, B, m, n, k, COL_MAJOR, layout_b, lda=lda, epilogue=1, alpha=0.5, beta=1.5,
                        c_in=c_in, bias=bias, act=g.GEMM_F32_ACT_GELU)
    assert info["name"] == name and info["epilogue"] == 1
    AB, S = oracle.gemm_f64(A, B, m, n, k, layout_b, lda=lda, layout_a=COL_MAJOR)
    ref, scale = oracle.epilogue_f64(AB, S, c_in, 0.5, 1.5, bias, g.GEMM_F32_ACT_GELU)
    check(C[:, :n], ref, scale, f"{name} column-major A {shape}")


@pytest.mark.parametrize("layout_b", [ROW_MAJOR, COL_MAJOR])
def test_stream_k_epilogue_default_plan(layout_b):
    """Few tiles and long k with the epilogue and row-major A: stream-K over
    64x64 tiles, the epilogue applied by the last segment of each split tile;
    against the oracle's epilogue, runs repeating bit for bit, and integer
    operands exact."""
    m, n, k = 1024, 1024, 8192
    A, B = random_operands(m, n, k, layout_b, "normal1", seed=900)
    c_in, bias = epilogue_operands(m, n, seed=901)
    AB, S = oracle.gemm_f64(A, B, m, n, k, layout_b)
    for act, alpha, beta in ((g.GEMM_F32_ACT_GELU, 0.5, -1.5), (g.GEMM_F32_ACT_NONE, 1.0, 0.0)):
        print(f"\n[case] stream-K epilogue layout_b={layout_b} act={act}", flush=True)
        C, info, outs = run_ex(A, B, m, n, k, ROW_MAJOR, layout_b, epilogue=1, alpha=alpha, beta=beta,
                               c_in=c_in, bias=bias, act=act, repeat=2)
        assert info["name"] == "dma_64x64x16_w2x2_s2" and info["stream_k"] > 1 and info["epilogue"] == 1
        ref, scale = oracle.epilogue_f64(AB, S, c_in, alpha, beta, bias, act)
        check(C[:, :n], ref, scale, f"stream-K epilogue act={act}")
        assert np.array_equal(outs[0], outs[1])
    A, B = random_operands(m, n, k, layout_b, "int8range", seed=902)
    rng = np.random.default_rng(903)
    c_in = rng.integers(-50, 51, (m, n)).astype(np.float32)
    bias = rng.integers(-9, 10, n).astype(np.float32)
    AB, S = oracle.gemm_f64(A, B, m, n, k, layout_b)
    C, _, _ = run_ex(A, B, m, n, k, ROW_MAJOR, layout_b, epilogue=1, alpha=1.0, beta=1.0, c_in=c_in, bias=bias,
                     act=g.GEMM_F32_ACT_RELU)
    ref, _ = oracle.epilogue_f64(AB, S, c_in, 1.0, 1.0, bias, g.GEMM_F32_ACT_RELU)
    assert np.array_equal(C[:, :n].astype(np.float64), ref)


@pytest.mark.parametrize("wgs,shared", [(3, None), (40, None), (7, 5)])
def test_stream_k_epilogue_forced(wgs, shared, monkeypatch):
    """Forced stream-K with the epilogue on ragged 64x64 tiles: segments
    shorter than a tile, tiles shared by many segments, and (with a subset of
    shared tiles) whole tiles stored by the stream-K kernel itself."""
    monkeypatch.setenv("GEMM_F32_VARIANT", str(variant_index("dma_64x64x16_w2x2_s2")))
    monkeypatch.setenv("GEMM_F32_SK_WGS", str(wgs))
    if shared is not None:
        monkeypatch.setenv("GEMM_F32_SK_TILES", str(shared))
    m, n, k = 300, 200, 999
    A, B = random_operands(m, n, k, ROW_MAJOR, "normal1", seed=910 + wgs)
    c_in, bias = epilogue_operands(m, n, seed=911)
    AB, S = oracle.gemm_f64(A, B, m, n, k, ROW_MAJOR)
    C, info, outs = run_ex(A, B, m, n, k, ROW_MAJOR, ROW_MAJOR, ldc=n + 3, epilogue=1, alpha=2.0, beta=0.5,
                           c_in=c_in, bias=bias, act=g.GEMM_F32_ACT_GELU, c_fill=-3.5, repeat=2)
    assert info["stream_k"] == wgs and info["stream_k_tiles"] == (shared or info["tiles_m"] * info["tiles_n"])
    ref, scale = oracle.epilogue_f64(AB, S, c_in, 2.0, 0.5, bias, g.GEMM_F32_ACT_GELU)
    check(C[:, :n], ref, scale, f"forced stream-K epilogue wgs={wgs}")
    assert np.array_equal(outs[0], outs[1])
    assert np.all(C[:, n:] == np.float32(-3.5))



# Column-major B with more than two and at most two and a half 128x128 tiles
# per CU: stream-K over 128x128 tiles with the epilogue from k = 3072;
# (shape, whether the plan is that one).
SUB_WAVE_EPI = [((1536, 5632, 3100), True), ((2048, 4608, 2048), False)]


@pytest.mark.parametrize("shape,taken", SUB_WAVE_EPI)
def test_stream_k_epilogue_over_128x128_tiles(shape, taken):
    """The epilogue on stream-K over 128x128 tiles (the last segment of each
    split tile applies it): every element against the oracle's epilogue,
    runs repeating bit for bit, integer operands exact."""
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the choice was measured on a 256-CU MI355X")
    m, n, k = shape
    print(f"\n[case] stream-K epilogue over 128x128 tiles {shape}", flush=True)
    A, B = random_operands(m, n, k, COL_MAJOR, "normal1", seed=920)
    c_in, bias = epilogue_operands(m, n, seed=921)
    AB, S = oracle.gemm_f64(A, B, m, n, k, COL_MAJOR)
    C, info, outs = run_ex(A, B, m, n, k, ROW_MAJOR, COL_MAJOR, epilogue=1, alpha=0.5, beta=-1.5, c_in=c_in,
                           bias=bias, act=g.GEMM_F32_ACT_GELU, repeat=2)
    assert (info["name"] == "dma_128x128x16_w2x2_s3" and info["stream_k"] == 768) == taken, info
    assert info["epilogue"] == 1
    ref, scale = oracle.epilogue_f64(AB, S, c_in, 0.5, -1.5, bias, g.GEMM_F32_ACT_GELU)
    check(C[:, :n], ref, scale, f"{info['name']} epilogue {shape}")
    assert np.array_equal(outs[0], outs[1])
    A, B = random_operands(m, n, k, COL_MAJOR, "int8range", seed=922)
    rng = np.random.default_rng(923)
    c_in = rng.integers(-50, 51, (m, n)).astype(np.float32)
    bias = rng.integers(-9, 10, n).astype(np.float32)
    AB, S = oracle.gemm_f64(A, B, m, n, k, COL_MAJOR)
    C, _, _ = run_ex(A, B, m, n, k, ROW_MAJOR, COL_MAJOR, epilogue=1, alpha=1.0, beta=1.0, c_in=c_in, bias=bias,
                     act=g.GEMM_F32_ACT_RELU)
    ref, _ = oracle.epilogue_f64(AB, S, c_in, 1.0, 1.0, bias, g.GEMM_F32_ACT_RELU)
    assert np.array_equal(C[:, :n].astype(np.float64), ref)

def test_stream_k_epilogue_column_major_a_stays_data_parallel():
    """Column-major A has no stream-K kernels: the few-tile long-k epilogue
    plan runs whole tiles."""
    m, n, k = 1024, 1024, 8192
    plan = g.Plan(m, n, k, ROW_MAJOR, m, n, n, layout_a=COL_MAJOR, epilogue=1)
    assert plan.info["stream_k"] == 0

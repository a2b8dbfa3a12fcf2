"""Parity of the HIP path with the CPU oracle, through the C ABI.

Acceptance per element: |C - C_ref| <= 1e-5 * S + 1e-6 with
S = sum_k |a_ik * b_kj| (both from the oracle, in float64), and bit-exact
equality on integer-valued inputs, where every summation order is exact.

Small shapes span several tiles and ragged tails and are compared element by
element with the full oracle for every compiled variant.  The full workload
shapes run in the plan the benchmark times and are compared element by
element with the full oracle (random and integer-valued inputs), plus a
closed-form integer product checked on every element.
"""
import time

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import run_gemm, variants
from workloads import (COL_MAJOR, ROW_MAJOR, WORKLOADS, mod_pattern_operands, permutation,
                       random_operands, sample_indices, workload_operands)

pytestmark = pytest.mark.gpu

REL, ABS = 1e-5, 1e-6

SMALL_SHAPES = [
    (256, 256, 256),     # the small square workload
    (300, 520, 77),      # ragged in every dimension
    (513, 257, 1000),    # one row/column past a tile edge, k tail
    (1, 1, 1),
    (1, 300, 17),
    (37, 1, 5),
    (129, 131, 33),
    (70, 130, 40),       # N even but not a multiple of 4
    (64, 64, 4096),      # long k
]


def check_close(C, Cref, S, what):
    ok, ratio = oracle.within_tolerance(C, Cref, S, REL, ABS)
    assert ok, f"{what}: max error ratio {ratio:.3g} (> 1 fails), finite={np.isfinite(C).all()}"
    return ratio


def closed_form(rows, cols, k):
    count = k - (k + 1) // 3
    return (((np.asarray(rows) % 7) - 3) * ((np.asarray(cols) % 5) - 2) * count).astype(np.float32)


@pytest.mark.parametrize("variant", variants())
@pytest.mark.parametrize("layout_b", [ROW_MAJOR, COL_MAJOR])
@pytest.mark.parametrize("shape", SMALL_SHAPES)
def test_small_shapes_vs_oracle(variant, layout_b, shape):
    m, n, k = shape
    print(f"\n[case] variant={variant} layout_b={layout_b} shape={shape}", flush=True)
    A, B = random_operands(m, n, k, layout_b, "normal1", seed=1000 + m + n + k)
    C, info = run_gemm(A, B, m, n, k, layout_b, variant=variant)
    Cref, S = oracle.gemm_f64(A, B, m, n, k, layout_b)
    check_close(C, Cref, S, f"{info['name']} {shape} layout {layout_b}")


@pytest.mark.parametrize("variant", variants())
@pytest.mark.parametrize("layout_b", [ROW_MAJOR, COL_MAJOR])
@pytest.mark.parametrize("shape", [(300, 520, 77), (256, 256, 256), (129, 131, 33)])
def test_small_shapes_integer_bitexact(variant, layout_b, shape):
    m, n, k = shape
    print(f"\n[case] integer variant={variant} layout_b={layout_b} shape={shape}", flush=True)
    A, B = random_operands(m, n, k, layout_b, "int8range", seed=2000 + m)
    C, _ = run_gemm(A, B, m, n, k, layout_b, variant=variant)
    Cref, _ = oracle.gemm_f64(A, B, m, n, k, layout_b)
    assert np.array_equal(C.astype(np.float64), Cref)


@pytest.mark.parametrize("variant", variants())
@pytest.mark.parametrize("layout_b", [ROW_MAJOR, COL_MAJOR])
def test_padded_strides_nan_padding_and_c_padding(variant, layout_b):
    """lda/ldb/ldc above the minimum: operand padding holds NaN (it must never
    reach C) and C's padding holds a sentinel (it must never be written)."""
    m, n, k = 200, 190, 70
    lda, ldb, ldc = k + 5, (n if layout_b == ROW_MAJOR else k) + 3, n + 7
    print(f"\n[case] padded variant={variant} layout_b={layout_b}", flush=True)
    A, B = random_operands(m, n, k, layout_b, "uniform", seed=33, lda=lda, ldb=ldb)
    C, _ = run_gemm(A, B, m, n, k, layout_b, lda, ldb, ldc, variant=variant, c_fill=-7.25)
    Cref, S = oracle.gemm_f64(A, B, m, n, k, layout_b, lda, ldb)
    check_close(C[:, :n], Cref, S, "padded")
    assert np.all(C[:-1, n:] == np.float32(-7.25)), "C row padding was written"


@pytest.mark.parametrize("variant", variants())
@pytest.mark.parametrize("layout_b", [ROW_MAJOR, COL_MAJOR])
def test_aligned_strides_with_misaligned_pointers(variant, layout_b):
    """Strides allow 16-byte accesses but the pointers are only 4-byte aligned:
    the per-element class must run and agree."""
    m, n, k = 160, 136, 96
    print(f"\n[case] misaligned variant={variant} layout_b={layout_b}", flush=True)
    A, B = random_operands(m, n, k, layout_b, "normal1", seed=34)
    Cref, S = oracle.gemm_f64(A, B, m, n, k, layout_b)
    for offs in [(1, 0, 0), (0, 3, 0), (0, 0, 2), (1, 1, 1)]:
        C, _ = run_gemm(A, B, m, n, k, layout_b, variant=variant, offsets=offs)
        check_close(C, Cref, S, f"offsets {offs}")


@pytest.mark.parametrize("variant", variants())
def test_identity_and_permutation_bitwise(variant):
    m, n, k = 96, 80, 128
    print(f"\n[case] identity/permutation variant={variant}", flush=True)
    A, B = random_operands(m, n, k, ROW_MAJOR, "normal1", seed=35)
    eye = np.eye(k, dtype=np.float32)
    C, _ = run_gemm(A, eye, m, k, k, ROW_MAJOR, variant=variant)
    assert np.array_equal(C, A)
    C, _ = run_gemm(eye, B, k, n, k, ROW_MAJOR, variant=variant)
    assert np.array_equal(C, B)
    p = permutation(k, 36)
    P = np.zeros((k, k), dtype=np.float32)
    P[p, np.arange(k)] = 1.0                           # (A.P)[i][j] = A[i][p[j]]
    C, _ = run_gemm(A, np.ascontiguousarray(P.T), m, k, k, COL_MAJOR, variant=variant)
    assert np.array_equal(C, A[:, p])


@pytest.mark.parametrize("variant", variants())
def test_run_to_run_bitwise_determinism(variant):
    m, n, k = 384, 320, 512
    print(f"\n[case] determinism variant={variant}", flush=True)
    A, B = random_operands(m, n, k, ROW_MAJOR, "normal1", seed=37)
    _, _, outs = run_gemm(A, B, m, n, k, ROW_MAJOR, variant=variant, repeat=3)
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


def test_split_k_plan_reused_across_inputs():
    """A few-row plan with k-splits keeps the previous run's partial sums in
    its workspace: alternating inputs on one plan must give each input's own
    result, bit for bit, every time."""
    import dense_gemm_optimisation_fp32_amd as g
    m, n, k = 16, 300, 2000
    plan = g.gemm_f32_create(m, n, k, ROW_MAJOR, k, n, n)
    try:
        info = g.gemm_f32_describe(plan)
        assert info["kind"] == g.GEMM_F32_KIND_SKINNY and info["split_k"] > 1
        sets = [random_operands(m, n, k, ROW_MAJOR, "normal1", seed=50 + i) for i in range(2)]
        dev = [(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()) for A, B in sets]
        refs = [oracle.gemm_f64(A, B, m, n, k, ROW_MAJOR) for A, B in sets]
        first = [None, None]
        stream = torch.cuda.current_stream().cuda_stream
        for it in range(6):
            i = it % 2
            C = torch.full((m, n), -1.0, device="cuda")
            g.gemm_f32_run(plan, dev[i][0].data_ptr(), dev[i][1].data_ptr(), C.data_ptr(), stream)
            out = C.cpu().numpy()
            check_close(out, refs[i][0], refs[i][1], f"run {it}")
            if first[i] is None:
                first[i] = out
            assert np.array_equal(out, first[i])
    finally:
        g.gemm_f32_destroy(plan)


@pytest.mark.parametrize("split", [2, 3, 7, 16])
@pytest.mark.parametrize("layout_b", [ROW_MAJOR, COL_MAJOR])
def test_split_k_counts_forced(split, layout_b, monkeypatch):
    """Few-row plans with a forced number of k-splits (the splits meet in the
    last workgroup of each tile): every run matches the oracle and repeats
    bit for bit, including runs after the arrival counters were reset."""
    import dense_gemm_optimisation_fp32_amd as g
    monkeypatch.setenv("GEMM_F32_SPLIT_K", str(split))
    m, n, k = 20, 130, 999
    print(f"\n[case] forced split={split} layout_b={layout_b}", flush=True)
    A, B = random_operands(m, n, k, layout_b, "normal1", seed=60 + split)
    ldb = n if layout_b == ROW_MAJOR else k
    plan = g.gemm_f32_create(m, n, k, layout_b, k, ldb, n)
    try:
        info = g.gemm_f32_describe(plan)
        assert info["kind"] == g.GEMM_F32_KIND_SKINNY and info["split_k"] == split
        dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
        Cref, S = oracle.gemm_f64(A, B, m, n, k, layout_b)
        stream = torch.cuda.current_stream().cuda_stream
        outs = []
        for _ in range(5):
            C = torch.full((m, n), float("nan"), device="cuda")
            g.gemm_f32_run(plan, dA.data_ptr(), dB.data_ptr(), C.data_ptr(), stream)
            outs.append(C.cpu().numpy())
        check_close(outs[0], Cref, S, f"split {split}")
        assert all(np.array_equal(outs[0], o) for o in outs[1:])
    finally:
        g.gemm_f32_destroy(plan)


def dma_variants():
    import dense_gemm_optimisation_fp32_amd as g
    return [v for v in variants() if g.gemm_f32_variant_info(v)["name"].startswith("dma_")]


@pytest.mark.parametrize("variant", dma_variants())
@pytest.mark.parametrize("layout_b", [ROW_MAJOR, COL_MAJOR])
@pytest.mark.parametrize("wgs", [2, 3, 7, 16, 40])
def test_stream_k_forced(variant, layout_b, wgs, monkeypatch):
    """Stream-K plans with a forced number of workgroups: tiles split at
    arbitrary slabs (including ranges shorter than the LDS ring and tiles
    shared by many ranges) match the oracle, integer inputs bit for bit, and
    repeated runs (new epochs, reset counters) repeat bit for bit."""
    monkeypatch.setenv("GEMM_F32_SK_WGS", str(wgs))
    for shape in [(513, 257, 1000), (300, 520, 77)]:
        m, n, k = shape
        print(f"\n[case] stream-K variant={variant} layout_b={layout_b} wgs={wgs} shape={shape}", flush=True)
        A, B = random_operands(m, n, k, layout_b, "normal1", seed=70 + wgs)
        C, info, outs = run_gemm(A, B, m, n, k, layout_b, variant=variant, repeat=3)
        tiles = info["tiles_m"] * info["tiles_n"]
        assert info["stream_k"] == min(wgs, tiles * info["k_tiles"]) and info["stream_k_tiles"] == tiles
        Cref, S = oracle.gemm_f64(A, B, m, n, k, layout_b)
        check_close(C, Cref, S, f"{info['name']} stream-K {wgs} {shape}")
        assert all(np.array_equal(outs[0], o) for o in outs[1:])
        A, B = random_operands(m, n, k, layout_b, "int8range", seed=80 + wgs)
        C, _ = run_gemm(A, B, m, n, k, layout_b, variant=variant)
        Cref, _ = oracle.gemm_f64(A, B, m, n, k, layout_b)
        assert np.array_equal(C.astype(np.float64), Cref)


@pytest.mark.parametrize("wgs", [256, 512])
def test_stream_k_many_segments_per_tile(wgs, monkeypatch):
    """16 tiles of 64x64 shared by 256 or 512 workgroups: each tile's k-slabs
    are cut into 16 or 32 segments, so the last one to arrive adds that many
    partial tiles (read back eight words per lane at a time).  Matches the
    oracle, integer inputs bit for bit, and repeats bit for bit."""
    import dense_gemm_optimisation_fp32_amd as g

    v = [x for x in dma_variants() if g.gemm_f32_variant_info(x)["name"] == "dma_64x64x16_w2x2_s2"][0]
    monkeypatch.setenv("GEMM_F32_SK_WGS", str(wgs))
    m, n, k = 256, 256, 4096
    print(f"\n[case] stream-K {wgs} workgroups over 16 tiles", flush=True)
    A, B = random_operands(m, n, k, ROW_MAJOR, "normal1", seed=104)
    C, info, outs = run_gemm(A, B, m, n, k, ROW_MAJOR, variant=v, repeat=3)
    assert info["stream_k"] == wgs and info["stream_k_tiles"] == 16
    Cref, S = oracle.gemm_f64(A, B, m, n, k, ROW_MAJOR)
    check_close(C, Cref, S, f"stream-K {wgs} over 16 tiles")
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
    A, B = random_operands(m, n, k, ROW_MAJOR, "int8range", seed=105)
    C, _ = run_gemm(A, B, m, n, k, ROW_MAJOR, variant=v)
    Cref, _ = oracle.gemm_f64(A, B, m, n, k, ROW_MAJOR)
    assert np.array_equal(C.astype(np.float64), Cref)


def test_stream_k_partial_area_limit(monkeypatch):
    """A forced stream-K plan whose partial-sum words would reach 2^31 bytes
    (they are addressed through a 32-bit buffer extent) is rejected at
    creation, before anything is allocated or launched."""
    import dense_gemm_optimisation_fp32_amd as g

    v = [x for x in dma_variants() if g.gemm_f32_variant_info(x)["name"] == "dma_256x128x16_w2x2_s3"][0]
    m = n = k = 4096            # 512 tiles of 256x128, 256 slabs each
    # 2 * P * 256 * 128 * 8 bytes >= 2^31 once P >= 4096
    monkeypatch.setenv("GEMM_F32_SK_WGS", "4096")
    with pytest.raises(g.GemmF32Error) as err:
        g.gemm_f32_create_variant(v, m, n, k, ROW_MAJOR, k, n, n)
    assert err.value.status == g.GEMM_F32_ERR_INVALID_VALUE
    monkeypatch.setenv("GEMM_F32_SK_WGS", "4095")   # just below: a valid plan
    plan = g.gemm_f32_create_variant(v, m, n, k, ROW_MAJOR, k, n, n)
    try:
        assert g.gemm_f32_describe(plan)["stream_k"] == 4095
    finally:
        g.gemm_f32_destroy(plan)


@pytest.mark.parametrize("variant", dma_variants())
@pytest.mark.parametrize("layout_b", [ROW_MAJOR, COL_MAJOR])
@pytest.mark.parametrize("wgs,shared", [(4, 2), (9, 3), (5, 5), (7, 1)])
def test_stream_k_hybrid_forced(variant, layout_b, wgs, shared, monkeypatch):
    """Stream-K over the first `shared` tiles, one workgroup per tile for the
    rest, in one launch: matches the oracle and repeats bit for bit."""
    monkeypatch.setenv("GEMM_F32_SK_WGS", str(wgs))
    monkeypatch.setenv("GEMM_F32_SK_TILES", str(shared))
    m, n, k = 513, 257, 1000
    print(f"\n[case] hybrid stream-K variant={variant} layout_b={layout_b} wgs={wgs} shared={shared}", flush=True)
    A, B = random_operands(m, n, k, layout_b, "normal1", seed=90 + wgs)
    C, info, outs = run_gemm(A, B, m, n, k, layout_b, variant=variant, repeat=3)
    tiles = info["tiles_m"] * info["tiles_n"]
    assert info["stream_k_tiles"] == min(shared, tiles)
    assert info["grid"] == info["stream_k"] + tiles - info["stream_k_tiles"]
    Cref, S = oracle.gemm_f64(A, B, m, n, k, layout_b)
    check_close(C, Cref, S, f"{info['name']} hybrid stream-K {wgs}/{shared}")
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


@pytest.mark.parametrize("layout_b", [ROW_MAJOR, COL_MAJOR])
def test_stream_k_chosen_for_few_tiles_long_k(layout_b):
    """Shapes with too few tiles for the GPU and a long k get a stream-K plan
    by default; it matches the oracle (integer inputs bit for bit)."""
    for (m, n, k) in [(2048, 512, 4096), (1024, 1024, 8192), (640, 2048, 8192), (1024, 1024, 2048),
                      (768, 700, 8192), (1536, 1536, 4096)]:
        print(f"\n[case] default stream-K layout_b={layout_b} shape={(m, n, k)}", flush=True)
        A, B = random_operands(m, n, k, layout_b, "normal1", seed=95)
        C, info, outs = run_gemm(A, B, m, n, k, layout_b, repeat=2)
        assert info["stream_k"] > 1 and info["stream_k_tiles"] == info["tiles_m"] * info["tiles_n"]
        assert np.array_equal(outs[0], outs[1])
        Cref, S = oracle.gemm_f64(A, B, m, n, k, layout_b)
        check_close(C, Cref, S, f"{info['name']} default stream-K {(m, n, k)}")
        A, B = random_operands(m, n, k, layout_b, "int8range", seed=97)
        C, _ = run_gemm(A, B, m, n, k, layout_b)
        Cref, _ = oracle.gemm_f64(A, B, m, n, k, layout_b)
        assert np.array_equal(C.astype(np.float64), Cref)


# One nearly full wave of 64x128 tiles: column-major B from 224 tiles on 256
# CUs (two-stage tiles), row-major B from 240 tiles with k up to 6144
# (three-stage tiles), data-parallel; stream-K over 64x64 tiles otherwise.
ONE_WAVE_CASES = [((512, 4096, 4096), COL_MAJOR, "dma_64x128x16_w2x2_s2", 0),
                  ((960, 2048, 3000), COL_MAJOR, "dma_64x128x16_w2x2_s2", 0),
                  ((128, 14336, 2049), COL_MAJOR, "dma_64x128x16_w2x2_s2", 0),
                  ((500, 4000, 3001), COL_MAJOR, "dma_64x128x16_w2x2_s2", 0),
                  ((384, 4096, 4096), COL_MAJOR, "dma_64x64x16_w2x2_s2", 1),
                  ((512, 4096, 4096), ROW_MAJOR, "dma_64x128x16_w2x2_s3", 0),
                  ((961, 2047, 3001), ROW_MAJOR, "dma_64x128x16_w2x2_s3", 0),
                  ((448, 4096, 4096), ROW_MAJOR, "dma_64x64x16_w2x2_s2", 1),
                  ((512, 4096, 8192), ROW_MAJOR, "dma_64x64x16_w2x2_s2", 1)]


@pytest.mark.parametrize("shape,layout_b,name,stream_k", ONE_WAVE_CASES)
def test_one_wave_of_64x128_tiles(shape, layout_b, name, stream_k):
    """The dispatch's plan where 64x128 tiles make one nearly full wave;
    every element against the oracle (integer inputs bit for bit)."""
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the choices were measured on a 256-CU MI355X")
    m, n, k = shape
    print(f"\n[case] one wave of 64x128 tiles {shape} layout_b={layout_b}", flush=True)
    A, B = random_operands(m, n, k, layout_b, "normal1", seed=3100 + m)
    C, info, outs = run_gemm(A, B, m, n, k, layout_b, repeat=2)
    assert info["name"] == name and (info["stream_k"] > 0) == bool(stream_k)
    assert np.array_equal(outs[0], outs[1])
    Cref, S = oracle.gemm_f64(A, B, m, n, k, layout_b)
    check_close(C, Cref, S, f"{name} {shape}")
    A, B = random_operands(m, n, k, layout_b, "int8range", seed=3200 + m)
    C, _ = run_gemm(A, B, m, n, k, layout_b)
    Cref, _ = oracle.gemm_f64(A, B, m, n, k, layout_b)
    assert np.array_equal(C.astype(np.float64), Cref)


# Column-major B with more than two and at most two and a half 128x128 tiles
# per CU and k from 2048: stream-K over 128x128 tiles; (shape, layout of B,
# whether the plan is that one).
SUB_WAVE_128_CASES = [((1536, 5632, 2100), COL_MAJOR, True),
                      ((2000, 5000, 2049), COL_MAJOR, True),
                      ((2048, 4608, 1024), COL_MAJOR, False),
                      ((2048, 4096, 2048), COL_MAJOR, False),
                      ((1536, 5632, 2100), ROW_MAJOR, False)]


@pytest.mark.parametrize("shape,layout_b,taken", SUB_WAVE_128_CASES)
def test_stream_k_over_128x128_tiles(shape, layout_b, taken):
    """The dispatch's stream-K plan over 128x128 tiles short of three per CU;
    every element against the oracle (integer inputs bit for bit)."""
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the choices were measured on a 256-CU MI355X")
    m, n, k = shape
    print(f"\n[case] stream-K over 128x128 tiles {shape} layout_b={layout_b}", flush=True)
    A, B = random_operands(m, n, k, layout_b, "normal1", seed=3300 + m)
    C, info, outs = run_gemm(A, B, m, n, k, layout_b, repeat=2)
    assert (info["name"] == "dma_128x128x16_w2x2_s3" and info["stream_k"] == 768) == taken, info
    assert np.array_equal(outs[0], outs[1])
    Cref, S = oracle.gemm_f64(A, B, m, n, k, layout_b)
    check_close(C, Cref, S, f"{info['name']} {shape}")
    A, B = random_operands(m, n, k, layout_b, "int8range", seed=3400 + m)
    C, _ = run_gemm(A, B, m, n, k, layout_b)
    Cref, _ = oracle.gemm_f64(A, B, m, n, k, layout_b)
    assert np.array_equal(C.astype(np.float64), Cref)


# Few tiles on the few-row kernel: (shape, the plan with row-major B, with
# column-major B), a plan being (variant, k-split count), or None for a tiled
# plan.  Measured on one MI355X, 256 CUs.
FEW_TILE_CASES = [
    ((256, 256, 256), ("skinny_16x16_w4_d4", 1), ("skinny_16x16_w4_d4", 1)),
    ((64, 256, 4096), ("skinny_16x16_w16_d4", 4), ("skinny_16x16_w16_d4", 4)),
    ((64, 128, 8192), ("skinny_16x16_w16_d4", 8), ("skinny_16x16_w16_d4", 8)),
    ((200, 200, 3000), ("skinny_16x16_w4_d4", 1), ("skinny_16x16_w4_d4", 1)),
    ((100, 100, 800), ("skinny_16x16_w4_d4", 1), ("skinny_16x16_w4_d4", 1)),
    ((128, 512, 4096), ("skinny_16x64_w16_d4", 4), ("skinny_16x64_w16_d4", 4)),
    ((40, 1000, 5000), ("skinny_16x64_w16_d4", 5), ("skinny_16x64_w16_d4", 5)),
    ((300, 700, 1500), ("skinny_16x64_w8_d4", 1), ("skinny_16x64_w8_d4", 1)),
    ((300, 300, 3000), ("skinny_16x64_w8_d4", 2), ("skinny_16x64_w8_d4", 2)),
    ((800, 600, 3000), ("skinny_16x64_w8_d4", 1), None),
    ((250, 600, 2500), ("skinny_16x64_w8_d4", 1), ("skinny_16x64_w8_d4", 1)),
    ((256, 1024, 4096), ("skinny_16x64_w8_d4", 1), None),
    ((768, 768, 1024), ("skinny_16x64_w8_d4", 1), None),
    ((512, 512, 8192), ("skinny_16x64_w8_d4", 1), None),
    ((1024, 1024, 1024), None, None),
    # A few dozen rows against a large B (row-major: the few-row plan up to
    # three 16 x 64 tiles per CU for k <= 4096; column-major: stream-K).
    ((48, 4096, 4096), ("skinny_16x64_w8_d4", 1), None),
    ((96, 2048, 4096), ("skinny_16x64_w8_d4", 1), None),
    ((128, 4096, 4096), ("skinny_16x64_w8_d4", 1), None),
    ((112, 4096, 2048), ("skinny_16x64_w8_d4", 1), None),
    ((48, 8192, 4096), ("skinny_16x64_w8_d4", 1), None),
    ((160, 4096, 4096), ("skinny_16x64_w8_d4", 1), None),
]


@pytest.mark.parametrize("layout_b", [ROW_MAJOR, COL_MAJOR])
@pytest.mark.parametrize("shape,row_plan,col_plan", FEW_TILE_CASES)
def test_few_tile_rows_plan(shape, row_plan, col_plan, layout_b):
    """Shapes with few tiles run the few-row kernel on 16-row tiles with the
    k-split the shape dispatch chose; every element matches the oracle
    (integer inputs bit for bit) and runs repeat bit for bit."""
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the choices were measured on a 256-CU MI355X")
    m, n, k = shape
    want = row_plan if layout_b == ROW_MAJOR else col_plan
    print(f"\n[case] few tiles layout_b={layout_b} shape={shape} plan={want}", flush=True)
    A, B = random_operands(m, n, k, layout_b, "normal1", seed=1700 + m + k)
    C, info, outs = run_gemm(A, B, m, n, k, layout_b, repeat=2)
    if want is None:
        assert info["kind"] == 0 and info["name"].startswith("dma_")
        if k >= 2048 and m < 256:
            assert info["name"] == "dma_64x64x16_w2x2_s2" and info["stream_k"] > 0
    else:
        assert (info["name"], info["split_k"]) == want
        assert info["grid"] == info["tiles_m"] * info["tiles_n"] * want[1]
        if want[1] > 1:
            assert info["grid"] <= 256       # the split fills one workgroup per CU at most
    assert np.array_equal(outs[0], outs[1])
    Cref, S = oracle.gemm_f64(A, B, m, n, k, layout_b)
    check_close(C, Cref, S, f"{info['name']} split {info['split_k']} {shape}")
    A, B = random_operands(m, n, k, layout_b, "int8range", seed=1800 + m + k)
    C, _ = run_gemm(A, B, m, n, k, layout_b)
    Cref, _ = oracle.gemm_f64(A, B, m, n, k, layout_b)
    assert np.array_equal(C.astype(np.float64), Cref)
    # the linear-layer plans take the same plan (the few-row kernel carries
    # the epilogue)
    import dense_gemm_optimisation_fp32_amd as g
    ldb = n if layout_b == ROW_MAJOR else k
    info_ex = g.Plan(m, n, k, layout_b, k, ldb, n, epilogue=1).info
    if want is None:
        assert info_ex["name"].startswith("dma_")
    else:
        assert (info_ex["name"], info_ex["split_k"]) == want


# The shape dispatch's choice on the shapes it was measured on (one MI355X,
# 256 CUs): the fastest of the candidate plans on each.  Plans only,
# nothing is launched.
# (shape, tile, tiles of the partial last wave split by stream-K over one
# workgroup per CU, or 0 for a data-parallel plan)
DISPATCH_CASES = [
    ((4096, 4096, 4096), "dma_256x256x16_w4x2_s4", 0),
    ((8192, 14336, 4096), "dma_256x256x16_w4x2_s4", 0),
    ((8192, 8192, 8192), "dma_256x256x16_w4x2_s4", 0),
    ((6144, 6144, 6144), "dma_128x128x16_w2x2_s3", 0),
    ((3000, 3000, 3000), "dma_64x64x16_w2x2_s2", 0),
    ((2048, 2048, 2048), "dma_64x128x16_w2x2_s2", 0),
    ((1536, 4096, 4096), "dma_64x128x16_w2x2_s2", 0),
    ((5003, 4097, 2049), "dma_128x128x16_w2x2_s3", 0),    # + a one-column sliver (test_column_sliver_plan)
    ((4096, 4608, 4096), "dma_64x64x16_w2x2_s2", 0),
    ((4096, 6144, 4096), "dma_128x128x16_w2x2_s3", 0),
    ((2048, 14336, 4096), "dma_128x128x16_w2x2_s3", 0),
    ((2304, 9216, 4096), "dma_64x128x16_w2x2_s2", 32),
    ((1536, 13824, 4096), "dma_64x128x16_w2x2_s2", 32),
    ((5120, 9856, 4096), "dma_64x128x16_w2x2_s2", 0),
    ((7424, 13568, 4096), "dma_256x128x16_w2x2_s3", 2),
    ((4608, 4608, 4096), "dma_64x128x16_w2x2_s2", 32),
    ((7964, 4668, 2048), "dma_64x128x16_w2x2_s2", 0),
    ((5239, 5308, 4096), "dma_128x128x16_w2x2_s3", 0),
    ((7511, 5443, 6144), "dma_128x128x16_w2x2_s3", 0),
]


@pytest.mark.parametrize("shape,name,tail", DISPATCH_CASES)
def test_dispatch_choice(shape, name, tail):
    import dense_gemm_optimisation_fp32_amd as g

    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the choices were measured on a 256-CU MI355X")
    m, n, k = shape
    info = g.Plan(m, n, k, ROW_MAJOR, k, n, n).info
    assert info["name"] == name
    assert info["sliver_cols"] == (1 if shape == (5003, 4097, 2049) else 0)
    if tail:
        # one workgroup per CU, at most 8 per split tile
        assert info["stream_k"] == min(256, 8 * tail) and info["stream_k_tiles"] == tail
    else:
        assert info["stream_k"] == 0
    # the linear-layer plans never use stream-K
    assert g.Plan(m, n, k, ROW_MAJOR, k, n, n, epilogue=1).info["stream_k"] == 0


def test_linear_plan_for_few_tiles_long_k():
    """A few-tile long-k shape gets stream-K as a plain product and with the
    epilogue and row-major A (the two-stage 64x64 tile's stream-K kernel
    carries it); with column-major A (no stream-K kernel) it gets the
    data-parallel tile with the most tiles rather than the stream-K tile run
    whole."""
    import dense_gemm_optimisation_fp32_amd as g

    m, n, k = 1024, 1024, 8192
    assert g.Plan(m, n, k, ROW_MAJOR, k, n, n).info["stream_k"] > 0
    info = g.Plan(m, n, k, ROW_MAJOR, k, n, n, epilogue=1).info
    assert info["stream_k"] > 0 and info["name"] == "dma_64x64x16_w2x2_s2"
    info = g.Plan(m, n, k, ROW_MAJOR, m, n, n, layout_a=COL_MAJOR, epilogue=1).info
    assert info["stream_k"] == 0 and info["name"] == "dma_64x64x16_w2x2_s2"


@pytest.mark.parametrize("layout_b", [ROW_MAJOR, COL_MAJOR])
def test_stream_k_tail_chosen(layout_b):
    """A plan with full waves of 256x128 tiles and a short last wave splits the
    last wave's tiles eight ways each; it matches the oracle
    (integer inputs bit for bit) and repeats bit for bit."""
    import dense_gemm_optimisation_fp32_amd as g

    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the choice was measured on a 256-CU MI355X")
    m, n, k = 7424, 13568, 4096    # 29 x 106 = 3074 tiles: 6 x 512 + 2
    print(f"\n[case] stream-K tail layout_b={layout_b} shape={(m, n, k)}", flush=True)
    A, B = random_operands(m, n, k, layout_b, "normal1", seed=98)
    C, info, outs = run_gemm(A, B, m, n, k, layout_b, repeat=2)
    assert info["name"] == "dma_256x128x16_w2x2_s3"
    assert info["stream_k"] == 16 and info["stream_k_tiles"] == 2
    assert np.array_equal(outs[0], outs[1])
    Cref, S = oracle.gemm_f64(A, B, m, n, k, layout_b)
    check_close(C, Cref, S, "stream-K tail")
    del Cref, S
    A, B = random_operands(m, n, k, layout_b, "int8range", seed=100)
    C, _ = run_gemm(A, B, m, n, k, layout_b)
    Cref, _ = oracle.gemm_f64(A, B, m, n, k, layout_b)
    assert np.array_equal(C.astype(np.float64), Cref)


@pytest.mark.parametrize("layout_b", [ROW_MAJOR, COL_MAJOR])
def test_stream_k_tail_64x128_ragged(layout_b, monkeypatch):
    """Without the column sliver, the ragged shape (boundary tiles on both
    edges, k = 16 * 128 + 1) runs 64x128 tiles with its last wave's 47 tiles
    split over one workgroup per CU; it matches the oracle (integer inputs
    bit for bit) and repeats bit for bit."""
    import dense_gemm_optimisation_fp32_amd as g

    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the choice was measured on a 256-CU MI355X")
    monkeypatch.setenv("GEMM_F32_SLIVER", "0")
    m, n, k = 5003, 4097, 2049    # 79 x 33 = 2607 tiles: 2 x 1280 + 47
    print(f"\n[case] 64x128 stream-K tail layout_b={layout_b} shape={(m, n, k)}", flush=True)
    A, B = random_operands(m, n, k, layout_b, "uniform", seed=101)
    C, info, outs = run_gemm(A, B, m, n, k, layout_b, repeat=2)
    assert info["name"] == "dma_64x128x16_w2x2_s2"
    assert info["stream_k"] == 256 and info["stream_k_tiles"] == 47
    assert np.array_equal(outs[0], outs[1])
    Cref, S = oracle.gemm_f64(A, B, m, n, k, layout_b)
    check_close(C, Cref, S, "64x128 stream-K tail")
    A, B = random_operands(m, n, k, layout_b, "int8range", seed=103)
    C, _ = run_gemm(A, B, m, n, k, layout_b)
    Cref, _ = oracle.gemm_f64(A, B, m, n, k, layout_b)
    assert np.array_equal(C.astype(np.float64), Cref)


# The whole-tile kernel stores NB adjacent C columns per instruction when B is
# row-major, there is no epilogue and N is a multiple of NB (the columns a lane
# holds per row: 2 for 64-column wavefront tiles, 4 for 128-column ones).
@pytest.mark.parametrize("variant_name,n,layout_b,width", [
    ("dma_256x128x16_w2x2_s3", 520, ROW_MAJOR, 2),
    ("dma_256x128x16_w2x2_s3", 130, ROW_MAJOR, 2),
    ("dma_256x128x16_w2x2_s3", 257, ROW_MAJOR, 1),
    ("dma_256x128x16_w2x2_s3", 520, COL_MAJOR, 1),
    ("dma_256x256x16_w2x2_s3", 520, ROW_MAJOR, 4),
    ("dma_256x256x16_w2x2_s3", 130, ROW_MAJOR, 1),
    ("dma_64x64x16_w2x2_s3", 520, ROW_MAJOR, 1),
    ("mfma_256x128x16_w2x2_32x32x2", 520, ROW_MAJOR, 1),
])
def test_c_store_width(variant_name, n, layout_b, width, monkeypatch):
    import dense_gemm_optimisation_fp32_amd as g

    v = next(i for i in variants() if g.gemm_f32_variant_info(i)["name"] == variant_name)
    m, k = 300, 77
    ldb = n if layout_b == ROW_MAJOR else k
    assert g.Plan(m, n, k, layout_b, k, ldb, n, v).info["c_store_width"] == width
    if layout_b == ROW_MAJOR and variant_name.startswith("dma_256x128"):
        # the epilogue kernels take the same width
        monkeypatch.setenv("GEMM_F32_VARIANT", str(v))
        info = g.Plan(m, n, k, layout_b, k, ldb, n, epilogue=1).info
        assert info["name"] == variant_name and info["c_store_width"] == width


# Operands whose byte extent is just under the 2^31 limit the plan accepts:
# the 32-bit buffer offsets of the last rows/columns are near 2^31 and must
# still address the right elements.  Integer inputs, so every sampled element
# is exact; the oracle sees only the sampled rows of A and columns of B (the
# sum of each element is the same sum over its row and column).
NEAR_LIMIT = {
    # name: (m, n, k, layout_a, layout_b), the operand near the limit
    # (enough 64x64 tiles, three per CU, for a data-parallel plan)
    "A": (32768, 192, 16383, ROW_MAJOR, ROW_MAJOR),
    "A_stream_k": (8192, 64, 65535, ROW_MAJOR, ROW_MAJOR),
    "A_col": (16383, 64, 32768, COL_MAJOR, ROW_MAJOR),
    "B_col": (192, 32768, 16383, ROW_MAJOR, COL_MAJOR),
    "B_few_rows": (16, 32768, 16383, ROW_MAJOR, ROW_MAJOR),
    "C": (32768, 16383, 64, ROW_MAJOR, ROW_MAJOR),
}


@pytest.mark.parametrize("name", list(NEAR_LIMIT))
def test_operand_extent_near_limit(name):
    import dense_gemm_optimisation_fp32_amd as g
    from workloads import a_storage_shape, b_storage_shape, int_storage

    m, n, k, la, lb = NEAR_LIMIT[name]
    print(f"\n[case] near-limit extent {name} shape={(m, n, k)} layout_a={la} layout_b={lb}", flush=True)
    A = int_storage(*a_storage_shape(m, k, la), seed=300)
    B = int_storage(*b_storage_shape(k, n, lb), seed=301)
    assert max(A.nbytes, B.nbytes, 4 * m * n) > (1 << 31) - (1 << 20)
    dev = torch.device("cuda", 0)
    dA, dB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
    dC = torch.full((m, n), float("nan"), dtype=torch.float32, device=dev)
    lda = k if la == ROW_MAJOR else m
    ldb = n if lb == ROW_MAJOR else k
    plan = g.Plan(m, n, k, lb, lda, ldb, n, layout_a=la)
    assert (plan.info["stream_k"] > 0) == (name == "A_stream_k")
    if la == ROW_MAJOR:
        plan.run(dA.data_ptr(), dB.data_ptr(), dC.data_ptr())
    else:
        plan.run_ex(dA.data_ptr(), dB.data_ptr(), dC.data_ptr())
    torch.cuda.synchronize()
    rows, cols = sample_indices(m, n, 64, seed=302)
    rows, cols = np.unique(rows), np.unique(cols)
    got = dC[torch.from_numpy(rows).to(dev)][:, torch.from_numpy(cols).to(dev)].cpu().numpy()
    # the sampled rows of A and columns of B as a small row-major problem
    a_sub = np.ascontiguousarray(A[rows, :] if la == ROW_MAJOR else A[:, rows].T)
    b_sub = np.ascontiguousarray(B[:, cols] if lb == ROW_MAJOR else B[cols, :].T)
    ref, _ = oracle.gemm_f64(a_sub, b_sub, rows.size, cols.size, k, ROW_MAJOR)
    assert np.array_equal(got.astype(np.float64), ref), f"{plan.info['name']} {name}"


# ---------------------------------------------------------------------------
# Full workload shapes, in the plan the benchmark times (gemm_f32_create).
# ---------------------------------------------------------------------------

FULL = ["sq256", "sq4096", "sq4096t", "ragged", "ffn", "skinny", "longk", "gemv_t", "decode4_t", "fewcol8"]


def record_ratio(what, ratio, oracle_s=None):
    """Print a full-size comparison's max error ratio and the oracle's time
    (and append them to the file named by GEMM_F32_PARITY_LOG, when set)."""
    import json
    import os
    line = json.dumps({"case": what, "max_error_ratio": ratio, "oracle_s": oracle_s,
                       "oracle_threads": oracle.num_threads()})
    print(f"\n[parity] {line}", flush=True)
    path = os.environ.get("GEMM_F32_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(line + "\n")


@pytest.mark.parametrize("name", FULL)
def test_workload_every_element_vs_oracle(name):
    """Every element of the full workload, in the plan the benchmark times,
    against the full oracle: |C - C_ref| <= 1e-5 * S + 1e-6."""
    w = WORKLOADS[name]
    print(f"\n[case] workload {name} random inputs, every element", flush=True)
    A, B = workload_operands(w)
    C, info = run_gemm(A, B, w.m, w.n, w.k, w.layout_b)
    assert np.isfinite(C).all()
    t0 = time.perf_counter()
    Cref, S = oracle.gemm_f64(A, B, w.m, w.n, w.k, w.layout_b)
    t_oracle = time.perf_counter() - t0
    ratio = check_close(C, Cref, S, f"{name} via {info['name']}")
    record_ratio(f"{name} {info['name']} random", ratio, round(t_oracle, 3))


@pytest.mark.parametrize("name", FULL)
def test_workload_integer_every_element_bitexact(name):
    """Integer-valued inputs at the full workload shape: every element equals
    the oracle exactly (every summation order is exact in float32)."""
    w = WORKLOADS[name]
    print(f"\n[case] workload {name} integer inputs, every element", flush=True)
    A, B = workload_operands(w, integer=True)
    C, info = run_gemm(A, B, w.m, w.n, w.k, w.layout_b)
    Cref, _ = oracle.gemm_f64(A, B, w.m, w.n, w.k, w.layout_b)
    bad = np.argwhere(C.astype(np.float64) != Cref)
    assert bad.size == 0, f"{len(bad)} elements differ, first {bad[:5].tolist()}"
    record_ratio(f"{name} {info['name']} integer (bit-exact)", 0.0)


@pytest.mark.parametrize("name", FULL)
def test_workload_closed_form_every_element(name):
    w = WORKLOADS[name]
    print(f"\n[case] workload {name} closed form", flush=True)
    A, B = mod_pattern_operands(w.m, w.n, w.k, w.layout_b)
    C, _ = run_gemm(A, B, w.m, w.n, w.k, w.layout_b)
    expect = closed_form(np.arange(w.m)[:, None], np.arange(w.n)[None, :], w.k)
    bad = np.argwhere(C != expect)
    assert bad.size == 0, f"{len(bad)} wrong elements, first {bad[:5].tolist()}"


def test_binding_matmul_matches_oracle_both_layouts():
    m, n, k = 250, 270, 190
    A, B = random_operands(m, n, k, ROW_MAJOR, "normal1", seed=43)
    import dense_gemm_optimisation_fp32_amd as g
    dA = torch.from_numpy(A).cuda()
    dB = torch.from_numpy(B).cuda()
    Cref, S = oracle.gemm_f64(A, B, m, n, k, ROW_MAJOR)
    check_close(g.matmul(dA, dB).cpu().numpy(), Cref, S, "matmul row-major B")
    dBt = dB.t().contiguous().t()                      # same values, column-major storage
    check_close(g.matmul(dA, dBt).cpu().numpy(), Cref, S, "matmul column-major B")


# Few columns (N <= 8): the matrix-vector-like path, chosen by the shape
# dispatch; k beyond one LDS chunk (2048) and with a tail, both B layouts.
FEWCOL_SHAPES = [(5003, 1, 2049), (300, 3, 77), (1000, 4, 4096), (777, 5, 2500), (4096, 8, 4096), (64, 2, 1),
                 (33, 7, 6000), (700, 3, 9000)]


@pytest.mark.parametrize("layout_b", [ROW_MAJOR, COL_MAJOR])
@pytest.mark.parametrize("shape", FEWCOL_SHAPES)
def test_few_columns_vs_oracle(shape, layout_b):
    import dense_gemm_optimisation_fp32_amd as g

    m, n, k = shape
    print(f"\n[case] few columns layout_b={layout_b} shape={shape}", flush=True)
    A, B = random_operands(m, n, k, layout_b, "normal1", seed=1700 + k)
    C, info, outs = run_gemm(A, B, m, n, k, layout_b, repeat=2)
    assert info["kind"] == g.GEMM_F32_KIND_FEWCOL and info["bn"] >= n
    assert np.array_equal(outs[0], outs[1])
    Cref, S = oracle.gemm_f64(A, B, m, n, k, layout_b)
    check_close(C, Cref, S, f"few columns {shape}")
    A, B = random_operands(m, n, k, layout_b, "int8range", seed=1800 + k)
    C, _ = run_gemm(A, B, m, n, k, layout_b)
    Cref, _ = oracle.gemm_f64(A, B, m, n, k, layout_b)
    assert np.array_equal(C.astype(np.float64), Cref)


# Shapes whose default plan has a one-column sliver, on 128 x 128 tiles in
# the tiles' launch (the first three) or as a second launch (the next four);
# then slivers of 2 columns (fused) and 4 columns (second launch).
SLIVER_SHAPES = [(5003, 4097, 2049), (8000, 1025, 520), (5003, 1537, 1024), (8000, 1537, 520),
                 (3001, 2049, 1500), (8000, 2049, 520), (4000, 1025, 1024), (5003, 4098, 2049),
                 (5003, 4100, 2049)]


@pytest.mark.parametrize("layout_b", [ROW_MAJOR, COL_MAJOR])
@pytest.mark.parametrize("shape", SLIVER_SHAPES)
def test_fused_sliver_matches_second_launch(shape, layout_b, monkeypatch):
    """A column sliver carried by the tiles' launch gives bitwise the C of
    the same plan with the sliver as a second launch (GEMM_F32_SLIVER_FUSE=0),
    and matches the oracle on every element (integer inputs bit for bit)."""
    m, n, k = shape
    print(f"\n[case] fused sliver {shape} layout_b={layout_b}", flush=True)
    A, B = random_operands(m, n, k, layout_b, "normal1", seed=2100 + m + k)
    C1, info1 = run_gemm(A, B, m, n, k, layout_b)
    monkeypatch.setenv("GEMM_F32_SLIVER_FUSE", "0")
    C0, info0 = run_gemm(A, B, m, n, k, layout_b)
    monkeypatch.delenv("GEMM_F32_SLIVER_FUSE")
    print(f"  {info1['name']} sliver {info1['sliver_cols']} fused {info1['sliver_fused']} "
          f"grid {info1['grid']} / {info0['grid']}", flush=True)
    assert info0["sliver_fused"] == 0 and info1["sliver_cols"] == info0["sliver_cols"]
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:   # the plans above were seen there
        assert info1["sliver_cols"] == (n - 4096 if m == 5003 and n > 4097 else 1)
        assert info1["sliver_fused"] == (shape in SLIVER_SHAPES[:3] + SLIVER_SHAPES[7:8])
    if info1["sliver_fused"]:
        rows = info1["threads"] // 64
        assert info1["grid"] == info0["grid"] + -(-m // rows) * info1["sliver_cols"]
    assert np.array_equal(C1, C0)
    Cref, S = oracle.gemm_f64(A, B, m, n, k, layout_b)
    check_close(C1, Cref, S, f"fused sliver {shape}")
    A, B = random_operands(m, n, k, layout_b, "int8range", seed=2200 + m + k)
    C, _ = run_gemm(A, B, m, n, k, layout_b)
    Cref, _ = oracle.gemm_f64(A, B, m, n, k, layout_b)
    assert np.array_equal(C.astype(np.float64), Cref)


def test_few_columns_padded_strides():
    """NaN padding of A's and B's rows never reaches C; C's padding is kept."""
    m, n, k = 700, 3, 2100
    for layout_b in (ROW_MAJOR, COL_MAJOR):
        lda, ldb, ldc = k + 3, (n if layout_b == ROW_MAJOR else k) + 5, n + 2
        A, B = random_operands(m, n, k, layout_b, "uniform", seed=1900, lda=lda, ldb=ldb)
        C, info = run_gemm(A, B, m, n, k, layout_b, lda, ldb, ldc, c_fill=-7.25)
        Cref, S = oracle.gemm_f64(A, B, m, n, k, layout_b, lda, ldb)
        check_close(C[:, :n], Cref, S, "few columns, padded")
        assert np.all(C[:-1, n:] == np.float32(-7.25))


@pytest.mark.parametrize("layout_b", [ROW_MAJOR, COL_MAJOR])
def test_column_sliver_plan(layout_b):
    """A shape whose last tile-column would hold one column runs it with
    the few-column method, in the tiles' launch: every element matches the
    oracle (integer inputs bit for bit) and repeats bit for bit."""
    import dense_gemm_optimisation_fp32_amd as g

    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the choice was measured on a 256-CU MI355X")
    m, n, k = 5003, 4097, 2049
    print(f"\n[case] column sliver layout_b={layout_b}", flush=True)
    A, B = random_operands(m, n, k, layout_b, "uniform", seed=2000)
    C, info, outs = run_gemm(A, B, m, n, k, layout_b, repeat=2)
    assert info["sliver_cols"] == 1 and info["sliver_variant"] == [
        v for v in range(g.gemm_f32_num_variants()) if g.gemm_f32_variant_info(v)["name"] == "fewcol_8x1_k2048"][0]
    # 1280 tiles of 128 x 128 in 768 slots: the sliver's 1251 one-row
    # workgroups ride in the idle slots of the second wave.
    assert info["sliver_fused"] == 1 and info["grid"] == info["tiles_m"] * info["tiles_n"] + (m + 3) // 4
    assert np.array_equal(outs[0], outs[1])
    Cref, S = oracle.gemm_f64(A, B, m, n, k, layout_b)
    check_close(C, Cref, S, "column sliver")
    A, B = random_operands(m, n, k, layout_b, "int8range", seed=2001)
    C, _ = run_gemm(A, B, m, n, k, layout_b)
    Cref, _ = oracle.gemm_f64(A, B, m, n, k, layout_b)
    assert np.array_equal(C.astype(np.float64), Cref)


# 17 to 32 rows: 32-row tiles where measured ahead (column-major B, or a B of
# 2^25 elements or more, N >= 1024), with the k split that fills the CUs.
ROWS32_CASES = [((32, 4096, 4096), COL_MAJOR, "skinny_32x64_w8_d4", 4),
                ((17, 14336, 4096), ROW_MAJOR, "skinny_32x64_w8_d4", 2),
                ((24, 4096, 14336), ROW_MAJOR, "skinny_32x64_w8_d4", 4),
                ((32, 4096, 4096), ROW_MAJOR, "skinny_16x64_w16_d4", 2),
                ((20, 512, 4096), COL_MAJOR, "skinny_16x64_w16_d4", None)]


@pytest.mark.parametrize("shape,layout_b,name,split", ROWS32_CASES)
def test_few_rows_32_row_tiles(shape, layout_b, name, split):
    """The dispatch's plan for 17 to 32 rows; every element against the
    oracle (integer inputs bit for bit) and runs repeat bit for bit."""
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the choices were measured on a 256-CU MI355X")
    m, n, k = shape
    print(f"\n[case] 32-row tiles {shape} layout_b={layout_b}", flush=True)
    A, B = random_operands(m, n, k, layout_b, "normal1", seed=2500 + m + n)
    C, info, outs = run_gemm(A, B, m, n, k, layout_b, repeat=2)
    assert info["name"] == name
    if split is not None:
        assert info["split_k"] == split and info["grid"] == info["tiles_m"] * info["tiles_n"] * split
    assert np.array_equal(outs[0], outs[1])
    Cref, S = oracle.gemm_f64(A, B, m, n, k, layout_b)
    check_close(C, Cref, S, f"{name} {shape}")
    A, B = random_operands(m, n, k, layout_b, "int8range", seed=2600 + m + n)
    C, _ = run_gemm(A, B, m, n, k, layout_b)
    Cref, _ = oracle.gemm_f64(A, B, m, n, k, layout_b)
    assert np.array_equal(C.astype(np.float64), Cref)


# Up to 16 rows: 32-column tiles with half the k splits of 64-column tiles
# where A is light (up to 4 rows, k per split up to 1024, or column-major B
# up to 8 rows), 64-column tiles otherwise.  n = 3000 and 2050 end in a
# ragged 32-column tile; k = 1999 and 777 end in a partial 16-k group.
COLS32_CASES = [((16, 2048, 2048), ROW_MAJOR, "skinny_16x32_w16_d4", 4),
                ((2, 4096, 4096), COL_MAJOR, "skinny_16x32_w16_d4", 2),
                ((8, 4096, 4096), COL_MAJOR, "skinny_16x32_w16_d4", 2),
                ((3, 8192, 4096), ROW_MAJOR, "skinny_16x32_w16_d4", 1),
                ((13, 3000, 1999), COL_MAJOR, "skinny_16x32_w16_d4", 2),
                ((5, 2050, 777), ROW_MAJOR, "skinny_16x32_w16_d4", 3),
                ((8, 4096, 4096), ROW_MAJOR, "skinny_16x64_w16_d4", 4),
                ((16, 4096, 4096), ROW_MAJOR, "skinny_16x64_w16_d4", 4),
                ((16, 8192, 4096), COL_MAJOR, "skinny_16x64_w16_d4", 2),
                ((4, 1024, 4096), ROW_MAJOR, "skinny_16x64_w16_d4", 16)]


@pytest.mark.parametrize("shape,layout_b,name,split", COLS32_CASES)
def test_few_rows_32_column_tiles(shape, layout_b, name, split):
    """The dispatch's tile width for up to 16 rows; every element against
    the oracle (integer inputs bit for bit) and runs repeat bit for bit."""
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the choices were measured on a 256-CU MI355X")
    m, n, k = shape
    print(f"\n[case] 32-column tiles {shape} layout_b={layout_b}", flush=True)
    A, B = random_operands(m, n, k, layout_b, "normal1", seed=2700 + m + n)
    C, info, outs = run_gemm(A, B, m, n, k, layout_b, repeat=2)
    assert info["name"] == name
    assert info["split_k"] == split and info["grid"] == info["tiles_m"] * info["tiles_n"] * split
    assert np.array_equal(outs[0], outs[1])
    Cref, S = oracle.gemm_f64(A, B, m, n, k, layout_b)
    check_close(C, Cref, S, f"{name} {shape}")
    A, B = random_operands(m, n, k, layout_b, "int8range", seed=2800 + m + n)
    C, _ = run_gemm(A, B, m, n, k, layout_b)
    Cref, _ = oracle.gemm_f64(A, B, m, n, k, layout_b)
    assert np.array_equal(C.astype(np.float64), Cref)


# Up to eight rows of C with column-major B: the transposed product
# C^T = B^T A^T on a few-column kernel (one row: k <= 16384 and N >= 1024 or
# N * K <= 2^22; 2 to 4 rows: N >= 6144 and 2048 <= K <= 5120, or N >= 4096
# and 10240 <= K <= 16384; 5 to 8 rows:
# 128 < N / 64 < 256 and 2048 <= K <= 4096); every other
# case keeps the few-row plan.  Padded leading dimensions (lda, ldb, ldc past
# the matrix), ragged N and K, and 3 rows on the four-column kernel included.
TRANSPOSED_CASES = [((1, 4096, 4096), COL_MAJOR, 0, "fewcol_8x1_k2048_w8"),
                    ((1, 2050, 2049), COL_MAJOR, 0, "fewcol_8x1_k2048_w8"),
                    ((1, 3001, 5003), COL_MAJOR, 7, "fewcol_8x1_k2048_w8"),
                    ((1, 14336, 4096), COL_MAJOR, 0, "fewcol_8x1_k2048_w8"),
                    ((1, 300, 1000), COL_MAJOR, 3, "fewcol_8x1_k2048_w8"),
                    ((3, 8192, 3000), COL_MAJOR, 0, "fewcol_8x4_k1024"),
                    ((4, 6144, 4096), COL_MAJOR, 5, "fewcol_8x4_k1024"),
                    ((2, 11009, 2049), COL_MAJOR, 0, "fewcol_8x4_k1024"),
                    ((1, 600, 20000), COL_MAJOR, 0, None),
                    ((1, 4096, 4096), ROW_MAJOR, 0, None),
                    ((2, 4096, 4096), COL_MAJOR, 0, None),
                    ((4, 6144, 8192), COL_MAJOR, 0, None),
                    ((5, 8192, 4096), COL_MAJOR, 0, None),
                    ((3, 4096, 11008), COL_MAJOR, 0, "fewcol_8x4_k1024"),
                    ((5, 11008, 4096), COL_MAJOR, 0, "fewcol_8x8_k1024_w8"),
                    ((8, 14336, 2049), COL_MAJOR, 5, "fewcol_8x8_k1024_w8"),
                    ((8, 11008, 8192), COL_MAJOR, 0, None),
                    ((9, 11008, 4096), COL_MAJOR, 0, None)]


@pytest.mark.parametrize("shape,layout_b,pad,name", TRANSPOSED_CASES)
def test_few_rows_transposed_product(shape, layout_b, pad, name):
    """The dispatch's plan for up to five rows; every element against the
    oracle (integer inputs bit for bit), runs repeat bit for bit, and the
    padding of C's rows is never written."""
    m, n, k = shape
    print(f"\n[case] transposed product {shape} layout_b={layout_b} pad={pad}", flush=True)
    lda, ldb, ldc = k + pad, (n if layout_b == ROW_MAJOR else k) + pad, n + pad
    for dist, seed in (("normal1", 2900 + n), ("int8range", 2950 + n)):
        A, B = random_operands(m, n, k, layout_b, dist, seed=seed, lda=lda, ldb=ldb)
        C, info, outs = run_gemm(A, B, m, n, k, layout_b, lda, ldb, ldc, c_fill=-7.25, repeat=2)
        assert info["transposed"] == (name is not None)
        if name is not None:
            assert info["name"] == name and info["split_k"] == 1
        assert np.array_equal(outs[0], outs[1])
        assert np.all(C[:, n:] == np.float32(-7.25)), "C row padding was written"
        Cref, S = oracle.gemm_f64(A, B, m, n, k, layout_b, lda, ldb)
        if dist == "int8range":
            assert np.array_equal(C[:, :n].astype(np.float64), Cref)
        else:
            check_close(C[:, :n], Cref, S, f"transposed product {shape}")


def test_one_row_transposed_product_switch(monkeypatch):
    """GEMM_F32_TRANSPOSE=0 keeps the few-row plan, and both plans agree
    with the oracle on the same inputs."""
    import dense_gemm_optimisation_fp32_amd as g
    m, n, k = 1, 4096, 4096
    A, B = random_operands(m, n, k, COL_MAJOR, "normal1", seed=2990)
    Cref, S = oracle.gemm_f64(A, B, m, n, k, COL_MAJOR)
    C1, info1 = run_gemm(A, B, m, n, k, COL_MAJOR)
    monkeypatch.setenv("GEMM_F32_TRANSPOSE", "0")
    C0, info0 = run_gemm(A, B, m, n, k, COL_MAJOR)
    assert info1["transposed"] == 1 and info0["transposed"] == 0 and info0["kind"] == g.GEMM_F32_KIND_SKINNY
    check_close(C1, Cref, S, "transposed")
    check_close(C0, Cref, S, "few-row")


# Seeded random shapes through the default dispatch (every path the shape
# classes select: few rows, few columns, few tiles with stream-K, column
# slivers, the whole-tile candidates), both B layouts, every element.
def _random_shapes(count, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        kind = rng.integers(0, 4)
        if kind == 0:      # few rows or few columns
            m, n = (int(rng.integers(1, 33)), int(rng.integers(1, 2049))) if rng.random() < 0.5 else \
                   (int(rng.integers(33, 3000)), int(rng.integers(1, 9)))
        elif kind == 1:    # a few tiles
            m, n = int(rng.integers(33, 700)), int(rng.integers(9, 700))
        else:              # many tiles, ragged edges
            m, n = int(rng.integers(700, 2600)), int(rng.integers(700, 2600))
        k = int(rng.choice([int(rng.integers(1, 300)), int(rng.integers(300, 2200)), int(rng.integers(2048, 4500))]))
        out.append((m, n, k))
    return out


def _random_small_shapes(count, seed):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 900)), int(rng.integers(1, 900)), int(rng.integers(1, 5000))) for _ in range(count)]


@pytest.mark.parametrize("layout_b", [ROW_MAJOR, COL_MAJOR])
@pytest.mark.parametrize("shape", _random_small_shapes(40, 7))
def test_random_small_shapes_default_plan(shape, layout_b):
    """Small seeded random shapes (ragged in every dimension) through the
    default dispatch: few-row, few-column, few-tile and tiled plans alike
    match the oracle on every element, integer inputs bit for bit."""
    m, n, k = shape
    print(f"\n[case] random small shape {shape} layout_b={layout_b}", flush=True)
    A, B = random_operands(m, n, k, layout_b, "normal1", seed=5000 + m + n + k)
    C, info = run_gemm(A, B, m, n, k, layout_b)
    Cref, S = oracle.gemm_f64(A, B, m, n, k, layout_b)
    check_close(C, Cref, S, f"random small {shape} via {info['name']} split {info['split_k']}")
    A, B = random_operands(m, n, k, layout_b, "int8range", seed=6000 + m + n + k)
    C, _ = run_gemm(A, B, m, n, k, layout_b)
    Cref, _ = oracle.gemm_f64(A, B, m, n, k, layout_b)
    assert np.array_equal(C.astype(np.float64), Cref)


@pytest.mark.parametrize("layout_b", [ROW_MAJOR, COL_MAJOR])
@pytest.mark.parametrize("shape", _random_shapes(16, 2024))
def test_random_shapes_default_plan(shape, layout_b):
    m, n, k = shape
    print(f"\n[case] random shape {shape} layout_b={layout_b}", flush=True)
    A, B = random_operands(m, n, k, layout_b, "normal1", seed=3000 + m + n + k)
    C, info = run_gemm(A, B, m, n, k, layout_b)
    Cref, S = oracle.gemm_f64(A, B, m, n, k, layout_b)
    check_close(C, Cref, S, f"random {shape} via {info['name']} (sliver {info['sliver_cols']})")
    A, B = random_operands(m, n, k, layout_b, "int8range", seed=4000 + m + n + k)
    C, _ = run_gemm(A, B, m, n, k, layout_b)
    Cref, _ = oracle.gemm_f64(A, B, m, n, k, layout_b)
    assert np.array_equal(C.astype(np.float64), Cref)

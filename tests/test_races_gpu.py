"""Checks for missing waits and barriers, and for the bounded waits of the
split plans, through the C ABI.

* The k order of every element is fixed by the tile shape (BM, BN, BK and
  the wavefront grid), not by how many LDS stages the ring has or whether
  the copies go through registers or straight to LDS.  So every kernel of
  one tile shape must give bitwise the same C; a missing wait or barrier
  (a read of a stage before its copy lands, or a copy over a stage still
  being read) shows up as a difference ("GEMM 性能优化", 台阶 6: the double
  buffer; "GPU 算子优化中的数据复用", section 10.1: barriers).
* With LDS filled with NaN before the first copy (GEMM_F32_POISON_LDS), a
  read of LDS ahead of the copy that fills it puts NaN into C.
* The split plans' waits for partial sums are bounded: forced to give up
  (GEMM_F32_TEST_LOST_WORDS), they write NaN for the split tiles, every
  kernel still ends, and gemm_f32_plan_check reports it.
* Plans with a workspace used from two streams at once (the binding gives
  each stream its own plan).
"""
import numpy as np
import pytest
import torch

import dense_gemm_optimisation_fp32_amd as g
import oracle
from tests.gpu_helpers import run_gemm, variants
from workloads import COL_MAJOR, ROW_MAJOR, random_operands

pytestmark = pytest.mark.gpu

REL, ABS = 1e-5, 1e-6


def by_name():
    return {g.gemm_f32_variant_info(v)["name"]: v for v in variants()}


# Kernels that share a tile shape, hence the k order of every element.
FAMILIES = {
    "256x256x16": ["mfma_256x256x16_w2x2_32x32x2", "dma_256x256x16_w2x2_s2", "dma_256x256x16_w2x2_s3",
                   "dma_256x256x16_w2x2_s4", "dma_256x256x16_w2x4_s4", "dma_256x256x16_w4x2_s4",
                   "dma_256x256x16_w4x2_s2", "dma_256x256x16_w4x4_s4"],
    "256x128x16": ["mfma_256x128x16_w2x2_32x32x2", "dma_256x128x16_w2x2_s3"],
    "128x128x16": ["mfma_128x128x16_w2x2_32x32x2", "dma_128x128x16_w2x2_s3"],
    "128x128x32": ["mfma_128x128x32_w2x2_32x32x2", "dma_128x128x32_w2x2_s3"],
    "64x64x16": ["dma_64x64x16_w2x2_s2", "dma_64x64x16_w2x2_s3"],
    "128x64x16": ["dma_128x64x16_w2x2_s2", "dma_128x64x16_w2x2_s3"],
    "64x128x16": ["dma_64x128x16_w2x2_s2", "dma_64x128x16_w2x2_s3"],
}
# Several slabs with a k tail, boundary tiles on both edges.
RACE_SHAPES = [(513, 257, 1000), (300, 520, 77), (700, 900, 129)]


@pytest.mark.parametrize("family", list(FAMILIES))
@pytest.mark.parametrize("layout_b", [ROW_MAJOR, COL_MAJOR])
@pytest.mark.parametrize("shape", RACE_SHAPES)
def test_stage_counts_bitwise_identical(family, layout_b, shape):
    names = by_name()
    m, n, k = shape
    A, B = random_operands(m, n, k, layout_b, "normal1", seed=1100 + m)
    outs = []
    for vname in FAMILIES[family]:
        print(f"\n[case] stage family {family} kernel {vname} layout_b={layout_b} shape={shape}", flush=True)
        C, info = run_gemm(A, B, m, n, k, layout_b, variant=names[vname])
        outs.append((vname, C))
    Cref, S = oracle.gemm_f64(A, B, m, n, k, layout_b)
    ok, ratio = oracle.within_tolerance(outs[0][1], Cref, S, REL, ABS)
    assert ok, f"{outs[0][0]}: max error ratio {ratio:.3g}"
    for vname, C in outs[1:]:
        diff = np.argwhere(C != outs[0][1])
        assert diff.size == 0, f"{vname} differs from {outs[0][0]} at {len(diff)} elements, first {diff[:4].tolist()}"


POISON_SHAPES = [(513, 257, 1000), (300, 520, 77), (64, 64, 16), (129, 131, 33)]


@pytest.mark.parametrize("layout_b", [ROW_MAJOR, COL_MAJOR])
def test_poisoned_lds_never_reaches_c(layout_b, monkeypatch):
    """Every tiled kernel (register-staged and direct-to-LDS) with LDS full of
    NaN before its first copy: C is finite and matches the oracle."""
    monkeypatch.setenv("GEMM_F32_POISON_LDS", "1")
    for v in variants():
        info = g.gemm_f32_variant_info(v)
        if info["kind"] != g.GEMM_F32_KIND_MFMA:
            continue
        for shape in POISON_SHAPES:
            m, n, k = shape
            print(f"\n[case] poisoned LDS {info['name']} layout_b={layout_b} shape={shape}", flush=True)
            A, B = random_operands(m, n, k, layout_b, "uniform", seed=1200 + k)
            C, _ = run_gemm(A, B, m, n, k, layout_b, variant=v)
            assert np.isfinite(C).all(), f"{info['name']} {shape}: NaN from LDS reached C"
            Cref, S = oracle.gemm_f64(A, B, m, n, k, layout_b)
            ok, ratio = oracle.within_tolerance(C, Cref, S, REL, ABS)
            assert ok, f"{info['name']} {shape}: max error ratio {ratio:.3g}"


@pytest.mark.parametrize("layout_b", [ROW_MAJOR, COL_MAJOR])
@pytest.mark.parametrize("wgs", [3, 16])
def test_poisoned_lds_stream_k(layout_b, wgs, monkeypatch):
    """Stream-K ranges start and end at arbitrary slabs, so their rings start
    cold mid-tile: with poisoned LDS the result is still exact to tolerance."""
    monkeypatch.setenv("GEMM_F32_POISON_LDS", "1")
    monkeypatch.setenv("GEMM_F32_SK_WGS", str(wgs))
    names = by_name()
    m, n, k = 300, 520, 1000
    for vname in ["dma_64x64x16_w2x2_s2", "dma_64x128x16_w2x2_s2", "dma_256x128x16_w2x2_s3",
                  "dma_256x256x16_w2x2_s4", "dma_256x256x16_w4x2_s4"]:
        print(f"\n[case] poisoned LDS stream-K {vname} wgs={wgs} layout_b={layout_b}", flush=True)
        A, B = random_operands(m, n, k, layout_b, "uniform", seed=1300 + wgs)
        C, info = run_gemm(A, B, m, n, k, layout_b, variant=names[vname])
        assert info["stream_k"] == wgs
        assert np.isfinite(C).all()
        Cref, S = oracle.gemm_f64(A, B, m, n, k, layout_b)
        ok, ratio = oracle.within_tolerance(C, Cref, S, REL, ABS)
        assert ok, f"{vname}: max error ratio {ratio:.3g}"


def _run_plan(plan, A, B, m, n):
    dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    C = torch.full((m, n), -3.0, device="cuda")
    g.gemm_f32_run(plan, dA.data_ptr(), dB.data_ptr(), C.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return C.cpu().numpy()


@pytest.mark.parametrize("kind", ["stream_k", "split_k"])
def test_lost_partial_sums_are_reported(kind, monkeypatch):
    """Readers forced to wait for a tag no writer uses give up after a small
    budget: the split tiles read NaN, the whole tiles stay exact, every
    kernel ends, and gemm_f32_plan_check reports it once."""
    names = by_name()
    if kind == "stream_k":
        m, n, k = 300, 520, 1000
        variant = names["dma_64x64x16_w2x2_s2"]
        monkeypatch.setenv("GEMM_F32_SK_WGS", "7")
        monkeypatch.setenv("GEMM_F32_SK_TILES", "5")   # 5 split tiles, the other 35 whole
    else:
        m, n, k = 16, 300, 2000
        variant = None
        monkeypatch.setenv("GEMM_F32_SPLIT_K", "4")
    A, B = random_operands(m, n, k, ROW_MAJOR, "normal1", seed=1400)
    Cref, S = oracle.gemm_f64(A, B, m, n, k, ROW_MAJOR)

    # An ordinary plan first: nothing lost.
    plan = (g.gemm_f32_create(m, n, k, ROW_MAJOR, k, n, n) if variant is None
            else g.gemm_f32_create_variant(variant, m, n, k, ROW_MAJOR, k, n, n))
    try:
        C = _run_plan(plan, A, B, m, n)
        ok, ratio = oracle.within_tolerance(C, Cref, S, REL, ABS)
        assert ok, ratio
        assert g.gemm_f32_plan_check(plan) is False
    finally:
        g.gemm_f32_destroy(plan)

    monkeypatch.setenv("GEMM_F32_TEST_LOST_WORDS", "1")
    monkeypatch.setenv("GEMM_F32_WAIT_BUDGET", "4")
    plan = (g.gemm_f32_create(m, n, k, ROW_MAJOR, k, n, n) if variant is None
            else g.gemm_f32_create_variant(variant, m, n, k, ROW_MAJOR, k, n, n))
    try:
        info = g.gemm_f32_describe(plan)
        print(f"\n[case] lost words {kind}: {info['name']} split_k={info['split_k']} "
              f"stream_k={info['stream_k']} over {info['stream_k_tiles']}", flush=True)
        C = _run_plan(plan, A, B, m, n)
        nan = np.isnan(C)
        assert nan.any(), "no split tile was written as NaN"
        if kind == "stream_k":
            # the whole tiles are untouched by the waits
            ok, ratio = oracle.within_tolerance(C[~nan], Cref[~nan], S[~nan], REL, ABS)
            assert ok, ratio
            assert nan.sum() <= 5 * 64 * 64
        assert g.gemm_f32_plan_check(plan) is True
        assert g.gemm_f32_plan_check(plan) is False      # the record was cleared
    finally:
        g.gemm_f32_destroy(plan)


@pytest.mark.parametrize("shape", [(16, 300, 2000), (256, 256, 4096)])
def test_workspace_plans_on_two_streams(shape):
    """The same workspace-plan shape run on two streams at once, with
    different inputs: each stream gets its own plan, and both results match
    the oracle."""
    m, n, k = shape
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    sets = [random_operands(m, n, k, ROW_MAJOR, "normal1", seed=1500 + i) for i in range(2)]
    dev = [(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()) for A, B in sets]
    torch.cuda.synchronize()
    outs = [[], []]
    for it in range(4):
        for i, s in enumerate((s1, s2)):
            with torch.cuda.stream(s):
                outs[i].append(g.matmul(dev[i][0], dev[i][1]))
    torch.cuda.synchronize()
    p1 = g.get_plan(m, n, k, ROW_MAJOR, k, n, n, None, 0, stream=s1.cuda_stream)
    p2 = g.get_plan(m, n, k, ROW_MAJOR, k, n, n, None, 0, stream=s2.cuda_stream)
    assert p1.has_workspace and p1.handle != p2.handle
    for i in range(2):
        Cref, S = oracle.gemm_f64(sets[i][0], sets[i][1], m, n, k, ROW_MAJOR)
        for C in outs[i]:
            ok, ratio = oracle.within_tolerance(C.cpu().numpy(), Cref, S, REL, ABS)
            assert ok, f"stream {i}: max error ratio {ratio:.3g}"

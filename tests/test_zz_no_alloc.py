"""gemm_f32_run_noalloc, the entry point that allocates nothing, through the C
ABI: the same result as gemm_f32_create + gemm_f32_run on the same inputs
(the same plan and kernels, so bit for bit, and within the oracle's
tolerance), on two calls in a row where the second is smaller, for plans
whose partial sums live in the static scratch area (the few-row split-k
path and stream-K) and a plain tiled plan; and the size limit of the
scratch area is rejected with its own status before anything runs.  Where
the plan entry point takes stream-K over 128x128 tiles (column-major B, two
to two and a half tiles per CU), whose partial sums outgrow the scratch
area, the allocation-free call runs the plan the dispatch takes without that
rule: the two then agree within the tolerance."""
import numpy as np
import pytest
import torch

import dense_gemm_optimisation_fp32_amd as g
import oracle
from workloads import COL_MAJOR, ROW_MAJOR, random_operands

pytestmark = pytest.mark.gpu

REL, ABS = 1e-5, 1e-6


def _both(m, n, k, layout_b, seed):
    """(C from gemm_f32_run_noalloc, C from a plan, plan info)."""
    A, B = random_operands(m, n, k, layout_b, "normal1", seed=seed)
    ldb = n if layout_b == ROW_MAJOR else k
    dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    stream = torch.cuda.current_stream().cuda_stream
    c_static = torch.full((m, n), float("nan"), device="cuda")
    g.gemm_f32_run_noalloc(m, n, k, layout_b, k, ldb, n, dA.data_ptr(), dB.data_ptr(), c_static.data_ptr(),
                           stream)
    torch.cuda.synchronize()
    plan = g.gemm_f32_create(m, n, k, layout_b, k, ldb, n)
    try:
        info = g.gemm_f32_describe(plan)
        c_plan = torch.full((m, n), float("nan"), device="cuda")
        g.gemm_f32_run(plan, dA.data_ptr(), dB.data_ptr(), c_plan.data_ptr(), stream)
        torch.cuda.synchronize()
    finally:
        g.gemm_f32_destroy(plan)
    Cref, S = oracle.gemm_f64(A, B, m, n, k, layout_b)
    return c_static.cpu().numpy(), c_plan.cpu().numpy(), info, Cref, S


@pytest.mark.parametrize("layout_b", [ROW_MAJOR, COL_MAJOR])
@pytest.mark.parametrize("first,second,kind", [
    ((16, 4096, 4096), (16, 300, 2000), "split_k"),       # few rows: split-k partial sums
    ((64, 256, 4096), (64, 200, 3000), "split_k"),        # few tiles on 16x16 tiles, k split 4 ways
    ((32, 4096, 4096), (24, 2048, 3000), "split_k"),      # 17-32 rows (32-row tiles with column-major B)
    ((1024, 1024, 8192), (1200, 700, 3000), "stream_k"),  # few tiles, long k: stream-K
    ((513, 257, 1000), (300, 520, 77), "tiles"),          # whole tiles, no scratch
    ((1, 4096, 4096), (1, 2050, 2049), "one_row"),        # column-major B: the transposed product
    ((2000, 5000, 2049), (1536, 5632, 2100), "sub_wave"),  # column-major B: stream-K over 128x128 tiles
])
def test_noalloc_matches_the_plan_entry_point(first, second, kind, layout_b):
    for shape, seed in ((first, 1600), (second, 1601)):
        m, n, k = shape
        print(f"\n[case] noalloc {kind} layout_b={layout_b} shape={shape}", flush=True)
        c_static, c_plan, info, Cref, S = _both(m, n, k, layout_b, seed)
        if kind == "split_k":
            assert info["split_k"] > 1
        elif kind == "stream_k":
            assert info["stream_k"] > 0
        elif kind == "one_row":
            assert info["transposed"] == (1 if layout_b == COL_MAJOR else 0)
        ok, ratio = oracle.within_tolerance(c_static, Cref, S, REL, ABS)
        assert ok, f"{shape}: max error ratio {ratio:.3g}"
        if kind == "sub_wave" and layout_b == COL_MAJOR:
            if torch.cuda.get_device_properties(0).multi_processor_count == 256:   # (rule measured there)
                assert info["name"] == "dma_128x128x16_w2x2_s3" and info["stream_k"] == 768
            ok, ratio = oracle.within_tolerance(c_plan, Cref, S, REL, ABS)
            assert ok, f"{shape}: gemm_f32_run max error ratio {ratio:.3g}"
            continue
        assert np.array_equal(c_static, c_plan), f"{shape}: differs from gemm_f32_run"


def test_noalloc_rejects_plans_beyond_the_scratch_area(monkeypatch):
    """A forced stream-K plan whose partial sums need more than the 64 MiB
    scratch area is rejected with GEMM_F32_ERR_SCRATCH_TOO_SMALL and C is
    left untouched."""
    m = n = k = 2048
    monkeypatch.setenv("GEMM_F32_VARIANT", "12")          # 256x128 tiles
    monkeypatch.setenv("GEMM_F32_SK_WGS", "512")           # 2 * 512 * 256 * 128 * 8 B = 256 MiB
    assert g.gemm_f32_variant_info(12)["name"] == "dma_256x128x16_w2x2_s3"
    dA = torch.zeros(m * k, device="cuda")
    dC = torch.full((m * n,), 5.0, device="cuda")
    with pytest.raises(g.GemmF32Error) as err:
        g.gemm_f32_run_noalloc(m, n, k, ROW_MAJOR, k, n, n, dA.data_ptr(), dA.data_ptr(), dC.data_ptr(),
                               torch.cuda.current_stream().cuda_stream)
    assert err.value.status == g.GEMM_F32_ERR_SCRATCH_TOO_SMALL
    torch.cuda.synchronize()
    assert bool((dC == 5.0).all())

"""Plans replayed from a captured HIP graph.

A captured launch replays the arguments it was recorded with.  Split plans
(few-row split-k, stream-K) tag each run's partial sums with an epoch that
the device keeps in the plan's workspace (or in the scratch area of the
allocation-free entry point) and advances at the end of every run, so each
replay is tagged afresh and never takes the previous replay's partial sums
for its own.  Every replay here runs on new operands, copied into the
captured buffers between replays, and must equal an eager run of the same
product on another plan bit for bit.
"""
import numpy as np
import pytest
import torch

import dense_gemm_optimisation_fp32_amd as g
import oracle
from workloads import COL_MAJOR, ROW_MAJOR, random_operands

pytestmark = pytest.mark.gpu

CASES = [
    ((16, 4096, 4096), ROW_MAJOR, "split_k"),          # few rows: 4 k-splits per 16x64 tile
    ((64, 256, 4096), COL_MAJOR, "split_k"),           # few tiles: 16x16 tiles, k split 4 ways
    ((24, 4096, 4096), COL_MAJOR, "split_k"),          # 32-row tiles, k split 4 ways
    ((4, 4096, 2048), COL_MAJOR, "split_k"),           # 16x32 tiles, k split 2 ways
    ((1, 4096, 2048), COL_MAJOR, "tiles"),             # one row: the transposed one-column product
    ((4, 8192, 3000), COL_MAJOR, "tiles"),             # four rows: the transposed four-column product
    ((1024, 1024, 8192), ROW_MAJOR, "stream_k"),       # few tiles, long k: stream-K over all tiles
    ((2304, 9216, 4096), ROW_MAJOR, "stream_k_tail"),  # the partial last wave split by stream-K
    ((5003, 4097, 2049), ROW_MAJOR, "sliver"),         # tiles and a one-column sliver
    ((300, 520, 77), ROW_MAJOR, "tiles"),              # whole tiles only
]


def _device_operands(m, n, k, layout_b, seed):
    A, B = random_operands(m, n, k, layout_b, "normal1", seed=seed)
    return torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()


def _eager(m, n, k, layout_b, dA, dB):
    """C from a plan of its own, run eagerly."""
    ldb = n if layout_b == ROW_MAJOR else k
    ref = g.Plan(m, n, k, layout_b, k, ldb, n)
    C = torch.full((m, n), float("nan"), device="cuda")
    ref.run(dA.data_ptr(), dB.data_ptr(), C.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return C.cpu().numpy()


def _check_kind(info, kind):
    if kind == "split_k":
        assert info["split_k"] > 1
    elif kind == "stream_k":
        assert info["stream_k"] > 0 and info["stream_k_tiles"] == info["tiles_m"] * info["tiles_n"]
    elif kind == "stream_k_tail":
        assert 0 < info["stream_k_tiles"] < info["tiles_m"] * info["tiles_n"]
    elif kind == "sliver":
        assert info["sliver_cols"] > 0
    else:
        assert info["split_k"] == 1 and info["stream_k"] == 0


@pytest.mark.parametrize("shape,layout_b,kind", CASES)
def test_plan_replayed_from_a_graph(shape, layout_b, kind):
    m, n, k = shape
    ldb = n if layout_b == ROW_MAJOR else k
    print(f"\n[case] graph replay {kind} shape={shape} layout_b={layout_b}", flush=True)
    plan = g.Plan(m, n, k, layout_b, k, ldb, n)
    _check_kind(plan.info, kind)
    dA, dB = _device_operands(m, n, k, layout_b, seed=2100)
    C = torch.full((m, n), float("nan"), device="cuda")
    # One eager run first, then the capture (plans and buffers exist before it).
    plan.run(dA.data_ptr(), dB.data_ptr(), C.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan.run(dA.data_ptr(), dB.data_ptr(), C.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    previous = None
    for rep in range(3):
        nA, nB = _device_operands(m, n, k, layout_b, seed=2200 + rep)
        dA.copy_(nA)
        dB.copy_(nB)
        C.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = C.cpu().numpy()
        want = _eager(m, n, k, layout_b, nA, nB)
        assert np.isfinite(got).all(), f"replay {rep}: NaN in C"
        assert np.array_equal(got, want), f"replay {rep} differs from the eager run"
        if previous is not None:
            assert not np.array_equal(got, previous)     # the replay computed the new product
        previous = got
    assert g.gemm_f32_plan_check(plan.handle) is False  # no wait gave up
    if m * n * k <= 1 << 27:
        A = dA.cpu().numpy()
        B = dB.cpu().numpy()
        Cref, S = oracle.gemm_f64(A, B, m, n, k, layout_b)
        ok, ratio = oracle.within_tolerance(previous, Cref, S, 1e-5, 1e-6)
        assert ok, ratio
    del graph


@pytest.mark.parametrize("shape,layout_b,kind", [c for c in CASES if c[2] in ("split_k", "stream_k", "sliver")])
def test_noalloc_replayed_from_a_graph(shape, layout_b, kind):
    m, n, k = shape
    ldb = n if layout_b == ROW_MAJOR else k
    print(f"\n[case] graph replay noalloc {kind} shape={shape} layout_b={layout_b}", flush=True)
    dA, dB = _device_operands(m, n, k, layout_b, seed=2300)
    C = torch.full((m, n), float("nan"), device="cuda")

    def call():
        g.gemm_f32_run_noalloc(m, n, k, layout_b, k, ldb, n, dA.data_ptr(), dB.data_ptr(), C.data_ptr(),
                               torch.cuda.current_stream().cuda_stream)

    call()                      # the first call on the device finds the scratch area, outside capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        nA, nB = _device_operands(m, n, k, layout_b, seed=2400 + rep)
        dA.copy_(nA)
        dB.copy_(nB)
        C.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = C.cpu().numpy()
        want = _eager(m, n, k, layout_b, nA, nB)
        assert np.isfinite(got).all(), f"replay {rep}: NaN in C"
        assert np.array_equal(got, want), f"replay {rep} differs from the eager run"
        # an eager allocation-free call between replays takes the next tag
        call()
        torch.cuda.synchronize()
        assert np.array_equal(C.cpu().numpy(), want)
    del graph


# Epilogue plans whose kernels split tiles along k: stream-K over 64x64 tiles
# and the few-row kernel's k splits, each with bias + GELU (beta = 0, so every
# replay computes the same function of the new inputs).
EPI_CASES = [((1024, 1024, 8192), ROW_MAJOR, "stream_k"),
             ((16, 4096, 4096), COL_MAJOR, "split_k"),
             ((4, 8192, 3000), COL_MAJOR, "transposed")]


@pytest.mark.parametrize("shape,layout_b,kind", EPI_CASES)
def test_epilogue_plan_replayed_from_a_graph(shape, layout_b, kind):
    m, n, k = shape
    ldb = n if layout_b == ROW_MAJOR else k
    print(f"\n[case] graph replay epilogue {kind} shape={shape} layout_b={layout_b}", flush=True)
    plan = g.Plan(m, n, k, layout_b, k, ldb, n, epilogue=1)
    info = plan.info
    if kind == "stream_k":
        assert info["stream_k"] > 1
    elif kind == "split_k":
        assert info["split_k"] > 1
    else:
        assert info["transposed"] == 1
    stream = lambda: torch.cuda.current_stream().cuda_stream
    dA, dB = _device_operands(m, n, k, layout_b, seed=2500)
    bias = torch.linspace(-1.0, 1.0, n, device="cuda")
    C = torch.full((m, n), float("nan"), device="cuda")
    run = lambda: plan.run_ex(dA.data_ptr(), dB.data_ptr(), C.data_ptr(), 1.0, 0.0, bias.data_ptr(),
                              g.GEMM_F32_ACT_GELU, stream())
    run()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        nA, nB = _device_operands(m, n, k, layout_b, seed=2600 + rep)
        dA.copy_(nA)
        dB.copy_(nB)
        C.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = C.cpu().numpy()
        C.fill_(float("nan"))
        run()                                   # the eager run of the same plan and inputs
        torch.cuda.synchronize()
        want = C.cpu().numpy()
        assert np.isfinite(got).all(), f"replay {rep}: NaN in C"
        assert np.array_equal(got, want), f"replay {rep} differs from the eager run"
    assert g.gemm_f32_plan_check(plan.handle) is False
    del graph

"""Performance-model helpers against the worked numbers the pages print
(tests/golden/perf_model_worked_numbers.json) and against the compiler's own
occupancy report for every compiled kernel."""
import json
import os
import re

import pytest

from dense_gemm_optimisation_fp32_amd import perfmodel as pm

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "perf_model_worked_numbers.json")))
RESOURCES = os.path.join(os.path.dirname(os.path.dirname(__file__)), "dense_gemm_optimisation_fp32_amd",
                         "_build", "kernel_resources.txt")


def test_ridge_point():
    g = GOLDEN["ridge_point"]
    r = pm.ridge_point(g["peak_flops"], g["bandwidth"])
    assert abs(r - g["expect"]) / g["expect"] < g["rel_tol"]
    # MI355X: 157.3 TFLOP/s over 8 TB/s
    assert abs(pm.ridge_point(pm.MI355X_FP32_MATRIX_PEAK, pm.MI355X_HBM_BANDWIDTH) - 19.66) < 0.01


def test_lds_loads_per_fma():
    g = GOLDEN["lds_loads_per_fma"]
    assert pm.lds_loads_per_fma(g["tm"], g["tn"]) == g["expect"]
    assert pm.lds_loads_per_fma(1, 1) == 2.0


@pytest.mark.parametrize("per_block,expect", GOLDEN["smem_residency"]["cases"])
def test_smem_residency(per_block, expect):
    assert pm.resident_by_capacity(GOLDEN["smem_residency"]["capacity_kb"], per_block) == expect


@pytest.mark.parametrize("regs,expect", GOLDEN["register_residency"]["cases"])
def test_register_residency(regs, expect):
    g = GOLDEN["register_residency"]
    assert pm.resident_by_registers(g["regs_per_sm"], g["threads"], regs) == expect


@pytest.mark.parametrize("regs,expect", GOLDEN["register_granularity"]["cases"])
def test_register_granularity_step(regs, expect):
    g = GOLDEN["register_granularity"]
    assert pm.resident_by_registers(g["regs_per_sm"], g["threads"], regs, g["granule"]) == expect


@pytest.mark.parametrize("limits,expect", GOLDEN["resident_min"]["cases"])
def test_resident_min(limits, expect):
    assert pm.resident_blocks(*limits) == expect


def test_boundary_tile():
    g = GOLDEN["boundary_tile"]
    tiles, last, frac = pm.boundary_tiles(g["extent"], g["tile"])
    assert (tiles, last) == (g["tiles"], g["last"])
    assert abs(frac - 300 / 512) < 1e-12


@pytest.mark.parametrize("cf,expect", GOLDEN["coarsening_saving"]["cases"])
def test_coarsening_saving(cf, expect):
    assert pm.coarsening_saving(cf) == pytest.approx(expect)
    # consistent with the general tile-traffic count: TW x (TW*CF) tiles vs TW x TW
    m = n = k = 1024
    tw = 32
    saving = 1 - pm.tiled_load_bytes(m, n, k, tw, tw * cf) / pm.tiled_load_bytes(m, n, k, tw, tw)
    assert saving == pytest.approx(expect)


def test_intensity():
    g = GOLDEN["intensity"]
    assert pm.intensity_tiled(g["tile_width"]) == pytest.approx(g["tiled"])
    assert pm.intensity_coarsened(g["tile_width"], g["coarse_factor"]) == pytest.approx(g["coarsened"])
    assert pm.intensity_tiled(1) == pytest.approx(GOLDEN["naive_intensity"]["expect"])


def test_workload_counts():
    assert pm.gemm_flops(4096, 4096, 4096) == 2 * 4096 ** 3
    assert pm.compulsory_bytes(4096, 4096, 4096) == 3 * 4 * 4096 ** 2
    # skinny case: 67.6 MB at 8 TB/s is about 8.45 us
    t = pm.compulsory_bytes(16, 4096, 4096) / pm.MI355X_HBM_BANDWIDTH
    assert 8.4e-6 < t < 8.5e-6
    assert pm.arithmetic_intensity(16, 4096, 4096) < pm.ridge_point(pm.MI355X_FP32_MATRIX_PEAK,
                                                                      pm.MI355X_HBM_BANDWIDTH)


def test_wave_quantisation():
    assert pm.wave_quantisation(256) == (1.0, 1.0)
    waves, eff = pm.wave_quantisation(340)
    assert waves == pytest.approx(340 / 256) and eff == pytest.approx(340 / 512)


def _parse_resources():
    text = open(RESOURCES).read()
    kernels = []
    cur = {}
    for line in text.splitlines():
        m = re.search(r"remark:\s+([A-Za-z /\[\]]+?):\s+(\S+)", line)
        if not m:
            continue
        key, val = m.group(1).strip(), m.group(2)
        if key == "Function Name":
            cur = {"name": val}
            kernels.append(cur)
        else:
            cur[key] = val
    return kernels


@pytest.mark.skipif(not os.path.exists(RESOURCES), reason="library not built")
def test_occupancy_model_matches_compiler_report():
    kernels = [k for k in _parse_resources() if "gemm" in k["name"]]
    assert kernels
    for k in kernels:
        vgpr = int(k["VGPRs"])
        agpr = int(k.get("AGPRs", 0))
        occ = int(k["Occupancy [waves/SIMD]"])
        assert int(k["ScratchSize [bytes/lane]"]) == 0, f"{k['name']} spills"
        lds = int(k["LDS Size [bytes/block]"])
        by_regs = pm.gfx950_waves_per_simd_from_regs(vgpr, agpr)
        # the compiler's figure is the register/LDS bound for one workgroup size class
        assert by_regs >= occ, (k["name"], by_regs, occ)
        assert lds <= pm.MI355X_LDS_PER_CU

"""Host-side logic of bench.py (CPU): the engine-clock sampler, the roofline
object and the counter-gating of the traffic figure."""
import os
import sys
import time

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import WORKLOADS  # noqa: E402


def test_clock_sampler_reads_the_current_level(tmp_path):
    p = tmp_path / "pp_dpm_sclk"
    p.write_text("0: 500Mhz\nS: 2387Mhz *\n1: 2400Mhz\n")
    c = bench.ClockSampler(period_s=0.001)
    c.path = str(p)
    with c:
        time.sleep(0.03)
    assert c.samples and set(c.samples) == {2387}
    assert c.mean_mhz() == 2387


def test_clock_sampler_without_a_single_gpu_reports_nothing(monkeypatch):
    import glob

    monkeypatch.setattr(glob, "glob", lambda pattern: ["/a/pp_dpm_sclk", "/b/pp_dpm_sclk"])
    c = bench.ClockSampler()
    assert c.path is None
    with c:
        pass
    assert c.mean_mhz() is None


def _res(name, kernel_avg_s, sclk, kind=0, plan_name="dma_256x256x16_w4x2_s4"):
    from dense_gemm_optimisation_fp32_amd import perfmodel as pm

    w = WORKLOADS[name]
    return {"workload": w, "plan": {"kind": kind, "name": plan_name}, "kernel_avg_s": kernel_avg_s,
            "sclk_mhz": sclk, "flops": pm.gemm_flops(w.m, w.n, w.k),
            "bytes": pm.compulsory_bytes(w.m, w.n, w.k)}


def test_roofline_scales_the_peak_to_the_measured_clock():
    flop = 2 * 4096 ** 3
    t = flop / 150e12                      # 150 TFLOP/s
    res = _res("sq4096", t, 2390.0)
    res["sclk_samples"] = 10
    r = bench.roofline(res)
    assert r["bound"] == "mfma" and r["achieved"] == pytest.approx(150.0, rel=1e-3)
    assert r["frac"] == pytest.approx(150.0 / 157.3, abs=1e-4)
    # at 2390 MHz the peak is 157.3 * 2390 / 2400
    assert r["frac_at_sclk"] == pytest.approx(150.0 / (157.3 * 2390 / 2400), abs=1e-4)
    r = bench.roofline(_res("sq4096", t, None))
    assert r["sclk_mhz"] is None and r["frac_at_sclk"] is None


def test_roofline_bandwidth_bound_and_traffic_gating():
    w = WORKLOADS["skinny"]
    nbytes = 4 * (w.m * w.k + w.k * w.n + w.m * w.n)
    r = bench.roofline(_res("skinny", nbytes / 4e12, None, kind=2, plan_name="skinny_16x64_w16_d4"))
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["achieved"] == pytest.approx(4000.0, rel=1e-3)
    assert r["traffic"] is None            # no counters taken for this kernel
    # the headline counters apply only while the kernel sources are unchanged
    rec = bench.TRAFFIC_COUNTERS["sq4096"]
    got = bench.traffic_bytes("sq4096", rec["kernel"])
    if rec["sources_sha1"] == bench.kernel_sources_sha1():
        assert got and got > 0
    else:
        assert got is None
    assert bench.traffic_bytes("sq4096", "some_other_kernel") is None


def test_clock_reading_below_what_the_rate_needs_is_dropped():
    """An idle-level reading (as pp_dpm_sclk gave on one box: 880 MHz while
    the kernel ran at 147 TFLOP/s) implies a fraction above 1: null."""
    flop = 2 * 4096 ** 3
    res = _res("sq4096", flop / 147e12, 880.0)
    res["sclk_samples"] = 10
    r = bench.roofline(res)
    assert r["frac_at_sclk"] is None and "did not track" in r["sclk_note"]
    res = _res("sq4096", flop / 147e12, 2380.0)
    res["sclk_samples"] = 2                  # too few samples
    r = bench.roofline(res)
    assert r["frac_at_sclk"] is None
    res["sclk_samples"] = 10
    r = bench.roofline(res)
    assert r["frac_at_sclk"] == pytest.approx(147.0 / (157.3 * 2380 / 2400), abs=1e-4)


def test_clock_sampler_idle_level_file(tmp_path):
    p = tmp_path / "pp_dpm_sclk"
    p.write_text("S: 880Mhz *\n0: 500Mhz\n1: 2400Mhz\n")
    c = bench.ClockSampler(period_s=0.001)
    c.path = str(p)
    with c:
        time.sleep(0.03)
    res = _res("sq4096", 2 * 4096 ** 3 / 147e12, c.mean_mhz())
    res["sclk_samples"] = len(c.samples)
    assert bench.roofline(res)["frac_at_sclk"] is None


def test_profile_kernel_short_names():
    """The profile summaries name kernels the way the variant table does."""
    from dense_gemm_optimisation_fp32_amd.rocprof_summary import short_name

    assert short_name("void gemmf32::gemm_mfma_dma_kernel<gemmf32::DmaTile<256, 256, 16, 4, 2, 4, true>, "
                      "false, false, false, true>(gemmf32::GemmArgs)") == "dma_256x256x16_w4x2_s4_wide"
    assert short_name("void gemmf32::gemm_mfma_dma_kernel<gemmf32::DmaTile<256, 128, 16, 2, 2, 3, true>, "
                      "true, false, false, false>(gemmf32::GemmArgs)") == "dma_256x128x16_s3_bcol"
    assert short_name("void gemmf32::gemm_mfma_dma_sk_kernel<gemmf32::DmaTile<64, 128, 16, 2, 2, 2, true>, "
                      "false>(gemmf32::GemmArgs)") == "sk_dma_64x128x16_s2"
    assert short_name("void gemmf32::gemm_skinny_kernel<gemmf32::SkinnyTile<16, 4, 16>, false>"
                      "(gemmf32::GemmArgs)") == "skinny_16x16_w16_d4"
    assert short_name("void gemmf32::gemm_skinny_kernel<gemmf32::SkinnyTile<8, 4, 64, 2>, true>"
                      "(gemmf32::GemmArgs)") == "skinny_32x64_w8_d4"
    assert short_name("void gemmf32::gemm_mfma_dma_sliver_kernel<gemmf32::DmaTile<128, 128, 16, 2, 2, 3, false>, "
                      "false, false, false, true>(gemmf32::GemmArgs)") == "dma_128x128x16_s3_wide_sliver"
    assert short_name("void gemmf32::gemm_fewcol_kernel<gemmf32::FewColTile<1, 4, 2>, false>"
                      "(gemmf32::GemmArgs)") == "fewcol_r1"
    assert short_name("void gemmf32::gemm_fewcol_kernel<gemmf32::FewColTile<1>, true>"
                      "(gemmf32::GemmArgs)") == "fewcol_r1_bcol"
    assert short_name("void gemmf32::gemm_fewcol_kernel<gemmf32::FewColTile<4, 4, 2, 1024>, false>"
                      "(gemmf32::GemmArgs)") == "fewcol_r4_k1024"
    assert short_name("void gemmf32::gemm_fewcol_t_kernel<gemmf32::FewColTile<1, 8, 1, 2048>, true>"
                      "(gemmf32::GemmArgs)") == "fewcol_r1_w8_t_bcol"
    assert short_name("_ZN7gemmf3220gemm_fewcol_t_kernelINS_10FewColTileILi4ELi8ELi1ELi1024EEELb1EEEvNS_8GemmArgsE"
                      ) == "fewcol_r4_k1024_w8_t_bcol"
    assert short_name("void gemmf32::gemm_fewcol_kernel<gemmf32::FewColTile<8, 4, 2, 1024>, false>"
                      "(gemmf32::GemmArgs)") == "fewcol_r8"
    assert short_name("void gemmf32::gemm_fewcol_t_kernel<gemmf32::FewColTile<1, 4, 2, 2048>, true>"
                      "(gemmf32::GemmArgs)") == "fewcol_r1_t_bcol"
    assert short_name("_ZN7gemmf3220gemm_fewcol_t_epi_kernelINS_10FewColTileILi4ELi4ELi2ELi1024EEELb1EEEvNS_8GemmArgsE"
                      ) == "fewcol_r4_k1024_t_bcol"
    assert short_name("_ZN7gemmf3218gemm_fewcol_kernelINS_10FewColTileILi1ELi4ELi2ELi2048EEELb0EEEvNS_8GemmArgsE"
                      ) == "fewcol_r1"

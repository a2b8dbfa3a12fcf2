"""Host-side checks of the C ABI (no GPU compute).

The library must load, export every function include/gemm_f32.h declares,
validate arguments without touching a device, and report the no-device case
cleanly.  Nothing here launches a kernel.
"""
import ctypes
import os
import re

import pytest
import torch

import dense_gemm_optimisation_fp32_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm_f32.h")
HAS_GPU = torch.cuda.is_available()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_f32_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(g.LIB_PATH):
        pytest.fail("libgemm_f32.so is not built (run __graft_entry__.build())")
    return g.load_library()


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(g.EXPORTED_FUNCTIONS)


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(g.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), f"{name} not exported"


def test_header_compiles_as_c(tmp_path):
    src = tmp_path / "t.c"
    src.write_text('#include "gemm_f32.h"\nint main(void){struct gemm_f32_info i; (void)i; '
                   'return GEMM_F32_SUCCESS + GEMM_F32_COL_MAJOR - 1;}\n')
    import subprocess
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER),
                        "-c", str(src), "-o", str(tmp_path / "t.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_info_struct_layout_matches_c(tmp_path):
    """The ctypes mirror of struct gemm_f32_info has the C size and offsets."""
    src = tmp_path / "s.c"
    fields = [f for f, _ in g.gemm_f32_info._fields_]
    body = "".join(f'printf("%zu ", offsetof(struct gemm_f32_info, {f}));' for f in fields)
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "gemm_f32.h"\n'
                   f'int main(void){{{body} printf("%zu\\n", sizeof(struct gemm_f32_info)); return 0;}}\n')
    import subprocess
    exe = tmp_path / "s"
    r = subprocess.run(["gcc", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True).stdout.split()]
    expect = [getattr(g.gemm_f32_info, f).offset for f in fields] + [ctypes.sizeof(g.gemm_f32_info)]
    assert out == expect


@pytest.mark.parametrize("args,ok", [
    ((4, 4, 4, 0, 4, 4, 4), True),
    ((4, 4, 4, 1, 4, 4, 4), True),
    ((5003, 4097, 2049, 0, 2049, 4097, 4097), True),
    ((8192, 14336, 4096, 0, 4096, 14336, 14336), True),
    ((4, 6, 5, 1, 5, 5, 6), True),           # column-major B needs ldb >= k
    ((4, 6, 5, 1, 5, 4, 6), False),
    ((4, 6, 5, 0, 5, 5, 6), False),          # row-major B needs ldb >= n
    ((0, 4, 4, 0, 4, 4, 4), False),
    ((4, 0, 4, 0, 4, 4, 4), False),
    ((4, 4, 0, 0, 4, 4, 4), False),
    ((-1, 4, 4, 0, 4, 4, 4), False),
    ((4, 4, 4, 2, 4, 4, 4), False),          # bad layout
    ((4, 4, 4, 0, 3, 4, 4), False),          # lda < k
    ((4, 4, 4, 0, 4, 4, 3), False),          # ldc < n
    ((1 << 16, 1 << 14, 1 << 14, 0, 1 << 14, 1 << 14, 1 << 14), False),  # C extent >= 2^31 bytes
    ((2, 2, 2, 0, 1 << 40, 2, 2), False),    # absurd stride
])
def test_validate(lib, args, ok):
    st = g.gemm_f32_validate(*args)
    assert st == (g.GEMM_F32_SUCCESS if ok else g.GEMM_F32_ERR_INVALID_VALUE)


@pytest.mark.parametrize("args,ok", [
    ((4, 6, 5, 0, 0, 5, 6, 6), True),
    ((4, 6, 5, 1, 0, 4, 6, 6), True),        # column-major A needs lda >= m
    ((4, 6, 5, 1, 0, 3, 6, 6), False),
    ((4, 6, 5, 1, 1, 7, 5, 6), True),
    ((4, 6, 5, 0, 0, 4, 6, 6), False),       # row-major A needs lda >= k
    ((4, 6, 5, 2, 0, 5, 6, 6), False),       # bad layout_a
    ((1 << 15, 4, 1 << 15, 1, 0, 1 << 15, 4, 4), False),  # column-major A extent >= 2^31 bytes
])
def test_validate_ex(lib, args, ok):
    st = g.gemm_f32_validate_ex(*args)
    assert st == (g.GEMM_F32_SUCCESS if ok else g.GEMM_F32_ERR_INVALID_VALUE)


def test_validate_is_validate_ex_with_row_major_a(lib):
    for args in [(4, 4, 4, 0, 4, 4, 4), (4, 6, 5, 1, 5, 4, 6), (4, 4, 4, 0, 3, 4, 4)]:
        m, n, k, lb, lda, ldb, ldc = args
        assert g.gemm_f32_validate(*args) == g.gemm_f32_validate_ex(m, n, k, 0, lb, lda, ldb, ldc)


def test_create_ex_rejects_invalid_before_device(lib):
    h = ctypes.c_void_p(1234)
    st = lib.gemm_f32_create_ex(ctypes.byref(h), 4, 4, 4, 1, 0, 3, 4, 4, 0)     # lda < m
    assert st == g.GEMM_F32_ERR_INVALID_VALUE and h.value is None
    st = lib.gemm_f32_create_ex(ctypes.byref(h), 4, 4, 4, 0, 0, 4, 4, 4, 2)     # bad epilogue flag
    assert st == g.GEMM_F32_ERR_INVALID_VALUE and h.value is None
    assert lib.gemm_f32_run_ex(None, 16, 16, 16, 1.0, 0.0, None, 0, None) == g.GEMM_F32_ERR_INVALID_VALUE


def test_create_rejects_invalid_before_device(lib):
    h = ctypes.c_void_p(1234)
    st = lib.gemm_f32_create(ctypes.byref(h), 0, 4, 4, 0, 4, 4, 4)
    assert st == g.GEMM_F32_ERR_INVALID_VALUE and h.value is None
    assert lib.gemm_f32_create(None, 4, 4, 4, 0, 4, 4, 4) == g.GEMM_F32_ERR_INVALID_VALUE
    st = lib.gemm_f32_create_variant(ctypes.byref(h), 999, 4, 4, 4, 0, 4, 4, 4)
    assert st == g.GEMM_F32_ERR_INVALID_VALUE and h.value is None


@pytest.mark.skipif(HAS_GPU, reason="checks the no-device path")
def test_create_without_device_reports_no_device(lib):
    h = ctypes.c_void_p()
    st = lib.gemm_f32_create(ctypes.byref(h), 64, 64, 64, 0, 64, 64, 64)
    assert st == g.GEMM_F32_ERR_NO_DEVICE and h.value is None
    with pytest.raises(g.GemmF32Error):
        g.gemm_f32_create(64, 64, 64, 0, 64, 64, 64)


def test_null_handling(lib):
    assert lib.gemm_f32_destroy(None) == g.GEMM_F32_SUCCESS
    info = g.gemm_f32_info()
    assert lib.gemm_f32_describe(None, ctypes.byref(info)) == g.GEMM_F32_ERR_INVALID_VALUE
    assert lib.gemm_f32_run(None, 16, 16, 16, None) == g.GEMM_F32_ERR_INVALID_VALUE
    assert lib.gemm_f32_variant_info(0, None) == g.GEMM_F32_ERR_INVALID_VALUE


def test_error_strings(lib):
    for st in range(7):
        s = g.gemm_f32_error_string(st)
        assert s and s != "unknown status"
    assert g.gemm_f32_error_string(99) == "unknown status"
    assert g.gemm_f32_last_hip_error() == 0


def test_variant_table(lib):
    n = g.gemm_f32_num_variants()
    assert n >= 4
    kinds = set()
    for v in range(n):
        info = g.gemm_f32_variant_info(v)
        assert info["variant"] == v and info["name"]
        assert info["threads"] % 64 == 0 and info["lds_bytes"] <= 160 * 1024
        assert info["bm"] % info["waves_m"] == 0 and info["bn"] % info["waves_n"] == 0
        kinds.add(info["kind"])
    assert g.GEMM_F32_KIND_MFMA in kinds and g.GEMM_F32_KIND_VALU in kinds
    with pytest.raises(g.GemmF32Error):
        g.gemm_f32_variant_info(n)


def test_binding_strides_from_tensors():
    A = torch.empty(8, 12)
    B = torch.empty(12, 20)
    assert g.operand_strides(A, B) == (8, 20, 12, 0, 0, 12, 20)
    Bt = torch.empty(20, 12).t()                      # column-major (12 x 20)
    assert g.operand_strides(A, Bt) == (8, 20, 12, 0, 1, 12, 12)
    Awide = torch.empty(8, 16)[:, :12]
    assert g.operand_strides(Awide, B) == (8, 20, 12, 0, 0, 16, 20)
    At = torch.empty(12, 8).t()                       # column-major A (8 x 12), lda = 8
    assert g.operand_strides(At, B) == (8, 20, 12, 1, 0, 8, 20)
    At_wide = torch.empty(12, 10)[:, :8].t()          # column-major A with lda = 10
    assert g.operand_strides(At_wide, Bt) == (8, 20, 12, 1, 1, 10, 12)
    with pytest.raises(ValueError):
        g.operand_strides(A, torch.empty(11, 20))
    with pytest.raises(ValueError):
        g.operand_strides(torch.empty(8, 24)[:, ::2], B)   # A with no unit stride


def test_variant_resources_from_the_build(lib):
    """Every variant reports its kernel's registers from the build's resource
    table; no kernel of any variant spills to scratch; the direct-to-LDS
    tiles hold their MFMA accumulators (16 per 32x32 block and lane) in the
    accumulation registers, or, where two or more wavefronts share a SIMD,
    among the ordinary ones, and their compiler occupancy agrees with the
    residency model of the registers and LDS they use."""
    from dense_gemm_optimisation_fp32_amd import perfmodel as pm

    for v in range(g.gemm_f32_num_variants()):
        info = g.gemm_f32_variant_info(v)
        assert info["vgprs"] > 0 and info["sgprs"] > 0, info["name"]
        assert info["scratch_bytes"] == 0, f"{info['name']} spills"
        assert 1 <= info["compiler_waves_per_simd"] <= 8
        assert info["workgroups_per_cu"] == 0 and info["waves_per_simd"] == 0   # plan-only fields
        if info["name"].startswith("dma_"):
            blocks = (info["wave_m"] // 32) * (info["wave_n"] // 32)
            if info["threads"] <= 256:
                assert info["agprs"] == 16 * blocks, info["name"]
            else:
                assert info["agprs"] in (0, 16 * blocks) and info["vgprs"] + info["agprs"] >= 16 * blocks, info["name"]
            wgs, waves = pm.gfx950_occupancy(info["vgprs"], info["agprs"], info["lds_bytes"], info["threads"])
            # the compiler's estimate per SIMD is at least what whole workgroups give
            assert info["compiler_waves_per_simd"] >= waves, info["name"]


def test_plan_check_null_handling(lib):
    lost = ctypes.c_int(7)
    assert lib.gemm_f32_plan_check(None, ctypes.byref(lost)) == g.GEMM_F32_ERR_INVALID_VALUE

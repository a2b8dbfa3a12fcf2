"""Python binding of libgemm_f32.so, the gfx950 single-precision GEMM.

Argument marshalling only: every step of C = A.B runs in the library's HIP
kernels.  PyTorch supplies device memory and streams.  The names mirror the C
ABI in include/gemm_f32.h; functions return Python values and raise
``GemmF32Error`` on a non-success status.  There is no fallback: if the
library is not built, loading it raises.

    import torch, dense_gemm_optimisation_fp32_amd as g
    C = g.matmul(A, B)          # A (M,K), B (K,N), each row- or column-major
    Y = g.linear(X, W, bias, activation="gelu")   # act(X.W + bias), fused
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch  # imported first so the library binds to the HIP runtime torch loaded

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libgemm_f32.so")

GEMM_F32_ROW_MAJOR = 0
GEMM_F32_COL_MAJOR = 1

GEMM_F32_SUCCESS = 0
GEMM_F32_ERR_INVALID_VALUE = 1
GEMM_F32_ERR_NO_DEVICE = 2
GEMM_F32_ERR_UNSUPPORTED_DEVICE = 3
GEMM_F32_ERR_HIP = 4
GEMM_F32_ERR_ALLOC = 5
GEMM_F32_ERR_SCRATCH_TOO_SMALL = 6

GEMM_F32_ACT_NONE = 0
GEMM_F32_ACT_RELU = 1
GEMM_F32_ACT_GELU = 2
_ACTIVATIONS = {None: 0, "none": 0, "relu": 1, "gelu": 2, 0: 0, 1: 1, 2: 2}

GEMM_F32_KIND_MFMA = 0
GEMM_F32_KIND_VALU = 1
GEMM_F32_KIND_SKINNY = 2
GEMM_F32_KIND_FEWCOL = 3

EXPORTED_FUNCTIONS = (
    "gemm_f32_validate", "gemm_f32_create", "gemm_f32_create_variant", "gemm_f32_run",
    "gemm_f32_destroy", "gemm_f32_describe", "gemm_f32_num_variants", "gemm_f32_variant_info",
    "gemm_f32_error_string", "gemm_f32_last_hip_error", "gemm_f32_validate_ex", "gemm_f32_create_ex",
    "gemm_f32_run_ex", "gemm_f32_plan_check", "gemm_f32_run_noalloc",
)


class gemm_f32_info(ctypes.Structure):
    _fields_ = [
        ("variant", ctypes.c_int), ("kind", ctypes.c_int),
        ("bm", ctypes.c_int), ("bn", ctypes.c_int), ("bk", ctypes.c_int),
        ("waves_m", ctypes.c_int), ("waves_n", ctypes.c_int),
        ("wave_m", ctypes.c_int), ("wave_n", ctypes.c_int),
        ("threads", ctypes.c_int), ("lds_bytes", ctypes.c_int), ("stages", ctypes.c_int),
        ("split_k", ctypes.c_int), ("stream_k", ctypes.c_int),
        ("stream_k_tiles", ctypes.c_int), ("layout_a", ctypes.c_int), ("epilogue", ctypes.c_int),
        ("aligned", ctypes.c_int),
        ("tiles_m", ctypes.c_int64), ("tiles_n", ctypes.c_int64), ("k_tiles", ctypes.c_int64),
        ("grid", ctypes.c_int64), ("group_m", ctypes.c_int), ("c_store_width", ctypes.c_int),
        ("name", ctypes.c_char * 64),
        ("vgprs", ctypes.c_int), ("agprs", ctypes.c_int), ("sgprs", ctypes.c_int),
        ("scratch_bytes", ctypes.c_int), ("compiler_waves_per_simd", ctypes.c_int),
        ("workgroups_per_cu", ctypes.c_int), ("waves_per_simd", ctypes.c_int),
        ("sliver_cols", ctypes.c_int64), ("sliver_variant", ctypes.c_int), ("sliver_stream_k", ctypes.c_int),
        ("sliver_fused", ctypes.c_int),
        ("transposed", ctypes.c_int),
    ]

    def as_dict(self):
        d = {name: getattr(self, name) for name, _ in self._fields_}
        d["name"] = self.name.decode()
        return d


class GemmF32Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        hip = gemm_f32_last_hip_error() if status == GEMM_F32_ERR_HIP else 0
        msg = f"{where}: {gemm_f32_error_string(status)} (status {status}"
        msg += f", hipError {hip})" if hip else ")"
        super().__init__(msg)


_lib = None
_lib_lock = threading.Lock()


def load_library():
    """Load libgemm_f32.so (raises if it has not been built)."""
    global _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                               "python -m dense_gemm_optimisation_fp32_amd.build")
        lib = ctypes.CDLL(LIB_PATH)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        plan_p = ctypes.POINTER(vp)
        info_p = ctypes.POINTER(gemm_f32_info)
        sig = {
            "gemm_f32_validate": ([i64, i64, i64, i32, i64, i64, i64], i32),
            "gemm_f32_create": ([plan_p, i64, i64, i64, i32, i64, i64, i64], i32),
            "gemm_f32_create_variant": ([plan_p, i32, i64, i64, i64, i32, i64, i64, i64], i32),
            "gemm_f32_run": ([vp, vp, vp, vp, vp], i32),
            "gemm_f32_destroy": ([vp], i32),
            "gemm_f32_describe": ([vp, info_p], i32),
            "gemm_f32_num_variants": ([], i32),
            "gemm_f32_variant_info": ([i32, info_p], i32),
            "gemm_f32_error_string": ([i32], ctypes.c_char_p),
            "gemm_f32_last_hip_error": ([], i32),
            "gemm_f32_validate_ex": ([i64, i64, i64, i32, i32, i64, i64, i64], i32),
            "gemm_f32_create_ex": ([plan_p, i64, i64, i64, i32, i32, i64, i64, i64, i32], i32),
            "gemm_f32_run_ex": ([vp, vp, vp, vp, ctypes.c_float, ctypes.c_float, vp, i32, vp], i32),
            "gemm_f32_plan_check": ([vp, ctypes.POINTER(i32)], i32),
            "gemm_f32_run_noalloc": ([i64, i64, i64, i32, i64, i64, i64, vp, vp, vp, vp], i32),
        }
        for name, (args, res) in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
        return lib


# --- the C ABI, one Python function per entry point -------------------------

def gemm_f32_validate(m, n, k, layout_b, lda, ldb, ldc) -> int:
    """Pure argument check; returns the status code (no device needed)."""
    return int(load_library().gemm_f32_validate(m, n, k, layout_b, lda, ldb, ldc))


def gemm_f32_create(m, n, k, layout_b, lda, ldb, ldc) -> int:
    """Returns the plan handle (an integer address)."""
    h = ctypes.c_void_p()
    st = load_library().gemm_f32_create(ctypes.byref(h), m, n, k, layout_b, lda, ldb, ldc)
    if st != GEMM_F32_SUCCESS:
        raise GemmF32Error(st, "gemm_f32_create")
    return h.value


def gemm_f32_create_variant(variant, m, n, k, layout_b, lda, ldb, ldc) -> int:
    h = ctypes.c_void_p()
    st = load_library().gemm_f32_create_variant(ctypes.byref(h), variant, m, n, k, layout_b, lda, ldb, ldc)
    if st != GEMM_F32_SUCCESS:
        raise GemmF32Error(st, "gemm_f32_create_variant")
    return h.value


def gemm_f32_run(plan, A_ptr, B_ptr, C_ptr, stream=None) -> None:
    st = load_library().gemm_f32_run(plan, A_ptr, B_ptr, C_ptr, stream)
    if st != GEMM_F32_SUCCESS:
        raise GemmF32Error(st, "gemm_f32_run")


def gemm_f32_run_noalloc(m, n, k, layout_b, lda, ldb, ldc, A_ptr, B_ptr, C_ptr, stream=None) -> None:
    """C = A.B with no allocation (partial sums in the library's per-GPU
    scratch area); calls on one GPU must not overlap in time."""
    st = load_library().gemm_f32_run_noalloc(m, n, k, layout_b, lda, ldb, ldc, A_ptr, B_ptr, C_ptr, stream)
    if st != GEMM_F32_SUCCESS:
        raise GemmF32Error(st, "gemm_f32_run_noalloc")


def gemm_f32_validate_ex(m, n, k, layout_a, layout_b, lda, ldb, ldc) -> int:
    return int(load_library().gemm_f32_validate_ex(m, n, k, layout_a, layout_b, lda, ldb, ldc))


def gemm_f32_create_ex(m, n, k, layout_a, layout_b, lda, ldb, ldc, epilogue=0) -> int:
    h = ctypes.c_void_p()
    st = load_library().gemm_f32_create_ex(ctypes.byref(h), m, n, k, layout_a, layout_b, lda, ldb, ldc, epilogue)
    if st != GEMM_F32_SUCCESS:
        raise GemmF32Error(st, "gemm_f32_create_ex")
    return h.value


def gemm_f32_run_ex(plan, A_ptr, B_ptr, C_ptr, alpha=1.0, beta=0.0, bias_ptr=None, activation=0,
                    stream=None) -> None:
    st = load_library().gemm_f32_run_ex(plan, A_ptr, B_ptr, C_ptr, alpha, beta, bias_ptr, activation, stream)
    if st != GEMM_F32_SUCCESS:
        raise GemmF32Error(st, "gemm_f32_run_ex")


def gemm_f32_plan_check(plan) -> bool:
    """True if a run of the plan since the last check gave up waiting for a
    partial sum (and wrote NaN for it); clears the record.  Synchronise the
    plan's streams first."""
    lost = ctypes.c_int(0)
    st = load_library().gemm_f32_plan_check(plan, ctypes.byref(lost))
    if st != GEMM_F32_SUCCESS:
        raise GemmF32Error(st, "gemm_f32_plan_check")
    return bool(lost.value)


def gemm_f32_destroy(plan) -> None:
    load_library().gemm_f32_destroy(plan)


def gemm_f32_describe(plan) -> dict:
    info = gemm_f32_info()
    st = load_library().gemm_f32_describe(plan, ctypes.byref(info))
    if st != GEMM_F32_SUCCESS:
        raise GemmF32Error(st, "gemm_f32_describe")
    return info.as_dict()


def gemm_f32_num_variants() -> int:
    return int(load_library().gemm_f32_num_variants())


def gemm_f32_variant_info(variant) -> dict:
    info = gemm_f32_info()
    st = load_library().gemm_f32_variant_info(variant, ctypes.byref(info))
    if st != GEMM_F32_SUCCESS:
        raise GemmF32Error(st, "gemm_f32_variant_info")
    return info.as_dict()


def gemm_f32_error_string(status) -> str:
    return load_library().gemm_f32_error_string(status).decode()


def gemm_f32_last_hip_error() -> int:
    return int(load_library().gemm_f32_last_hip_error())


# --- torch-tensor convenience (marshalling only) ------------------------------

class Plan:
    """Owns a plan handle for one (shape, layouts, strides, variant, epilogue)."""

    def __init__(self, m, n, k, layout_b, lda, ldb, ldc, variant=None, layout_a=0, epilogue=0):
        self.key = (m, n, k, layout_b, lda, ldb, ldc, variant, layout_a, epilogue)
        if layout_a != GEMM_F32_ROW_MAJOR or epilogue:
            if variant is not None:
                raise ValueError("column-major A and the epilogue use the default variant choice")
            self.handle = gemm_f32_create_ex(m, n, k, layout_a, layout_b, lda, ldb, ldc, epilogue)
        elif variant is None:
            self.handle = gemm_f32_create(m, n, k, layout_b, lda, ldb, ldc)
        else:
            self.handle = gemm_f32_create_variant(variant, m, n, k, layout_b, lda, ldb, ldc)
        self.info = gemm_f32_describe(self.handle)
        # Plans that split tiles along k own a device workspace that two runs
        # must not share at the same time: such a plan serves one stream.
        self.has_workspace = self.info["split_k"] > 1 or self.info["stream_k"] > 0 or self.info["sliver_stream_k"] > 0
        self.stream = None

    def run(self, A_ptr, B_ptr, C_ptr, stream=None):
        gemm_f32_run(self.handle, A_ptr, B_ptr, C_ptr, stream)

    def run_ex(self, A_ptr, B_ptr, C_ptr, alpha=1.0, beta=0.0, bias_ptr=None, activation=0, stream=None):
        gemm_f32_run_ex(self.handle, A_ptr, B_ptr, C_ptr, alpha, beta, bias_ptr, activation, stream)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h and _lib is not None:
            _lib.gemm_f32_destroy(h)
            self.handle = None


_plan_cache: dict = {}
_plan_lock = threading.Lock()


def get_plan(m, n, k, layout_b, lda, ldb, ldc, variant=None, device=None, layout_a=0, epilogue=0,
             stream=None) -> Plan:
    """The cached plan for a shape.  A plan with a workspace (split-k or
    stream-K) belongs to the first stream that asks for it; another stream
    gets a plan (and workspace) of its own, so runs on two streams never
    share partial sums."""
    key = (device, m, n, k, layout_b, lda, ldb, ldc, variant, layout_a, epilogue)
    with _plan_lock:
        p = _plan_cache.get(key)
        if p is None:
            p = Plan(m, n, k, layout_b, lda, ldb, ldc, variant, layout_a, epilogue)
            _plan_cache[key] = p
        if not p.has_workspace:
            return p
        if p.stream is None:
            p.stream = stream
        if p.stream == stream:
            return p
        skey = key + (stream,)
        q = _plan_cache.get(skey)
        if q is None:
            q = Plan(m, n, k, layout_b, lda, ldb, ldc, variant, layout_a, epilogue)
            q.stream = stream
            _plan_cache[skey] = q
        return q


def operand_strides(A: torch.Tensor, B: torch.Tensor, layout_b=None, layout_a=None):
    """(m, n, k, layout_a, layout_b, lda, ldb) from tensor shapes and strides.

    A is the logical (M, K) matrix: unit stride along K means row-major, unit
    stride along M (a transposed view of a (K, M) tensor) column-major.  B is
    the logical (K, N) matrix: unit stride along N means row-major, unit
    stride along K column-major."""
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("A and B must be 2-D")
    m, k = A.shape
    k2, n = B.shape
    if k != k2:
        raise ValueError(f"inner dimensions differ: A is {tuple(A.shape)}, B is {tuple(B.shape)}")
    layouts = {"row": GEMM_F32_ROW_MAJOR, "col": GEMM_F32_COL_MAJOR}
    if layout_a is None:
        layout_a = GEMM_F32_ROW_MAJOR if (A.stride(1) == 1 or k == 1) else GEMM_F32_COL_MAJOR
    if isinstance(layout_a, str):
        layout_a = layouts[layout_a]
    if layout_a == GEMM_F32_ROW_MAJOR:
        if A.stride(1) != 1 and m > 1 and k > 1:
            raise ValueError("row-major A needs unit stride along K")
        lda = A.stride(0) if m > 1 else k
    else:
        if A.stride(0) != 1 and m > 1:
            raise ValueError("column-major A needs unit stride along M")
        lda = A.stride(1) if k > 1 else m
    if layout_b is None:
        layout_b = GEMM_F32_ROW_MAJOR if (B.stride(1) == 1 or n == 1) else GEMM_F32_COL_MAJOR
    if isinstance(layout_b, str):
        layout_b = layouts[layout_b]
    if layout_b == GEMM_F32_ROW_MAJOR:
        if B.stride(1) != 1 and n > 1:
            raise ValueError("row-major B needs unit stride along N")
        ldb = B.stride(0) if k > 1 else n
    else:
        if B.stride(0) != 1 and k > 1:
            raise ValueError("column-major B needs unit stride along K")
        ldb = B.stride(1) if n > 1 else k
    return m, n, k, layout_a, layout_b, lda, ldb


def _check_pair(A, B):
    if A.dtype != torch.float32 or B.dtype != torch.float32:
        raise TypeError("float32 operands only")
    if not (A.is_cuda and B.is_cuda) or A.device != B.device:
        raise ValueError("A and B must be on the same GPU")


def _output(out, m, n, device):
    if out is None:
        return torch.empty((m, n), dtype=torch.float32, device=device)
    if out.shape != (m, n) or out.dtype != torch.float32 or out.device != device:
        raise ValueError("out must be a float32 (M, N) tensor on A's device")
    if out.stride(1) != 1 and n > 1:
        raise ValueError("out must be row-major")
    return out


def matmul(A: torch.Tensor, B: torch.Tensor, layout_b=None, out: torch.Tensor | None = None,
           variant: int | None = None) -> torch.Tensor:
    """C = A.B on A's device and the current stream (float32 only)."""
    _check_pair(A, B)
    m, n, k, layout_a, layout_b, lda, ldb = operand_strides(A, B, layout_b)
    out = _output(out, m, n, A.device)
    ldc = out.stride(0) if m > 1 else n
    stream = torch.cuda.current_stream(A.device).cuda_stream
    plan = get_plan(m, n, k, layout_b, lda, ldb, ldc, variant, A.device.index, layout_a, stream=stream)
    plan.run(A.data_ptr(), B.data_ptr(), out.data_ptr(), stream)
    return out


def linear(A: torch.Tensor, B: torch.Tensor, bias: torch.Tensor | None = None, activation=None,
           alpha: float = 1.0, beta: float = 0.0, out: torch.Tensor | None = None) -> torch.Tensor:
    """C = act(alpha * A.B + beta * C + bias) in one kernel (float32 only);
    ``activation`` is None/"none", "relu" or "gelu"; ``out`` supplies C when
    beta != 0."""
    _check_pair(A, B)
    act = _ACTIVATIONS[activation]
    m, n, k, layout_a, layout_b, lda, ldb = operand_strides(A, B)
    if beta != 0.0 and out is None:
        raise ValueError("beta != 0 reads C: pass it as out")
    out = _output(out, m, n, A.device)
    ldc = out.stride(0) if m > 1 else n
    bias_ptr = None
    if bias is not None:
        if bias.dtype != torch.float32 or bias.device != A.device or bias.numel() != n or not bias.is_contiguous():
            raise ValueError("bias must be a contiguous float32 tensor of N values on A's device")
        bias_ptr = bias.data_ptr()
    stream = torch.cuda.current_stream(A.device).cuda_stream
    plan = get_plan(m, n, k, layout_b, lda, ldb, ldc, None, A.device.index, layout_a, 1, stream=stream)
    plan.run_ex(A.data_ptr(), B.data_ptr(), out.data_ptr(), alpha, beta, bias_ptr, act, stream)
    return out

"""Helpers for the GPU tests: move numpy storage buffers to the device, run one
GEMM through the C ABI binding, bring C back."""
import numpy as np
import torch

import dense_gemm_optimisation_fp32_amd as g


def device():
    return torch.device("cuda", 0)


def to_dev(x: np.ndarray, offset_elems: int = 0) -> torch.Tensor:
    """Flat float32 device buffer holding x, starting `offset_elems` in (for
    misaligned-pointer tests).  Returns the base tensor."""
    flat = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    t = torch.empty(flat.size + offset_elems, dtype=torch.float32, device=device())
    t[offset_elems:].copy_(torch.from_numpy(flat))
    return t


def run_gemm(A: np.ndarray, B: np.ndarray, m, n, k, layout_b, lda=None, ldb=None, ldc=None,
             variant=None, offsets=(0, 0, 0), c_fill=0.0, repeat=1):
    """C = A.B through gemm_f32_create(_variant)/gemm_f32_run.

    Returns (C as an (m, ldc) numpy array including its padding, plan info)."""
    lda = k if lda is None else lda
    ldb = (n if layout_b == 0 else k) if ldb is None else ldb
    ldc = n if ldc is None else ldc
    dA = to_dev(A, offsets[0])
    dB = to_dev(B, offsets[1])
    c_elems = (m - 1) * ldc + n
    dC = torch.full((c_elems + offsets[2],), c_fill, dtype=torch.float32, device=device())
    if variant is None:
        plan = g.gemm_f32_create(m, n, k, layout_b, lda, ldb, ldc)
    else:
        plan = g.gemm_f32_create_variant(variant, m, n, k, layout_b, lda, ldb, ldc)
    try:
        info = g.gemm_f32_describe(plan)
        stream = torch.cuda.current_stream().cuda_stream
        outs = []
        for _ in range(repeat):
            g.gemm_f32_run(plan, dA.data_ptr() + 4 * offsets[0], dB.data_ptr() + 4 * offsets[1],
                           dC.data_ptr() + 4 * offsets[2], stream)
            torch.cuda.synchronize()
            outs.append(dC[offsets[2]:].cpu().numpy().copy())
    finally:
        g.gemm_f32_destroy(plan)
    full = np.full(m * ldc, np.float32(c_fill), dtype=np.float32)
    full[:c_elems] = outs[-1]
    if repeat > 1:
        return full.reshape(m, ldc), info, outs
    return full.reshape(m, ldc), info


def variants():
    return list(range(g.gemm_f32_num_variants()))

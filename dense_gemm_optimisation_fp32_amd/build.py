"""Build libgemm_f32.so in-tree with hipcc for gfx950.

Usage: ``python -m dense_gemm_optimisation_fp32_amd.build`` (or call
``build()``).  Always recompiles.  The compiler's per-kernel resource report
(VGPRs, AGPRs, LDS, scratch, occupancy) is written next to the build log in
``_build/kernel_resources.txt`` for the tile/occupancy sweep.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(REPO_DIR, "include")
LIB_PATH = os.path.join(PKG_DIR, "libgemm_f32.so")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
SOURCES = [os.path.join(CSRC, "gemm_f32.hip")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-mcode-object-version=5",
    # Packed FP32 instructions stay off in every kernel.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC,
           "-Rpass-analysis=kernel-resource-usage", "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    report = os.path.join(BUILD_DIR, "kernel_resources.txt")
    with open(report, "w") as f:
        f.write(proc.stderr)
    if proc.returncode != 0:
        errors = [ln for ln in proc.stderr.splitlines() if "error" in ln or "Error" in ln]
        raise RuntimeError("hipcc failed:\n" + "\n".join(errors[:40] or proc.stderr.splitlines()[-40:]))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""Performance-model arithmetic for the GEMM: work counts, roofline, per-tile
traffic and occupancy.  Host-side bookkeeping for the benchmark and the
tile/occupancy sweep; nothing here touches the device or the product's
results.

Sources:
  * TFLOPS = 2*M*N*K / t, and the ridge point = peak FLOP/s / bandwidth
    ("GEMM 性能优化", sections 指标与目标 and Roofline 与平衡点).
  * Shared-memory accesses per multiply-add of a TM x TN register tile scale
    as 1/TM + 1/TN ("GEMM 性能优化", 台阶 2).
  * Global traffic of a tiled product and of thread coarsening, and the
    resulting arithmetic intensity ("PMPP Chapter 06", section 3, the traffic
    analysis after the coarsened kernel).
  * Resident blocks = the minimum over the shared-memory, register, thread,
    wave and hardware limits, each a floor division ("GPU 算子优化中的数据复用",
    sections 4, 6 and 12); boundary-tile waste (section 10.3).

The MI355X figures are AMD's published ones, not the pages'.
"""
from __future__ import annotations

import math

# MI355X (gfx950) published peaks.
MI355X_FP32_MATRIX_PEAK = 157.3e12    # FLOP/s, dense FP32 on the matrix cores
# FLOP/s, published FP32 vector peak: 256 CUs x 4 SIMDs x 64 lanes x 2 FLOP
# per 2 cycles x 2.4 GHz.  Unpacked FMAs reach it in their two-operand form:
# a probe of independent FMA chains (one MI355X, not shipped) issued
# v_fmac_f32_e32 (VOP2) at 127.6 TFLOP/s with 32 chains per lane (0.81 of
# this, with the loop's own instructions), i.e. one wavefront instruction
# every two cycles per SIMD, while the three-operand v_fma_f32 (VOP3) topped
# out at 75.7 (half the rate).  The vector-ALU kernel here emits only
# v_fmac_f32_e32 (packed FP32 is disabled in every kernel).
MI355X_FP32_VECTOR_PEAK = 157.3e12
MI355X_HBM_BANDWIDTH = 8.0e12         # B/s
MI355X_CUS = 256
MI355X_XCDS = 8
MI355X_PEAK_SCLK_HZ = 2.4e9
MI355X_LDS_PER_CU = 160 * 1024
MI355X_REGS_PER_SIMD_LANE = 512       # architectural + accumulation VGPRs per lane of a SIMD
MI355X_MAX_WAVES_PER_SIMD = 8
MI355X_SIMDS_PER_CU = 4


def gemm_flops(m: int, n: int, k: int) -> float:
    """One multiply and one add per (i, j, k)."""
    return 2.0 * m * n * k


def tflops(m: int, n: int, k: int, seconds: float) -> float:
    return gemm_flops(m, n, k) / seconds / 1e12


def compulsory_bytes(m: int, n: int, k: int, elem: int = 4) -> float:
    """Read A and B once and write C once (C is not read: it is overwritten)."""
    return float(elem) * (m * k + k * n + m * n)


def arithmetic_intensity(m: int, n: int, k: int) -> float:
    return gemm_flops(m, n, k) / compulsory_bytes(m, n, k)


def ridge_point(peak_flops: float, bandwidth: float) -> float:
    """FLOP/byte at which a kernel turns from bandwidth- to compute-bound."""
    return peak_flops / bandwidth


def roofline_bound(intensity: float, peak_flops: float, bandwidth: float) -> float:
    """Attainable FLOP/s at a given arithmetic intensity."""
    return min(peak_flops, intensity * bandwidth)


def lds_loads_per_fma(tm: int, tn: int) -> float:
    """Values read from shared memory per multiply-add of a TM x TN register
    outer product: TM + TN loads feed TM*TN multiply-adds."""
    return 1.0 / tm + 1.0 / tn


def tiled_load_bytes(m: int, n: int, k: int, bm: int, bn: int, elem: int = 4) -> float:
    """Global-memory bytes loaded by a tiled product with BM x BN output tiles:
    every A element is loaded once per tile column (n/BN times), every B
    element once per tile row (m/BM times)."""
    return float(elem) * (m * k * (n / bn) + k * n * (m / bm))


def coarsening_saving(coarse_factor: int) -> float:
    """Fraction of global loads saved by coarsening square TW x TW tiles by
    COARSE_FACTOR along one dimension: 1/2 (1 - 1/CF)."""
    return 0.5 * (1.0 - 1.0 / coarse_factor)


def intensity_tiled(tile_width: int, elem: int = 4) -> float:
    """FLOP/byte of a square-tiled product (loads only): 2mnk / (2*elem*mnk/TW)."""
    return tile_width / elem


def intensity_coarsened(tile_width: int, coarse_factor: int, elem: int = 4) -> float:
    """FLOP/byte with 1-D coarsening: 2mnk / (elem * mnk/TW * (1 + 1/CF))."""
    return 2.0 * tile_width / (elem * (1.0 + 1.0 / coarse_factor))


def resident_by_capacity(capacity: float, per_block: float) -> int:
    """Blocks that fit a capacity, rounding down (a leftover smaller than one
    block is wasted)."""
    if per_block <= 0:
        return 10 ** 9
    return int(math.floor(capacity / per_block))


def resident_by_registers(regs_per_sm: int, threads_per_block: int, regs_per_thread: int,
                          granule: int = 1) -> int:
    """Blocks the register file holds when registers are allocated per thread
    in multiples of `granule`."""
    alloc = int(math.ceil(regs_per_thread / granule) * granule)
    return resident_by_capacity(regs_per_sm, threads_per_block * alloc)


def resident_blocks(*limits: int) -> int:
    """Resident blocks are the minimum of every individual limit."""
    return min(limits)


def boundary_tiles(extent: int, tile: int):
    """(number of tiles, valid rows in the last tile, fraction of computed rows
    that are real) for one dimension."""
    tiles = -(-extent // tile)
    last = extent - (tiles - 1) * tile
    return tiles, last, extent / (tiles * tile)


# --- gfx950 occupancy ---------------------------------------------------------

def gfx950_waves_per_simd_from_regs(vgprs: int, agprs: int) -> int:
    """Waves per SIMD allowed by the unified register file: the accumulation
    registers start at the first multiple of 4 after the architectural VGPRs,
    and the whole allocation comes in granules of 8 (at most 512 per lane)."""
    arch = max(vgprs, 1)
    total = int(math.ceil(arch / 4) * 4) + agprs if agprs else arch
    total = int(math.ceil(total / 8) * 8)
    return max(0, min(MI355X_MAX_WAVES_PER_SIMD, MI355X_REGS_PER_SIMD_LANE // total))


def gfx950_occupancy(vgprs: int, agprs: int, lds_bytes: int, threads: int):
    """(workgroups per CU, waves per SIMD) from the register, LDS and wave
    limits of one CU."""
    waves_per_wg = -(-threads // 64)
    wg_per_simd_set = -(-waves_per_wg // MI355X_SIMDS_PER_CU)  # waves each SIMD gets per WG
    by_regs = gfx950_waves_per_simd_from_regs(vgprs, agprs) // wg_per_simd_set
    by_lds = resident_by_capacity(MI355X_LDS_PER_CU, lds_bytes) if lds_bytes else 10 ** 9
    by_waves = MI355X_MAX_WAVES_PER_SIMD // wg_per_simd_set
    wgs = resident_blocks(by_regs, by_lds, by_waves)
    return wgs, wgs * wg_per_simd_set


def wave_quantisation(tiles: int, cus: int = MI355X_CUS, wgs_per_cu: int = 1):
    """(waves of workgroups, efficiency of the last wave): the grid runs in
    ceil(tiles / slots) rounds of `slots = cus * wgs_per_cu` workgroups
    ("GEMM 性能优化", Wave 模型)."""
    slots = cus * wgs_per_cu
    rounds = -(-tiles // slots)
    return tiles / slots, tiles / (rounds * slots)

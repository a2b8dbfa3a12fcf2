// A whole-tile launch that also computes a narrow block of columns after its
// tiles (a "column sliver": n mod BN is a few columns, whose tiles would run
// the whole k-loop for them, "GPU 算子优化中的数据复用", 10.3).
//
// The grid's first sliver_wg0 workgroups are the tiles' (the whole-tile
// kernel's grid and rasterisation, unchanged); the workgroups after them run
// the few-column method on the sliver, one column each.  Workgroups are
// dispatched in grid order, so the sliver's workgroups start once every
// tile has a place, and fill the slots a partly filled last wave of tiles leaves idle
// instead of taking a launch of their own.  The few-column workgroups use
// the copy ring's LDS for their B chunk, and every row of the sliver is
// computed as the few-column kernel computes it (lane partial sums over k in
// the same order, the same butterfly), so C is bitwise the same as with the
// sliver launched on its own.
#pragma once

#include "fewcol_gemm.hpp"
#include "mfma_dma_gemm.hpp"

namespace gemmf32 {

// The sliver's tile: one column per workgroup, as many wavefronts as the
// whole-tile kernel's workgroup, one row per wavefront (half the few-column
// kernel's registers for A, so that the launch keeps the whole-tile
// kernel's occupancy).
template <class T>
using SliverTile = FewColTile<1, T::THREADS / 64, 1>;

// Registers are held to the whole-tile kernel's count of workgroups per CU
// (the few-column path would otherwise take more than the tiles' path and
// cost the launch a workgroup per CU).
template <class T, bool B_COL, bool A_COL = false, bool EPI = false, bool WIDE_C = false>
__global__ __launch_bounds__(T::THREADS, sk_waves_per_simd<T>()) void gemm_mfma_dma_sliver_kernel(GemmArgs g)
{
    static_assert(!A_COL && !EPI, "plain products only");
    using S = SliverTile<T>;
    constexpr int RING = T::STAGES * (T::A_CHUNKS + T::B_CHUNKS);
    static_assert(S::LDS_BYTES <= RING * 16, "the sliver's B chunk fits in the copy ring");
    __shared__ f32x4 lds[RING];
    if ((int)blockIdx.x >= g.sliver_wg0) {
        GemmArgs s = g;
        s.n = g.sliver_cols;
        s.B = g.sliver_B;
        s.b_bytes = g.sliver_b_bytes;
        s.C = g.sliver_C;
        fewcol_body<S, B_COL>(s, (int)blockIdx.x - g.sliver_wg0, lds);
        return;
    }
    dma_whole_tile<T, B_COL, false, false, WIDE_C>(g, lds);
}

}  // namespace gemmf32

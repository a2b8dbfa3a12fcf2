// Few-row FP32 GEMM (M <= 32): the bandwidth-bound shape.
//
// With M = 16 the product does ~8 FLOP per byte of B, below the MI355X ridge
// point of ~19.7 FLOP/B ("GEMM 性能优化", Roofline 与平衡点: below the ridge
// the kernel is bandwidth-limited), so the goal is to stream B from HBM once
// at full bandwidth.  Every element of B is used by all M rows in a single
// v_mfma_f32_16x16x4_f32 and never again, so B goes straight from HBM into
// MFMA operand registers (no LDS), and the work is split along k so that
// enough wavefronts keep enough loads in flight ("GPU 算子优化中的数据复用",
// 11.1: memory-bound kernels need parallelism to hide latency; "PMPP Chapter
// 06", section 2: many concurrent requests).
//
// MFMA 16x16x4 (f32): lane l supplies A[i = l%16][kk = l/16] and
// B[kk = l/16][j = l%16]; the 16x16 result sits as 4 values per lane at row
// 4*(l/16) + v, column l%16.  Lane group h = l/16 walks the k-run
// kq + 4h + t (t = 0..3) of each 16-k block, so one 16-byte load of A gives a
// lane its A values for 4 k-steps.  A wavefront covers 64 columns as 4 MFMA
// blocks with interleaved columns (lane column j stands for column 4*j + nb
// in block nb), so one 16-byte load of row-major B feeds all 4 blocks of a
// k-step; column-major B is loaded as 16 bytes along k of one column (4
// k-steps of one block).
//
// Split-k: a workgroup of WAVES wavefronts owns 16 rows x 64 columns x one
// k-split; each wavefront takes a contiguous share of the split, the shares
// are added in LDS in wavefront order, and the split's partial sums go to the
// plan's workspace (or straight to C when there is one split).  A second
// kernel adds the splits in split order.  Both orders are fixed, so results
// are reproducible run to run.  (Splitting k over workgroups is the
// partial-result-then-merge pattern the checklist of "PMPP Chapter 06",
// section 4, calls privatization.)
#pragma once

#include "device_common.hpp"

namespace gemmf32 {

template <int WAVES_>
struct SkinnyTile {
    static constexpr int WAVES = WAVES_;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int BM = 16, BN = 64, KQ = 16;   // rows, columns, k per load group
    static constexpr int UNROLL = 4;                  // k groups in flight per wavefront
};

// Loads of one 16-k group for lane (j, h): A[row][kq+4h .. +3] and the B
// values of the 4 k-steps x 4 blocks.  Element checks only when the group is
// not whole (tail of a split, or k past K).
template <bool B_COL>
__device__ __forceinline__ void skinny_load(const GemmArgs &g, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                            int row, int col0, int j, int h, int kq, int kend, bool whole,
                                            f32x4 &a, f32x4 (&b)[4])
{
    const int ka = kq + 4 * h;
    if (whole) {
        a = buf_load_x4(ra, elem_off(row < g.m, row, g.lda, ka));
        if constexpr (!B_COL) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
                b[t] = buf_load_x4(rb, (uint32_t)((ka + t) * g.ldb + col0 + 4 * j) * 4u);
        } else {
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const int col = col0 + 4 * j + nb;
                b[nb] = buf_load_x4(rb, elem_off(col < g.n, col, g.ldb, ka));
            }
        }
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) a[q] = buf_load_x1(ra, elem_off(row < g.m && ka + q < kend, row, g.lda, ka + q));
        if constexpr (!B_COL) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    const int col = col0 + 4 * j + nb;
                    b[t][nb] = buf_load_x1(rb, elem_off(ka + t < kend && col < g.n, ka + t, g.ldb, col));
                }
        } else {
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int col = col0 + 4 * j + nb;
                    b[nb][q] = buf_load_x1(rb, elem_off(col < g.n && ka + q < kend, col, g.ldb, ka + q));
                }
        }
    }
}

template <bool B_COL>
__device__ __forceinline__ void skinny_mfma(const f32x4 &a, const f32x4 (&b)[4], f32x4 (&acc)[4])
{
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const float bv = B_COL ? b[nb][t] : b[t][nb];
            acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t], bv, acc[nb], 0, 0, 0);
        }
}

// Grid: tiles_m * tiles_n * split_k workgroups.  Writes the split's partial
// sums to g.partial[split][m][n] (row stride n), or C when split_k == 1.
template <class T, bool B_COL>
__global__ __launch_bounds__(T::THREADS) void gemm_skinny_kernel(GemmArgs g)
{
    __shared__ float red[T::WAVES][T::BM * T::BN];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int j = lane & 15, h = lane >> 4;

    const int per_split = g.tiles_m * g.tiles_n;
    const int split = blockIdx.x / per_split;
    const int rest = blockIdx.x - split * per_split;
    const int tm = rest / g.tiles_n, tn = rest - (rest / g.tiles_n) * g.tiles_n;
    const int row0 = tm * T::BM, col0 = tn * T::BN;

    // This wavefront's k-range: the split's range cut into WAVES shares of
    // whole 16-k groups.
    const int ks0 = split * g.k_per_split;
    const int ks1 = min(g.k, ks0 + g.k_per_split);
    const int groups = (ks1 - ks0 + T::KQ - 1) / T::KQ;
    const int per_wave = (groups + T::WAVES - 1) / T::WAVES;
    const int kw0 = ks0 + wave * per_wave * T::KQ;
    const int kw1 = min(ks1, kw0 + per_wave * T::KQ);

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.A, g.a_bytes);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(g.B, g.b_bytes);

    const int row = row0 + j;    // A row this lane supplies
    f32x4 acc[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    int kq = kw0;
    // Whole groups, UNROLL at a time so that UNROLL * 5 loads are in flight.
    for (; kq + T::UNROLL * T::KQ <= kw1; kq += T::UNROLL * T::KQ) {
        f32x4 a[T::UNROLL];
        f32x4 b[T::UNROLL][4];
#pragma unroll
        for (int u = 0; u < T::UNROLL; ++u)
            skinny_load<B_COL>(g, ra, rb, row, col0, j, h, kq + u * T::KQ, kw1, true, a[u], b[u]);
#pragma unroll
        for (int u = 0; u < T::UNROLL; ++u) skinny_mfma<B_COL>(a[u], b[u], acc);
    }
    for (; kq < kw1; kq += T::KQ) {
        f32x4 a, b[4];
        skinny_load<B_COL>(g, ra, rb, row, col0, j, h, kq, kw1, kq + T::KQ <= kw1, a, b);
        skinny_mfma<B_COL>(a, b, acc);
    }

    // Add the wavefronts' shares in wavefront order.  Element (r, c) of the
    // 16 x 64 tile: r = 4*h + v, c = 4*j + nb.
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[wave][(4 * h + v) * T::BN + 4 * j + nb] = acc[nb][v];
    __syncthreads();
    float *out = g.split_k > 1 ? g.partial + (size_t)split * g.m * g.n : g.C;
    const int ld = g.split_k > 1 ? g.n : g.ldc;
    for (int e = tid; e < T::BM * T::BN; e += T::THREADS) {
        float s = red[0][e];
#pragma unroll
        for (int w = 1; w < T::WAVES; ++w) s += red[w][e];
        const int r = row0 + e / T::BN, c = col0 + e % T::BN;
        if (r < g.m && c < g.n) out[(size_t)r * ld + c] = s;
    }
}

// C[i][j] = sum over splits s = 0, 1, ... of partial[s][i][j], in that
// order.  The loads of up to 8 splits are issued together before they are
// added, so the kernel pays one memory latency per 8 splits, not per split.
// (Folding this into the split kernel with a last-arriver counter needs
// device-scope release/acquire fences, which write back and invalidate an
// XCD's L2 under all the other workgroups' streaming loads; measured 2-3x
// slower than this second launch.)
__global__ __launch_bounds__(256) void gemm_skinny_reduce_kernel(GemmArgs g)
{
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= g.m * g.n) return;
    const int r = idx / g.n, c = idx - (idx / g.n) * g.n;
    const size_t plane = (size_t)g.m * g.n;
    const float *p = g.partial + idx;
    float s = p[0];
    for (int s0 = 1; s0 < g.split_k; s0 += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = s0 + u < g.split_k ? p[(size_t)(s0 + u) * plane] : 0.0f;
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (s0 + u < g.split_k) s += v[u];
    }
    g.C[(size_t)r * g.ldc + c] = s;
}

}  // namespace gemmf32

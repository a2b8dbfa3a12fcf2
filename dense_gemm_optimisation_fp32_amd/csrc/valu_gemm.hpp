// LDS-tiled FP32 GEMM on the vector ALU: per-thread register outer product.
//
// Kept as the measured comparison to the matrix-core path.  It follows the
// parameter set recommended in "GEMM 性能优化" (推荐参数 table): a 128 x 128
// workgroup tile, k slabs of 8, 256 threads each owning an 8 x 8 block of C
// (台阶 2, register outer product: per k a thread reads 8 values of A and 8
// of B from LDS and does 64 multiply-adds), 16-byte vector loads
// (台阶 3) with A stored transposed in LDS so that a thread's 8 A values are
// two 16-byte reads, and two LDS buffers along k (台阶 6).
//
// Thread (ty, tx) of the 16 x 16 grid owns rows {4ty..4ty+3, 64+4ty..64+4ty+3}
// and columns {4tx..4tx+3, 64+4tx..64+4tx+3} of the tile, so the 16 threads of
// a row of the grid read 256 contiguous bytes of a B k-row and the A reads of
// a wavefront are four broadcast addresses.  The transposed (scalar) LDS
// writes use a row stride of BM + 4 floats, which moves the two k-halves of a
// wavefront's writes to different banks (padding, 台阶 4).
//
// Global loads are 16 bytes when the 4 elements are inside the matrix (4-byte
// alignment suffices), element by element in the k-tail slab and the tile
// column at the n edge; out-of-range elements read as zero.
//
// The FMAs are plain float multiply-adds (v_fmac_f32; packed FP32 is not
// used).  Its roofline is the FP32 vector peak, 157.3 TFLOP/s: measured at
// 85 TFLOP/s on 4096^3, unpacked FMAs are not held to half of that figure.
#pragma once

#include "device_common.hpp"

namespace gemmf32 {

struct ValuTile {
    static constexpr int BM = 128, BN = 128, BK = 8, TM = 8, TN = 8;
    static constexpr int THREADS = 256;
    static constexpr int AS = BM + 4;   // LDS row stride (floats) of transposed A
    static constexpr int BS = BN + 4;   // LDS row stride (floats) of B
    static constexpr int LDS_BYTES = 2 * BK * (AS + BS) * 4;
};

template <bool B_COL>
__global__ __launch_bounds__(ValuTile::THREADS) void gemm_valu_kernel(GemmArgs g)
{
    using T = ValuTile;
    __shared__ __attribute__((aligned(16))) float lds_a[2][T::BK * T::AS];  // [k][m]
    __shared__ __attribute__((aligned(16))) float lds_b[2][T::BK * T::BS];  // [k][n]

    const int tid = threadIdx.x;
    const int ty = tid >> 4, tx = tid & 15;

    int tm, tn;
    raster_tile(blockIdx.x, g, tm, tn);
    const int row0 = tm * T::BM, col0 = tn * T::BN;

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.A, g.a_bytes);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(g.B, g.b_bytes);
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(g.C, g.c_bytes);

    // Staging: one 4-float piece of A and one of B per thread and slab.
    //  A: row r = tid/2, k = 4*(tid%2) .. +3           -> As[k][r] (transposed)
    //  B row-major: k-row tid/32, n = 4*(tid%32) .. +3  -> Bs[k][n..n+3]
    //  B column-major: column tid/2, k = 4*(tid%2)..+3  -> Bs[k][n] (turned)
    const int a_r = tid >> 1, a_k = 4 * (tid & 1);
    const int b_kr = tid >> 5, b_n = 4 * (tid & 31);
    const int bc_n = tid >> 1, bc_k = 4 * (tid & 1);

    auto load = [&](int kt, f32x4 &va, f32x4 &vb) {
        const int k0 = kt * T::BK;
        const bool full_k = k0 + T::BK <= g.k;   // uniform: 16-byte loads along k are whole
        const int gr = row0 + a_r, gk = k0 + a_k;
        if (full_k) {
            va = buf_load_x4(ra, elem_off(gr < g.m, gr, g.lda, gk));
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                va[q] = buf_load_x1(ra, elem_off(gr < g.m && gk + q < g.k, gr, g.lda, gk + q));
        }
        if constexpr (!B_COL) {
            const bool full_n = col0 + T::BN <= g.n;
            const int bk = k0 + b_kr, bn = col0 + b_n;
            if (full_n) {
                vb = buf_load_x4(rb, elem_off(bk < g.k, bk, g.ldb, bn));
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    vb[q] = buf_load_x1(rb, elem_off(bk < g.k && bn + q < g.n, bk, g.ldb, bn + q));
            }
        } else {
            const int bn = col0 + bc_n, bk = k0 + bc_k;
            if (full_k) {
                vb = buf_load_x4(rb, elem_off(bn < g.n, bn, g.ldb, bk));
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    vb[q] = buf_load_x1(rb, elem_off(bn < g.n && bk + q < g.k, bn, g.ldb, bk + q));
            }
        }
    };
    auto store = [&](int buf, const f32x4 &va, const f32x4 &vb) {
        float *As = lds_a[buf];
        float *Bs = lds_b[buf];
#pragma unroll
        for (int q = 0; q < 4; ++q) As[(a_k + q) * T::AS + a_r] = va[q];
        if constexpr (!B_COL) {
            *reinterpret_cast<f32x4 *>(Bs + b_kr * T::BS + b_n) = vb;
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) Bs[(bc_k + q) * T::BS + bc_n] = vb[q];
        }
    };

    float acc[T::TM][T::TN];
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j) acc[i][j] = 0.0f;

    f32x4 va, vb;
    load(0, va, vb);
    store(0, va, vb);
    __syncthreads();

    for (int kt = 0; kt < g.k_tiles; ++kt) {
        const int buf = kt & 1;
        const bool more = kt + 1 < g.k_tiles;
        if (more) load(kt + 1, va, vb);
        const float *As = lds_a[buf];
        const float *Bs = lds_b[buf];
#pragma unroll
        for (int kk = 0; kk < T::BK; ++kk) {
            const f32x4 a0 = *reinterpret_cast<const f32x4 *>(As + kk * T::AS + 4 * ty);
            const f32x4 a1 = *reinterpret_cast<const f32x4 *>(As + kk * T::AS + 64 + 4 * ty);
            const f32x4 b0 = *reinterpret_cast<const f32x4 *>(Bs + kk * T::BS + 4 * tx);
            const f32x4 b1 = *reinterpret_cast<const f32x4 *>(Bs + kk * T::BS + 64 + 4 * tx);
            const float a[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            const float b[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
            for (int i = 0; i < T::TM; ++i)
#pragma unroll
                for (int j = 0; j < T::TN; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
        }
        if (more) store(buf ^ 1, va, vb);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < T::TM; ++i) {
        const int r = row0 + (i < 4 ? 4 * ty + i : 64 + 4 * ty + (i - 4));
#pragma unroll
        for (int hj = 0; hj < 2; ++hj) {
            const int c = col0 + 64 * hj + 4 * tx;
            if (c + 3 < g.n) {
                const f32x4 out = {acc[i][4 * hj], acc[i][4 * hj + 1], acc[i][4 * hj + 2], acc[i][4 * hj + 3]};
                buf_store_x4(out, rc, elem_off(r < g.m, r, g.ldc, c));
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    buf_store_x1(acc[i][4 * hj + q], rc, elem_off(r < g.m && c + q < g.n, r, g.ldc, c + q));
            }
        }
    }
}

}  // namespace gemmf32

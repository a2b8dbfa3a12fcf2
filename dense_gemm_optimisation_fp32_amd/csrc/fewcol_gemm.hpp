// Few-column FP32 GEMM (N <= 8): the matrix-vector-like shape.
//
// With a handful of columns every element of A is used N times and never
// again, so the product is bound by reading A once from memory ("GEMM 性能优化",
// Roofline 与平衡点: an arithmetic intensity of N/2 FLOP per byte is far
// below the ridge).  A tile of the matrix-core kernels would spend a whole
// 64- or 128-column k-loop on these few columns; here A streams straight
// into registers with 16-byte loads along k (64 lanes cover 1 KiB of one
// row per instruction, "PMPP Chapter 06", section 1: adjacent lanes read
// adjacent addresses) and meets the few B columns, which every row shares,
// in LDS.
//
// Workgroup: 4 wavefronts (WAVES), ROWS_PER_WAVE rows each (grid over row
// blocks and groups of R columns).  k runs in chunks of KC: the workgroup copies the
// chunk of its R columns of B into LDS (k-contiguous per column, zeros past
// K and past N), then each wavefront reads its rows' k-chunk, lane l taking
// k = 4l + 256q + t (t = 0..3), multiplies with one 16-byte LDS read per
// column and accumulates per lane.  The 64 lanes' partial sums of each
// output are then added by a butterfly over the wavefront (a fixed order, so
// results repeat bit for bit), and lane 0 stores them.
#pragma once

#include "device_common.hpp"

namespace gemmf32 {

template <int R_, int WAVES_ = 4, int ROWS_PER_WAVE_ = 2>
struct FewColTile {
    static_assert(R_ == 1 || R_ == 4 || R_ == 8, "columns per workgroup");
    static constexpr int R = R_;                 // columns of C per workgroup
    static constexpr int WAVES = WAVES_;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int ROWS_PER_WAVE = ROWS_PER_WAVE_;
    static constexpr int ROWS = WAVES * ROWS_PER_WAVE;   // rows of C per workgroup
    static constexpr int KC = R_ == 8 ? 1024 : 2048;   // k per LDS chunk (at most 32 KiB of B)
    static constexpr int GROUPS = KC / 256;      // 16-byte loads per lane per row and chunk
    static constexpr int LD = KC + 4;             // LDS floats per column (padded: conflict-free copies)
    static constexpr int LDS_BYTES = R * LD * 4;
};

// Workgroup barrier that waits for this wavefront's LDS accesses only
// (lgkmcnt(0); vmcnt, expcnt left at their maxima in the gfx9 encoding), so
// global loads issued before it stay in flight; the "memory" clobber keeps
// the compiler from moving LDS accesses across it.
__device__ __forceinline__ void fewcol_barrier()
{
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
    asm volatile("s_barrier" ::: "memory");
}

// Sum over the 64 lanes of a wavefront, butterfly order (every lane ends
// with the same total).
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// The B chunk into LDS: element (k, column j0 + j) for k < klen and
// j0 + j < n, zero elsewhere, at bsf[j * LD + k].  Column-major B: 16-byte
// loads along k of one column, one 16-byte LDS write each.  Row-major B with
// 4 or 8 columns: 16-byte loads of 4 columns of one k-row, four 4-byte LDS
// writes (the padded column stride spreads them over the banks).  One
// column of row-major B: 4-byte loads.  Partial groups (at K, or at N)
// element by element.
template <class T, bool B_COL>
__device__ __forceinline__ void fewcol_copy_b(const GemmArgs &g, __amdgpu_buffer_rsrc_t rb, f32x4 *bs, float *bsf,
                                              int kc, int klen, int j0, int tid)
{
    if constexpr (B_COL) {
        for (int e = tid; e < T::R * T::KC / 4; e += T::THREADS) {
            const int j = e / (T::KC / 4), kk = 4 * (e % (T::KC / 4));
            const bool col_ok = j0 + j < g.n;
            f32x4 v;
            if (col_ok && kk + 4 <= klen) {
                v = buf_load_x4(rb, elem_off(true, j0 + j, g.ldb, kc + kk));
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u) v[u] = buf_load_x1(rb, elem_off(col_ok && kk + u < klen, j0 + j, g.ldb, kc + kk + u));
            }
            bs[(j * T::LD + kk) / 4] = v;
        }
    } else if constexpr (T::R >= 4) {
        constexpr int Q = T::R / 4;
        for (int e = tid; e < T::KC * Q; e += T::THREADS) {
            const int kk = e / Q, c = e % Q;
            const int col = j0 + 4 * c;
            f32x4 v;
            if (kk < klen && col + 4 <= g.n) {
                v = buf_load_x4(rb, elem_off(true, kc + kk, g.ldb, col));
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u) v[u] = buf_load_x1(rb, elem_off(kk < klen && col + u < g.n, kc + kk, g.ldb, col + u));
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) bsf[(4 * c + u) * T::LD + kk] = v[u];
        }
    } else {
        for (int kk = tid; kk < T::KC; kk += T::THREADS)
            bsf[kk] = buf_load_x1(rb, elem_off(kk < klen && j0 < g.n, kc + kk, g.ldb, j0));
    }
}

// Workgroup `block` of the grid: ceil(m / ROWS) row blocks x ceil(n / R)
// column groups (row block fastest).  `bs`: LDS for the B chunk
// (T::LDS_BYTES).  Every row is computed the same way whatever the number of
// wavefronts, so a tile with more wavefronts gives bitwise the same C.
// C_T: the product is the transpose of the caller's (see gemm_fewcol_t_kernel),
// so result (row, j) is stored at C[j * ldc + row].
template <class T, bool B_COL, bool C_T = false>
__device__ __forceinline__ void fewcol_body(const GemmArgs &g, int block, f32x4 *bs)
{
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int row_blocks = (g.m + T::ROWS - 1) / T::ROWS;
    const int rb = block % row_blocks;
    const int j0 = (block / row_blocks) * T::R;
    const int row0 = rb * T::ROWS + wave * T::ROWS_PER_WAVE;

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.A, g.a_bytes);
    const __amdgpu_buffer_rsrc_t rb_ = make_rsrc(g.B, g.b_bytes);
    float *const bsf = reinterpret_cast<float *>(bs);

    float acc[T::ROWS_PER_WAVE][T::R];
#pragma unroll
    for (int t = 0; t < T::ROWS_PER_WAVE; ++t)
#pragma unroll
        for (int j = 0; j < T::R; ++j) acc[t][j] = 0.0f;

    for (int kc = 0; kc < g.k; kc += T::KC) {
        const int klen = min(T::KC, g.k - kc);
        // This chunk's A loads first (ROWS_PER_WAVE * GROUPS 16-byte loads
        // per lane), so that they are in flight with the B chunk's.
        f32x4 a[T::ROWS_PER_WAVE][T::GROUPS];
        if (klen == T::KC) {
            // A whole chunk: every group is whole (uniform branch).
#pragma unroll
            for (int t = 0; t < T::ROWS_PER_WAVE; ++t)
#pragma unroll
                for (int q = 0; q < T::GROUPS; ++q)
                    a[t][q] = buf_load_x4(ra, elem_off(row0 + t < g.m, row0 + t, g.lda, kc + 4 * lane + 256 * q));
        } else {
            // The last chunk: the groups below K with one load each, zeros
            // past it, and the group that K cuts element by element
            // (elements past K may be the next row's, or padding).
#pragma unroll
            for (int t = 0; t < T::ROWS_PER_WAVE; ++t)
#pragma unroll
                for (int q = 0; q < T::GROUPS; ++q) {
                    const int kk = 4 * lane + 256 * q;
                    const bool row_ok = row0 + t < g.m;
                    a[t][q] = buf_load_x4(ra, elem_off(row_ok && kk + 4 <= klen, row0 + t, g.lda, kc + kk));
                    if (kk < klen && kk + 4 > klen) {
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            a[t][q][u] = buf_load_x1(ra, elem_off(row_ok && kk + u < klen, row0 + t, g.lda, kc + kk + u));
                    }
                }
        }
        // The B chunk: element (k, column j0 + j) for k < klen and j0 + j < n,
        // zero elsewhere.  Column-major B is read along k; row-major B along
        // its few columns.  The barriers wait for LDS only: the A loads stay
        // in flight (the compiler waits for each load where its value is
        // used).
        fewcol_barrier();   // the previous chunk's LDS reads are done
        fewcol_copy_b<T, B_COL>(g, rb_, bs, bsf, kc, klen, j0, tid);
        fewcol_barrier();

#pragma unroll
        for (int q = 0; q < T::GROUPS; ++q) {
            const int kk = 4 * lane + 256 * q;
#pragma unroll
            for (int j = 0; j < T::R; ++j) {
                const f32x4 b = bs[(j * T::LD + kk) / 4];
#pragma unroll
                for (int t = 0; t < T::ROWS_PER_WAVE; ++t)
#pragma unroll
                    for (int u = 0; u < 4; ++u) acc[t][j] += a[t][q][u] * b[u];
            }
        }
    }

#pragma unroll
    for (int t = 0; t < T::ROWS_PER_WAVE; ++t) {
        const int row = row0 + t;
#pragma unroll
        for (int j = 0; j < T::R; ++j) {
            const float v = wave_sum(acc[t][j]);
            if (lane == 0 && row < g.m && j0 + j < g.n) {
                if constexpr (C_T)
                    g.C[(size_t)(j0 + j) * g.ldc + row] = v;
                else
                    g.C[(size_t)row * g.ldc + j0 + j] = v;
            }
        }
    }
}

// (Registers are held to four wavefronts per SIMD, 16 per CU, so that enough
// loads of A are in flight.)
template <class T, bool B_COL>
__global__ __launch_bounds__(T::THREADS, 4) void gemm_fewcol_kernel(GemmArgs g)
{
    __shared__ f32x4 bs[T::R * T::LD / 4];   // [column][k] chunk of B, k-contiguous
    fewcol_body<T, B_COL>(g, (int)blockIdx.x, bs);
}

// The transposed product C^T = B^T . A^T for one row of C and column-major B
// (y = W x with the weight W stored one output per row).  The kernel's A is
// the caller's B read as a row-major N x K matrix (its columns are contiguous
// along k, so every load instruction covers 1 KiB of one of them, where the
// few-row kernel's operand layout reads 64 bytes of each of 16 columns); its
// B is the caller's A read as a column-major K x M matrix; result (row, j) is
// element (j, row) of the caller's C.
template <class T, bool B_COL>
__global__ __launch_bounds__(T::THREADS, 4) void gemm_fewcol_t_kernel(GemmArgs g)
{
    __shared__ f32x4 bs[T::R * T::LD / 4];
    fewcol_body<T, B_COL, true>(g, (int)blockIdx.x, bs);
}

}  // namespace gemmf32

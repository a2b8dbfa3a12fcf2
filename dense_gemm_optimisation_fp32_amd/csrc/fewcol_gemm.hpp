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
#include "epilogue.hpp"

namespace gemmf32 {

template <int R_, int WAVES_ = 4, int ROWS_PER_WAVE_ = 2, int KC_ = (R_ == 8 ? 1024 : 2048)>
struct FewColTile {
    static_assert(R_ == 1 || R_ == 4 || R_ == 8, "columns per workgroup");
    static_assert(KC_ % 256 == 0 && R_ * (KC_ + 4) * 4 <= 33 * 1024, "k chunk: whole 256-k groups, at most ~32 KiB of B");
    static constexpr int R = R_;                 // columns of C per workgroup
    static constexpr int WAVES = WAVES_;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int ROWS_PER_WAVE = ROWS_PER_WAVE_;
    static constexpr int ROWS = WAVES * ROWS_PER_WAVE;   // rows of C per workgroup
    static constexpr int KC = KC_;               // k per LDS chunk
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
//
// Two ways to order it against the chunk's loads of A.  fewcol_copy_b loads
// and writes in one pass after A's loads are issued; memory loads complete in
// issue order, so its LDS writes wait for A's loads from memory as well.
// With 4 or 8 columns, a copy of 8 to 16 KiB per workgroup, that wait cost
// up to a fifth of the time: there fewcol_load_b issues the copy's loads into
// registers (FewColStage) before A's and fewcol_store_b writes them after,
// waiting for the B loads only (B is small and read from the L2).  Measured
// on one MI355X (us, staged / one pass): 4096x4x4096 14.8 / 18.0,
// 8192x4x8192 53.6 / 56.5, 8192x8x8192 68.1 / 79.8; the 8-column kernel on
// the transposed product of 8x4096x4096 with column-major B 21.2 / 26.4.
// Staged: the 8-column tile and the 4-column tile with 1024-k chunks.  Not
// staged: one column (no gain: 4096-row transposed products 1 % slower
// staged) and the 4-column tile with 2048-k chunks, whose staged copy does
// not fit the registers beside A's chunk (it spilled).  The two 4-column
// tiles split the shapes by k: the 1024-k staged tile took 4096x4x4096 from
// 18.0 to 14.6 us and 16384x3x4096 from 56.1 to 50.9, but 8192x4x8192 from
// 56.4 to 62.3 (twice the chunks, each a round trip of A's loads).  The
// staged 4-column tile runs eight wavefronts of one row each (the same 8 rows
// per workgroup, twice the wavefronts to cover the loads' latency):
// 4096x4x4096 13.61 against 14.57 us with four wavefronts of two rows,
// 16384x3x4096 49.63 / 50.86, the transposed 4x6144x4096 21.10 / 21.57
// (4x14336x4096 level).  The same change lost on the 8-column tile at
// 8192x8x8192 (70.95 / 67.77) and on the one-column tile at 8192x1x8192
// (51.50 / 49.70).
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

template <class T, bool B_COL>
constexpr bool fewcol_staged() { return T::R == 8 || (T::R == 4 && T::KC == 1024); }

template <class T, bool B_COL>
struct FewColStage {
    static constexpr bool ONE = !B_COL && T::R == 1;   // one column of row-major B: 4-byte elements
    static constexpr int TOTAL = B_COL ? T::R * T::KC / 4 : ONE ? T::KC : T::KC * (T::R / 4);
    static constexpr int CP = (TOTAL + T::THREADS - 1) / T::THREADS;   // elements per thread
    f32x4 v[ONE ? 1 : CP];
    float s[ONE ? CP : 1];
};

template <class T, bool B_COL>
__device__ __forceinline__ void fewcol_load_b(const GemmArgs &g, __amdgpu_buffer_rsrc_t rb, FewColStage<T, B_COL> &st,
                                              int kc, int klen, int j0, int tid)
{
    using S = FewColStage<T, B_COL>;
#pragma unroll
    for (int i = 0; i < S::CP; ++i) {
        const int e = tid + i * T::THREADS;
        const bool live = S::TOTAL % T::THREADS == 0 || e < S::TOTAL;
        if constexpr (B_COL) {
            const int j = e / (T::KC / 4), kk = 4 * (e % (T::KC / 4));
            const bool col_ok = live && j0 + j < g.n;
            if (col_ok && kk + 4 <= klen) {
                st.v[i] = buf_load_x4(rb, elem_off(true, j0 + j, g.ldb, kc + kk));
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    st.v[i][u] = buf_load_x1(rb, elem_off(col_ok && kk + u < klen, j0 + j, g.ldb, kc + kk + u));
            }
        } else if constexpr (!S::ONE) {
            constexpr int Q = T::R / 4;
            const int kk = e / Q, c = e % Q;
            const int col = j0 + 4 * c;
            if (live && kk < klen && col + 4 <= g.n) {
                st.v[i] = buf_load_x4(rb, elem_off(true, kc + kk, g.ldb, col));
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    st.v[i][u] = buf_load_x1(rb, elem_off(live && kk < klen && col + u < g.n, kc + kk, g.ldb, col + u));
            }
        } else {
            st.s[i] = buf_load_x1(rb, elem_off(live && e < klen && j0 < g.n, kc + e, g.ldb, j0));
        }
    }
}

template <class T, bool B_COL>
__device__ __forceinline__ void fewcol_store_b(const FewColStage<T, B_COL> &st, f32x4 *bs, float *bsf, int tid)
{
    using S = FewColStage<T, B_COL>;
#pragma unroll
    for (int i = 0; i < S::CP; ++i) {
        const int e = tid + i * T::THREADS;
        if (S::TOTAL % T::THREADS != 0 && e >= S::TOTAL) break;
        if constexpr (B_COL) {
            const int j = e / (T::KC / 4), kk = 4 * (e % (T::KC / 4));
            bs[(j * T::LD + kk) / 4] = st.v[i];
        } else if constexpr (!S::ONE) {
            constexpr int Q = T::R / 4;
            const int kk = e / Q, c = e % Q;
#pragma unroll
            for (int u = 0; u < 4; ++u) bsf[(4 * c + u) * T::LD + kk] = st.v[i][u];
        } else {
            bsf[e] = st.s[i];
        }
    }
}

// Workgroup `block` of the grid: ceil(m / ROWS) row blocks x ceil(n / R)
// column groups (row block fastest).  `bs`: LDS for the B chunk
// (T::LDS_BYTES).  Every row is computed the same way whatever the number of
// wavefronts, so a tile with more wavefronts gives bitwise the same C.
// C_T: the product is the transpose of the caller's (see gemm_fewcol_t_kernel),
// so result (row, j) is stored at C[j * ldc + row].  EPI: with the
// linear-layer epilogue (linear_epilogue) on C's element.
template <class T, bool B_COL, bool C_T = false, bool EPI = false>
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
        // This chunk's A loads (ROWS_PER_WAVE * GROUPS 16-byte loads per
        // lane), for a staged copy after the B chunk's loads.
        constexpr bool STAGED = fewcol_staged<T, B_COL>();
        FewColStage<T, B_COL> st;
        if constexpr (STAGED) fewcol_load_b<T, B_COL>(g, rb_, st, kc, klen, j0, tid);
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
        // The B chunk into LDS.  The barriers wait for LDS only: the A loads
        // stay in flight (the compiler waits for each load where its value
        // is used, and for the B loads before their LDS writes).
        fewcol_barrier();   // the previous chunk's LDS reads are done
        if constexpr (STAGED)
            fewcol_store_b<T, B_COL>(st, bs, bsf, tid);
        else
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
                const int cr = C_T ? j0 + j : row, cc = C_T ? row : j0 + j;   // C's row and column
                g.C[(size_t)cr * g.ldc + cc] = EPI ? linear_epilogue(g, v, cr, cc) : v;
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

// The same with the linear-layer epilogue.
template <class T, bool B_COL>
__global__ __launch_bounds__(T::THREADS, 4) void gemm_fewcol_epi_kernel(GemmArgs g)
{
    __shared__ f32x4 bs[T::R * T::LD / 4];
    fewcol_body<T, B_COL, false, true>(g, (int)blockIdx.x, bs);
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

// The same with the linear-layer epilogue.
template <class T, bool B_COL>
__global__ __launch_bounds__(T::THREADS, 4) void gemm_fewcol_t_epi_kernel(GemmArgs g)
{
    __shared__ f32x4 bs[T::R * T::LD / 4];
    fewcol_body<T, B_COL, true, true>(g, (int)blockIdx.x, bs);
}

}  // namespace gemmf32

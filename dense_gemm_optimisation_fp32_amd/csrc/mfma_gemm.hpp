// LDS-tiled FP32 GEMM on the gfx950 matrix cores (v_mfma_f32_32x32x2_f32).
//
// One workgroup computes a BM x BN tile of C, walking k in slabs of BK
// ("GEMM 性能优化", 台阶 1: the k-sum may be cut into slabs and the partial
// sums added).  Per slab:
//   * A (BM x BK, row-major in HBM) is copied into LDS with 16-byte loads
//     along k, k-contiguous per row ("PMPP Chapter 06", section 1: adjacent
//     lanes read adjacent addresses).
//   * B (BK x BN) lands in LDS n-contiguous per k-row.  Row-major B is read
//     with 16-byte loads along n.  Column-major B is read with 16-byte loads
//     along k of one column (the coalesced direction) and each lane turns its
//     4(k) x 4(n) block in registers before writing it: the corner turning
//     of "PMPP Chapter 06", section 1 (strategy 3), done in the staging step.
//   * Each wavefront owns a WM x WN tile of C held in MFMA accumulators
//     (register reuse: "GEMM 性能优化", 台阶 2 and 台阶 5).  An MFMA block is
//     32 x 32; a wavefront holds MB x NB of them.
//   * Two LDS buffers: the global loads of slab kt+1 are in flight while the
//     matrix cores work on slab kt, and land in the other buffer afterwards,
//     one barrier per slab ("GEMM 性能优化", 台阶 6, K-loop level).  Inside a
//     slab every fragment is read from LDS ahead of the MFMAs that use it
//     (台阶 6, p-loop level).
//
// k order inside a slab.  The MFMA takes two k values per lane pair
// (lane l < 32 holds k-index 0, lane l + 32 holds k-index 1).  Lane half h
// takes the contiguous run k = h*BK/2 + p, p = 0..BK/2-1, so one 16-byte LDS
// read gives a lane four consecutive k of its A row.  A and B use the same
// run, so every product A[i][k]*B[k][j] is formed exactly once.
//
// Column order inside a wavefront tile.  In MFMA block nb, lane column j
// stands for C column  NB*j + nb  of the wavefront tile, so a lane's B values
// for all NB blocks at one k are NB adjacent floats (one LDS read), and its
// results for the NB blocks are NB adjacent columns of C (one 16-byte store
// when NB = 4).
//
// LDS layout (both operands, both buffers):
//   As[row][chunk ^ swz_a(row)]   row < BM, chunk < BK/4 (16-byte chunks)
//   Bs[krow][chunk ^ swz_b(krow)] krow < BK, chunk < BN/4
// The XOR swizzles spread the 16-byte accesses of neighbouring lanes over
// distinct bank groups ("GEMM 性能优化", 台阶 4: padding or XOR swizzle,
// re-derived for 16-byte transactions).  swz_a serves the fragment reads
// (lanes on consecutive rows, same chunk); swz_b serves the corner-turning
// writes (lanes on k-rows 4 apart).  Both are correct for any bank count;
// their conflict-freedom is measured, not assumed.
#pragma once

#include "device_common.hpp"

namespace gemmf32 {

template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_>
struct MfmaTile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int THREADS = 64 * WAVES_M * WAVES_N;
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    static constexpr int MB = WM / 32, NB = WN / 32;     // MFMA blocks per wavefront
    static constexpr int KH = BK / 2;                    // k per lane half per slab
    static constexpr int ACH = BK / 4;                   // 16-byte chunks per A row
    static constexpr int BCH = BN / 4;                   // 16-byte chunks per B k-row
    static constexpr int A_CHUNKS = BM * ACH;
    static constexpr int B_CHUNKS = BK * BCH;
    static constexpr int A_PER_T = A_CHUNKS / THREADS;   // A chunks staged per thread
    static constexpr int B_PER_T = B_CHUNKS / THREADS;   // row-major B chunks per thread
    static constexpr int B_MICRO = (BN / 4) * (BK / 4);  // 4x4 blocks of column-major B
    static constexpr int B_MICRO_PER_T = (B_MICRO + THREADS - 1) / THREADS;
    static constexpr int SB = B_PER_T > 4 * B_MICRO_PER_T ? B_PER_T : 4 * B_MICRO_PER_T;
    static constexpr int LDS_BYTES = 2 * (A_CHUNKS + B_CHUNKS) * 16;

    static_assert(BK == 16, "swz_a assumes four 16-byte chunks per A row");
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wavefront tile is whole MFMA blocks");
    static_assert(NB == 1 || NB == 2 || NB == 4, "B fragment read is 4, 8 or 16 bytes");
    static_assert(A_CHUNKS % THREADS == 0 && B_CHUNKS % THREADS == 0, "even staging split");
    static_assert(BN % 64 == 0, "swz_b permutes within groups of 16 chunks");
    static_assert(LDS_BYTES <= 160 * 1024, "fits the 160 KB LDS of a CU");
};

// Chunk permutation of A row `row` (4 chunks per row).  Rows r, r+1, ... read
// at the same logical chunk land on distinct 16-byte bank groups for 8
// consecutive rows (32 four-byte banks) and for 16 consecutive rows (64 banks).
__device__ __forceinline__ int swz_a(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }

// Chunk permutation of B k-row `krow`: the corner-turning writes put lanes on
// k-rows 4*g + q (g = 0..3); this maps g to 0, 10, 4, 14 so that 8 and 16
// consecutive lanes hit distinct bank groups.  Values stay below 16.
__device__ __forceinline__ int swz_b(int krow)
{
    const int g = (krow >> 2) & 3;
    return 2 * g + 8 * (g & 1);
}

template <class T, bool B_COL, bool VEC>
__device__ __forceinline__ void mfma_load_slab(const GemmArgs &g, __amdgpu_buffer_rsrc_t ra,
                                               __amdgpu_buffer_rsrc_t rb, int row0, int col0,
                                               int kt, int tid, f32x4 (&sa)[T::A_PER_T],
                                               f32x4 (&sb)[T::SB])
{
    const int k0 = kt * T::BK;
#pragma unroll
    for (int i = 0; i < T::A_PER_T; ++i) {
        const int c = tid + i * T::THREADS;
        const int r = c / T::ACH, kc = c % T::ACH;
        const int gr = row0 + r, gk = k0 + kc * 4;
        if constexpr (VEC) {
            sa[i] = buf_load_x4(ra, elem_off(gr < g.m && gk < g.k, gr, g.lda, gk));
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                sa[i][q] = buf_load_x1(ra, elem_off(gr < g.m && gk + q < g.k, gr, g.lda, gk + q));
        }
    }
    if constexpr (!B_COL) {
#pragma unroll
        for (int i = 0; i < T::B_PER_T; ++i) {
            const int c = tid + i * T::THREADS;
            const int kr = c / T::BCH, nc = c % T::BCH;
            const int gk = k0 + kr, gn = col0 + nc * 4;
            if constexpr (VEC) {
                sb[i] = buf_load_x4(rb, elem_off(gk < g.k && gn < g.n, gk, g.ldb, gn));
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    sb[i][q] = buf_load_x1(rb, elem_off(gk < g.k && gn + q < g.n, gk, g.ldb, gn + q));
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < T::B_MICRO_PER_T; ++i) {
            const int u = tid + i * T::THREADS;
            if (T::B_MICRO % T::THREADS == 0 || u < T::B_MICRO) {
                const int kc = u % (T::BK / 4), ng = u / (T::BK / 4);
                const int gk = k0 + 4 * kc;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int gn = col0 + 4 * ng + c;   // column of B, k-contiguous in HBM
                    if constexpr (VEC) {
                        sb[4 * i + c] = buf_load_x4(rb, elem_off(gn < g.n && gk < g.k, gn, g.ldb, gk));
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            sb[4 * i + c][q] =
                                buf_load_x1(rb, elem_off(gn < g.n && gk + q < g.k, gn, g.ldb, gk + q));
                    }
                }
            }
        }
    }
}

template <class T, bool B_COL>
__device__ __forceinline__ void mfma_store_slab(f32x4 *As, f32x4 *Bs, int tid,
                                                const f32x4 (&sa)[T::A_PER_T],
                                                const f32x4 (&sb)[T::SB])
{
#pragma unroll
    for (int i = 0; i < T::A_PER_T; ++i) {
        const int c = tid + i * T::THREADS;
        const int r = c / T::ACH, kc = c % T::ACH;
        As[r * T::ACH + (kc ^ swz_a(r))] = sa[i];
    }
    if constexpr (!B_COL) {
#pragma unroll
        for (int i = 0; i < T::B_PER_T; ++i) {
            const int c = tid + i * T::THREADS;
            const int kr = c / T::BCH, nc = c % T::BCH;
            Bs[kr * T::BCH + (nc ^ swz_b(kr))] = sb[i];
        }
    } else {
#pragma unroll
        for (int i = 0; i < T::B_MICRO_PER_T; ++i) {
            const int u = tid + i * T::THREADS;
            if (T::B_MICRO % T::THREADS == 0 || u < T::B_MICRO) {
                const int kc = u % (T::BK / 4), ng = u / (T::BK / 4);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int kr = 4 * kc + q;
                    const f32x4 v = {sb[4 * i + 0][q], sb[4 * i + 1][q], sb[4 * i + 2][q],
                                     sb[4 * i + 3][q]};
                    Bs[kr * T::BCH + (ng ^ swz_b(kr))] = v;
                }
            }
        }
    }
}

template <class T>
__device__ __forceinline__ void mfma_compute_slab(const f32x4 *As, const f32x4 *Bs, int wr, int wc,
                                                  int l32, int half,
                                                  f32x16 (&acc)[T::MB][T::NB])
{
    // A fragments for the whole slab: KH consecutive k of one row per MFMA block.
    f32x4 af[T::MB][T::KH / 4];
#pragma unroll
    for (int mb = 0; mb < T::MB; ++mb) {
        const int r = wr * T::WM + mb * 32 + l32;
#pragma unroll
        for (int q = 0; q < T::KH / 4; ++q) {
            const int kc = half * (T::KH / 4) + q;
            af[mb][q] = As[r * T::ACH + (kc ^ swz_a(r))];
        }
    }
#pragma unroll
    for (int p = 0; p < T::KH; ++p) {
        const int kr = half * T::KH + p;
        const f32x4 *brow = Bs + kr * T::BCH;
        const int sw = swz_b(kr);
        float bv[T::NB];
        if constexpr (T::NB == 4) {
            const f32x4 t = brow[(wc * (T::WN / 4) + l32) ^ sw];
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) bv[nb] = t[nb];
        } else if constexpr (T::NB == 2) {
            const float *cp = reinterpret_cast<const float *>(brow + ((wc * (T::WN / 4) + (l32 >> 1)) ^ sw));
            const f32x2 t = *reinterpret_cast<const f32x2 *>(cp + 2 * (l32 & 1));
            bv[0] = t[0];
            bv[1] = t[1];
        } else {
            const float *cp = reinterpret_cast<const float *>(brow + ((wc * (T::WN / 4) + (l32 >> 2)) ^ sw));
            bv[0] = cp[l32 & 3];
        }
#pragma unroll
        for (int mb = 0; mb < T::MB; ++mb) {
            const float a = af[mb][p >> 2][p & 3];
#pragma unroll
            for (int nb = 0; nb < T::NB; ++nb)
                acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, bv[nb], acc[mb][nb], 0, 0, 0);
        }
    }
}

template <class T, bool B_COL, bool VEC>
__global__ __launch_bounds__(T::THREADS) void gemm_mfma_kernel(GemmArgs g)
{
    __shared__ f32x4 lds[2 * (T::A_CHUNKS + T::B_CHUNKS)];
    f32x4 *const lds_a = lds;                      // [2][A_CHUNKS]
    f32x4 *const lds_b = lds + 2 * T::A_CHUNKS;    // [2][B_CHUNKS]

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wr = wave % T::WAVES_M, wc = wave / T::WAVES_M;
    const int l32 = lane & 31, half = lane >> 5;

    int tm, tn;
    raster_tile(blockIdx.x, g, tm, tn);
    const int row0 = tm * T::BM, col0 = tn * T::BN;

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.A, g.a_bytes);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(g.B, g.b_bytes);
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(g.C, g.c_bytes);

    f32x16 acc[T::MB][T::NB];
#pragma unroll
    for (int mb = 0; mb < T::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < T::NB; ++nb) acc[mb][nb] = f32x16{};

    f32x4 sa[T::A_PER_T];
    f32x4 sb[T::SB];
    mfma_load_slab<T, B_COL, VEC>(g, ra, rb, row0, col0, 0, tid, sa, sb);
    mfma_store_slab<T, B_COL>(lds_a, lds_b, tid, sa, sb);
    __syncthreads();

    for (int kt = 0; kt < g.k_tiles; ++kt) {
        const int buf = kt & 1;
        const bool more = kt + 1 < g.k_tiles;
        if (more) mfma_load_slab<T, B_COL, VEC>(g, ra, rb, row0, col0, kt + 1, tid, sa, sb);
        mfma_compute_slab<T>(lds_a + buf * T::A_CHUNKS, lds_b + buf * T::B_CHUNKS, wr, wc, l32, half, acc);
        if (more) mfma_store_slab<T, B_COL>(lds_a + (buf ^ 1) * T::A_CHUNKS,
                                            lds_b + (buf ^ 1) * T::B_CHUNKS, tid, sa, sb);
        __syncthreads();
    }

    // Epilogue: lane (l32, half), accumulator element v of block (mb, nb) is
    // C row  mb*32 + 8*(v/4) + 4*half + v%4  and column  NB*l32 + nb  of the
    // wavefront tile.  C is overwritten; rows >= m and columns >= n are not
    // written (row padding of C included).
    const int cb = col0 + wc * T::WN + T::NB * l32;
#pragma unroll
    for (int mb = 0; mb < T::MB; ++mb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int r = row0 + wr * T::WM + mb * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
            if constexpr (VEC && T::NB == 4) {
                const f32x4 out = {acc[mb][0][v], acc[mb][1][v], acc[mb][2][v], acc[mb][3][v]};
                buf_store_x4(out, rc, elem_off(r < g.m && cb < g.n, r, g.ldc, cb));
            } else {
#pragma unroll
                for (int nb = 0; nb < T::NB; ++nb)
                    buf_store_x1(acc[mb][nb][v], rc, elem_off(r < g.m && cb + nb < g.n, r, g.ldc, cb + nb));
            }
        }
    }
}

}  // namespace gemmf32

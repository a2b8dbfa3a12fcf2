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
//
// Two-level double buffering ("GEMM 性能优化", 台阶 6), as a software
// pipeline over the k-steps of a slab:
//   * K-loop level: two LDS buffers.  The 16-byte global loads of slab kt+2
//     are issued in the middle of slab kt, right after the loads of slab kt+1
//     (issued one slab earlier) are written to the other LDS buffer; one
//     barrier per slab publishes that buffer.
//   * k-step level: the fragments of step p+1 are read from LDS while the
//     MFMAs of step p run (two register sets).  The barrier sits before the
//     last k-step of the slab: the MFMAs of that step, whose fragments are
//     already in registers, cover the latency of the first reads of the next
//     slab.
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
// writes (lanes on k-rows 4 apart).  Both permute chunks inside a row, so
// they are correct for any bank count; conflict-freedom is measured.
//
// Global accesses go through range-checked buffer descriptors.  Every slab but
// the last moves 4-element chunks with one 16-byte load each (the address then
// only needs 4-byte alignment); the last slab loads element by element with
// full m/n/k checks, and out-of-range elements read as zero, so they add
// nothing to the sums.  The main loop therefore carries no per-element branch.
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
    static constexpr int KH = BK / 2;                    // k-steps per slab
    static constexpr int AQ = KH / 4;                    // 16-byte A reads per row per slab
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
    static constexpr int STORE_STEP = KH / 2 - 1;        // k-step after which the next slab is written

    static_assert(BK == 16 || BK == 32, "swizzles are derived for 4 or 8 chunks per A row");
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wavefront tile is whole MFMA blocks");
    static_assert(NB == 1 || NB == 2 || NB == 4, "B fragment read is 4, 8 or 16 bytes");
    static_assert(A_CHUNKS % THREADS == 0 && B_CHUNKS % THREADS == 0, "even staging split");
    static_assert(BN % 64 == 0, "swz_b permutes within groups of 16 chunks");
    static_assert(LDS_BYTES <= 160 * 1024, "fits the 160 KB LDS of a CU");
};

// Chunk permutation of A row `row`.  A fragment read has lanes l and l+32 on
// the same row r = l % 32 and 16-byte chunks 2 apart; gfx950 serves a 16-byte
// read 16 lanes at a time from 64 four-byte banks (256 bytes), so the 16 rows
// of a lane group must land on 16 distinct 16-byte bank slots.  XOR-ing the
// chunk with the row's index among the rows that share a 256-byte line
// (r / 4 for 64-byte rows, r / 2 for 128-byte rows) does that; measured
// conflict-free with SQ_LDS_BANK_CONFLICT, where r>>1-based variants cost 2x.
template <int ACH>
__device__ __forceinline__ int swz_a(int row)
{
    if constexpr (ACH == 4) return (row >> 2) & 3;  // 64-byte rows: 4 per 256 bytes
    else return (row >> 1) & 7;                     // 128-byte rows: 2 per 256 bytes
}

// Chunk permutation of B k-row `krow`.  The corner-turning writes put the
// lanes of a group on k-rows 4*g + q (g = k-chunk index); the map of g gives
// distinct bank groups for 8 and for 16 consecutive lanes.  Values < 16.
template <int BK>
__device__ __forceinline__ int swz_b(int krow)
{
    if constexpr (BK == 16) {
        const int g = (krow >> 2) & 3;
        return 2 * g + 8 * (g & 1);
    } else {
        const int g = (krow >> 2) & 7;
        return 2 * g + (g >> 2);
    }
}

// Staging is split into pieces, one 16-byte global load and one 16-byte LDS
// write each, so the slab body can spread them between MFMAs.
//   pieces 0 .. A_PER_T-1            A chunks (row r, k-chunk kc)
//   pieces A_PER_T .. PIECES-1       B: row-major chunks, or for column-major
//                                    B the 4 columns (load) / 4 k-rows (write)
//                                    of each 4x4 micro-block
template <class T, bool B_COL>
struct Pieces {
    static constexpr int B = B_COL ? 4 * T::B_MICRO_PER_T : T::B_PER_T;
    static constexpr int COUNT = T::A_PER_T + B;
};

// Global -> register piece j of slab kt.
//
// MASKED = false is for every slab but the last: all BK values of k exist,
// so each 4-element chunk is one 16-byte load.  A rows >= m and column-major
// B columns >= n take the out-of-range offset (read as zero).  Row-major B is
// loaded whole even at the n edge: columns >= n only feed columns of C that
// are never stored, and a chunk that holds a valid column ends at most 3
// elements past it, inside the operand's extent because the next k-row
// exists and ldb >= 4 (the plan requires it for this path).
// MASKED = true (the last slab, or every slab of a plan whose ldb < 4) checks
// every element against m, n and k.
template <class T, bool B_COL, bool MASKED>
__device__ __forceinline__ void load_piece(int j, const GemmArgs &g, __amdgpu_buffer_rsrc_t ra,
                                           __amdgpu_buffer_rsrc_t rb, int row0, int col0, int kt, int tid,
                                           f32x4 (&sa)[T::A_PER_T], f32x4 (&sb)[T::SB])
{
    const int k0 = kt * T::BK;
    if (j < T::A_PER_T) {
        const int c = tid + j * T::THREADS;
        const int r = c / T::ACH, kc = c % T::ACH;
        const int gr = row0 + r, gk = k0 + kc * 4;
        if constexpr (!MASKED) {
            sa[j] = buf_load_x4(ra, elem_off(gr < g.m, gr, g.lda, gk));
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                sa[j][q] = buf_load_x1(ra, elem_off(gr < g.m && gk + q < g.k, gr, g.lda, gk + q));
        }
        return;
    }
    const int jb = j - T::A_PER_T;
    if constexpr (!B_COL) {
        const int c = tid + jb * T::THREADS;
        const int kr = c / T::BCH, nc = c % T::BCH;
        const int gk = k0 + kr, gn = col0 + nc * 4;
        if constexpr (!MASKED) {
            sb[jb] = buf_load_x4(rb, (uint32_t)(gk * g.ldb + gn) * 4u);
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                sb[jb][q] = buf_load_x1(rb, elem_off(gk < g.k && gn + q < g.n, gk, g.ldb, gn + q));
        }
    } else {
        const int i = jb >> 2, cc = jb & 3;
        const int u = tid + i * T::THREADS;
        if (T::B_MICRO % T::THREADS == 0 || u < T::B_MICRO) {
            const int kc = u % (T::BK / 4), ng = u / (T::BK / 4);
            const int gk = k0 + 4 * kc;
            const int gn = col0 + 4 * ng + cc;   // column of B, k-contiguous in HBM
            if constexpr (!MASKED) {
                sb[jb] = buf_load_x4(rb, elem_off(gn < g.n, gn, g.ldb, gk));
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    sb[jb][q] = buf_load_x1(rb, elem_off(gn < g.n && gk + q < g.k, gn, g.ldb, gk + q));
            }
        }
    }
}

// Register -> LDS piece j (column-major B: k-row q of micro-block i, built
// from the q-th element of its 4 column loads -- the corner turn).
template <class T, bool B_COL>
__device__ __forceinline__ void store_piece(int j, f32x4 *As, f32x4 *Bs, int tid,
                                            const f32x4 (&sa)[T::A_PER_T], const f32x4 (&sb)[T::SB])
{
    if (j < T::A_PER_T) {
        const int c = tid + j * T::THREADS;
        const int r = c / T::ACH, kc = c % T::ACH;
        As[r * T::ACH + (kc ^ swz_a<T::ACH>(r))] = sa[j];
        return;
    }
    const int jb = j - T::A_PER_T;
    if constexpr (!B_COL) {
        const int c = tid + jb * T::THREADS;
        const int kr = c / T::BCH, nc = c % T::BCH;
        Bs[kr * T::BCH + (nc ^ swz_b<T::BK>(kr))] = sb[jb];
    } else {
        const int i = jb >> 2, q = jb & 3;
        const int u = tid + i * T::THREADS;
        if (T::B_MICRO % T::THREADS == 0 || u < T::B_MICRO) {
            const int kc = u % (T::BK / 4), ng = u / (T::BK / 4);
            const int kr = 4 * kc + q;
            const f32x4 v = {sb[4 * i + 0][q], sb[4 * i + 1][q], sb[4 * i + 2][q], sb[4 * i + 3][q]};
            Bs[kr * T::BCH + (ng ^ swz_b<T::BK>(kr))] = v;
        }
    }
}

template <class T, bool B_COL, bool MASKED>
__device__ __forceinline__ void mfma_load_slab(const GemmArgs &g, __amdgpu_buffer_rsrc_t ra,
                                               __amdgpu_buffer_rsrc_t rb, int row0, int col0, int kt,
                                               int tid, f32x4 (&sa)[T::A_PER_T], f32x4 (&sb)[T::SB])
{
#pragma unroll
    for (int j = 0; j < Pieces<T, B_COL>::COUNT; ++j)
        load_piece<T, B_COL, MASKED>(j, g, ra, rb, row0, col0, kt, tid, sa, sb);
}

template <class T, bool B_COL>
__device__ __forceinline__ void mfma_store_slab(f32x4 *As, f32x4 *Bs, int tid, const f32x4 (&sa)[T::A_PER_T],
                                                const f32x4 (&sb)[T::SB])
{
#pragma unroll
    for (int j = 0; j < Pieces<T, B_COL>::COUNT; ++j) store_piece<T, B_COL>(j, As, Bs, tid, sa, sb);
}

// B values of one k-step for the NB blocks of a wavefront: NB adjacent floats.
template <int NB>
struct BFrag {
    float v[NB];
};

// A chunk q of the slab (k = half*KH + 4q .. +3) for the MB blocks.
template <class T>
__device__ __forceinline__ void read_a(const f32x4 *As, int wr, int l32, int half, int q,
                                       f32x4 (&af)[T::MB])
{
#pragma unroll
    for (int mb = 0; mb < T::MB; ++mb) {
        const int r = wr * T::WM + mb * 32 + l32;
        const int kc = half * T::AQ + q;
        af[mb] = As[r * T::ACH + (kc ^ swz_a<T::ACH>(r))];
    }
}

template <class T>
__device__ __forceinline__ void read_b(const f32x4 *Bs, int wc, int l32, int half, int p,
                                       BFrag<T::NB> &bf)
{
    const int kr = half * T::KH + p;
    const f32x4 *brow = Bs + kr * T::BCH;
    const int sw = swz_b<T::BK>(kr);
    if constexpr (T::NB == 4) {
        const f32x4 t = brow[(wc * (T::WN / 4) + l32) ^ sw];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) bf.v[nb] = t[nb];
    } else if constexpr (T::NB == 2) {
        const float *cp = reinterpret_cast<const float *>(brow + ((wc * (T::WN / 4) + (l32 >> 1)) ^ sw));
        const f32x2 t = *reinterpret_cast<const f32x2 *>(cp + 2 * (l32 & 1));
        bf.v[0] = t[0];
        bf.v[1] = t[1];
    } else {
        const float *cp = reinterpret_cast<const float *>(brow + ((wc * (T::WN / 4) + (l32 >> 2)) ^ sw));
        bf.v[0] = cp[l32 & 3];
    }
}

template <class T>
__device__ __forceinline__ void mfma_one(int i, const f32x4 (&af)[T::MB], int e, const BFrag<T::NB> &bf,
                                         f32x16 (&acc)[T::MB][T::NB])
{
    const int mb = i / T::NB, nb = i % T::NB;
    acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[mb][e], bf.v[nb], acc[mb][nb], 0, 0, 0);
}

template <class T>
__device__ __forceinline__ void mfma_step(const f32x4 (&af)[T::MB], int e, const BFrag<T::NB> &bf,
                                          f32x16 (&acc)[T::MB][T::NB])
{
#pragma unroll
    for (int mb = 0; mb < T::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < T::NB; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[mb][e], bf.v[nb], acc[mb][nb], 0, 0, 0);
}

// What one slab body does besides its MFMAs.
enum SlabLoad { LOAD_NONE = 0, LOAD_WHOLE = 1, LOAD_MASKED = 2 };

// Everything one wavefront needs while walking the slabs.
template <class T>
struct MfmaState {
    f32x16 acc[T::MB][T::NB];
    f32x4 sa[T::A_PER_T];      // staged global loads of a later slab
    f32x4 sb[T::SB];
    f32x4 af[2][T::MB];        // A chunk q of the current slab lives in af[q & 1]
    BFrag<T::NB> bf[2];        // B values of k-step p live in bf[p & 1]
};

// One slab kt: k-steps 0..KH-1 on LDS buffer kt&1, as an explicit schedule.
// At the top of k-step p the B values of step p+1 are read (and, every four
// steps, the next A chunk); then the step's MB*NB MFMAs issue.  From step
// STORE_STEP on, one staging piece follows every second MFMA: first the LDS
// writes of slab kt+1 into the other buffer (STORE), then the global loads of
// slab kt+2 (LOAD), so LDS and global traffic trickle between MFMAs instead
// of arriving as a burst.  The barrier sits before the last k-step; after it
// the first fragments of slab kt+1 are read (NEXT) while that step's MFMAs
// run.  sched_barrier fences keep this order through the scheduler.
template <class T, bool B_COL, int LOAD, bool STORE, bool NEXT>
__device__ __forceinline__ void mfma_slab(const GemmArgs &g, f32x4 *lds_a, f32x4 *lds_b,
                                          __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                          int row0, int col0, int kt, int tid, int wr, int wc, int l32,
                                          int half, MfmaState<T> &st)
{
    constexpr int NM = T::MB * T::NB;                         // MFMAs per k-step
    constexpr int NP = Pieces<T, B_COL>::COUNT;
    constexpr int W = STORE ? NP : 0;                         // LDS writes this slab
    constexpr int L = LOAD != LOAD_NONE ? NP : 0;             // global loads this slab
    constexpr int SLOTS = (T::KH - 1) * NM - T::STORE_STEP * NM;
    constexpr int GAP = (W + L) == 0 ? 1 : (2 * (W + L) <= SLOTS ? 2 : 1);
    constexpr int T0 = T::STORE_STEP * NM;                    // first MFMA of the store step
    static_assert(W + L <= SLOTS, "staging pieces fit before the barrier");

    const int cur = kt & 1, nxt = cur ^ 1;
    const f32x4 *As = lds_a + cur * T::A_CHUNKS;
    const f32x4 *Bs = lds_b + cur * T::B_CHUNKS;
    f32x4 *As_n = lds_a + nxt * T::A_CHUNKS;
    f32x4 *Bs_n = lds_b + nxt * T::B_CHUNKS;
#pragma unroll
    for (int p = 0; p < T::KH - 1; ++p) {
        read_b<T>(Bs, wc, l32, half, p + 1, st.bf[(p + 1) & 1]);
        if ((p & 3) == 1 && (p >> 2) + 1 < T::AQ)
            read_a<T>(As, wr, l32, half, (p >> 2) + 1, st.af[((p >> 2) + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            mfma_one<T>(i, st.af[(p >> 2) & 1], p & 3, st.bf[p & 1], st.acc);
            const int t = p * NM + i - T0;                    // MFMA slot from the store step on
            if (t >= 0 && (t + 1) % GAP == 0) {
                const int piece = (t + 1) / GAP - 1;
                if (piece < W) {
                    store_piece<T, B_COL>(piece, As_n, Bs_n, tid, st.sa, st.sb);
                } else if (piece < W + L) {
                    if constexpr (LOAD == LOAD_WHOLE)
                        load_piece<T, B_COL, false>(piece - W, g, ra, rb, row0, col0, kt + 2, tid, st.sa, st.sb);
                    if constexpr (LOAD == LOAD_MASKED)
                        load_piece<T, B_COL, true>(piece - W, g, ra, rb, row0, col0, kt + 2, tid, st.sa, st.sb);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    __syncthreads();
    if constexpr (NEXT) {
        read_a<T>(As_n, wr, l32, half, 0, st.af[0]);
        read_b<T>(Bs_n, wc, l32, half, 0, st.bf[0]);
    }
    mfma_step<T>(st.af[((T::KH - 1) >> 2) & 1], (T::KH - 1) & 3, st.bf[(T::KH - 1) & 1], st.acc);
}

template <class T, bool B_COL>
__global__ __launch_bounds__(T::THREADS) void gemm_mfma_kernel(GemmArgs g)
{
    __shared__ f32x4 lds[2 * (T::A_CHUNKS + T::B_CHUNKS)];
    f32x4 *const lds_a = lds;                      // [2][A_CHUNKS]
    f32x4 *const lds_b = lds + 2 * T::A_CHUNKS;    // [2][B_CHUNKS]

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wr = wave % T::WAVES_M, wc = wave / T::WAVES_M;
    const int l32 = lane & 31, half = lane >> 5;
    if (g.poison_lds) poison_lds(lds, 2 * (T::A_CHUNKS + T::B_CHUNKS), tid, T::THREADS);

    int tm, tn;
    raster_tile(blockIdx.x, g, tm, tn);
    const int row0 = tm * T::BM, col0 = tn * T::BN;

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.A, g.a_bytes);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(g.B, g.b_bytes);
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(g.C, g.c_bytes);

    MfmaState<T> st;
#pragma unroll
    for (int mb = 0; mb < T::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < T::NB; ++nb) st.acc[mb][nb] = f32x16{};

    // Slabs 0 .. KT-2 load whole 16-byte chunks; the last slab loads element
    // by element (so does every slab when the plan asks for it).
    const int kt_count = g.k_tiles;
    const bool whole = !g.masked_loads;

    // Prologue: slab 0 into buffer 0, slab 1 staged in registers, fragments
    // of slab 0 step 0 in registers.
    if (kt_count > 1 && whole)
        mfma_load_slab<T, B_COL, false>(g, ra, rb, row0, col0, 0, tid, st.sa, st.sb);
    else
        mfma_load_slab<T, B_COL, true>(g, ra, rb, row0, col0, 0, tid, st.sa, st.sb);
    mfma_store_slab<T, B_COL>(lds_a, lds_b, tid, st.sa, st.sb);
    __syncthreads();
    if (kt_count > 2 && whole)
        mfma_load_slab<T, B_COL, false>(g, ra, rb, row0, col0, 1, tid, st.sa, st.sb);
    else if (kt_count > 1)
        mfma_load_slab<T, B_COL, true>(g, ra, rb, row0, col0, 1, tid, st.sa, st.sb);
    read_a<T>(lds_a, wr, l32, half, 0, st.af[0]);
    read_b<T>(lds_b, wc, l32, half, 0, st.bf[0]);

    // Steady state: slab kt+2 exists and is not the last one.
    int kt = 0;
    if (whole) {
        for (; kt + 3 < kt_count; ++kt)
            mfma_slab<T, B_COL, LOAD_WHOLE, true, true>(g, lds_a, lds_b, ra, rb, row0, col0, kt, tid, wr, wc,
                                                        l32, half, st);
    } else {
        for (; kt + 3 < kt_count; ++kt)
            mfma_slab<T, B_COL, LOAD_MASKED, true, true>(g, lds_a, lds_b, ra, rb, row0, col0, kt, tid, wr, wc,
                                                         l32, half, st);
    }
    // Tail: the slab that loads the last slab, then the last two slabs.
    if (kt + 3 == kt_count) {
        mfma_slab<T, B_COL, LOAD_MASKED, true, true>(g, lds_a, lds_b, ra, rb, row0, col0, kt, tid, wr, wc,
                                                     l32, half, st);
        ++kt;
    }
    if (kt + 2 == kt_count) {
        mfma_slab<T, B_COL, LOAD_NONE, true, true>(g, lds_a, lds_b, ra, rb, row0, col0, kt, tid, wr, wc, l32,
                                                   half, st);
        ++kt;
    }
    mfma_slab<T, B_COL, LOAD_NONE, false, false>(g, lds_a, lds_b, ra, rb, row0, col0, kt, tid, wr, wc, l32,
                                                 half, st);

    // Epilogue: lane (l32, half), accumulator element v of block (mb, nb) is
    // C row  mb*32 + 8*(v/4) + 4*half + v%4  and column  NB*l32 + nb  of the
    // wavefront tile.  C is overwritten; rows >= m and columns >= n are not
    // written (row padding of C included).  Interior tiles store without
    // checks (uniform branch).
    const int cb = col0 + wc * T::WN + T::NB * l32;
    const bool interior = row0 + T::BM <= g.m && col0 + T::BN <= g.n;
#pragma unroll
    for (int mb = 0; mb < T::MB; ++mb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int r = row0 + wr * T::WM + mb * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
            if (interior) {
                if constexpr (T::NB == 4) {
                    const f32x4 out = {st.acc[mb][0][v], st.acc[mb][1][v], st.acc[mb][2][v], st.acc[mb][3][v]};
                    buf_store_x4(out, rc, (uint32_t)(r * g.ldc + cb) * 4u);
                } else {
#pragma unroll
                    for (int nb = 0; nb < T::NB; ++nb)
                        buf_store_x1(st.acc[mb][nb][v], rc, (uint32_t)(r * g.ldc + cb + nb) * 4u);
                }
            } else {
#pragma unroll
                for (int nb = 0; nb < T::NB; ++nb)
                    buf_store_x1(st.acc[mb][nb][v], rc, elem_off(r < g.m && cb + nb < g.n, r, g.ldc, cb + nb));
            }
        }
    }
}

}  // namespace gemmf32

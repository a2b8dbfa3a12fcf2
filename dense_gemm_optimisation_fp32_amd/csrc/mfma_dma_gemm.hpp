// FP32 GEMM on the gfx950 matrix cores with direct global -> LDS loads.
//
// Same wavefront tiles, k order and MFMA (v_mfma_f32_32x32x2_f32) as
// mfma_gemm.hpp, but the operands travel from HBM straight into LDS with
// buffer_load_dwordx4 ... lds (the gfx950 analogue of the asynchronous copy of
// "GEMM 性能优化", 台阶 7): no staging registers and no LDS write
// instructions, so the matrix cores are not interrupted by the copy, and a
// ring of STAGES LDS buffers lets the loads of slab kt+STAGES-1 fly while slab
// kt is computed (the N-stage generalisation of 台阶 6's double buffer).
//
// The DMA writes lane i's 16 bytes at the wavefront's LDS base + 16*i, so a
// layout is chosen by choosing which global chunk each lane fetches:
//   * A:  As[r][c ^ swz_a(r)], k-contiguous rows of BK (as in mfma_gemm.hpp).
//   * B row-major: Bs[kr][nc], n-contiguous k-rows of BN; the fragment read of
//     a k-step is one 16-byte read covering the NB interleaved columns
//     (C column NB*j + nb of the wavefront tile for lane column j).
//   * B column-major: Bs[n][c ^ swz_a(n)], k-contiguous like A -- the tile is
//     copied in its HBM orientation and the corner turn happens in the
//     fragment read, which fetches four consecutive k of one column per lane
//     ("PMPP Chapter 06", section 1: the unfavourable access pattern moves to
//     on-chip memory).  Columns are block-major here (C column nb*32 + j).
//
// Column-major A (A[i][k] at A[k*lda + i]) is the mirror image of row-major
// B: the tile lands m-contiguous, As_t[kr][mc], and one 16-byte read of a
// k-row gives the A values of one k-step for the MB interleaved blocks (tile
// row MB*l32 + mb of the wavefront tile for lane row l32 of block mb).
//
// The slab body is an explicit schedule: straight-line code fenced with
// sched_barrier, one copy after every two MFMAs, the MFMA section optionally
// at a raised wavefront priority (s_setprio), then a wait that leaves the
// copies of the later slabs in flight and a bare s_barrier (ring_barrier).
//
// Range checking is per 4-byte element: a chunk that straddles an operand's
// byte extent keeps its in-range elements and reads zeros past the end, rows
// of A (columns of column-major B) past m (n) get the out-of-range offset and
// read as zero, and columns of row-major B past n only feed columns of C that
// are never stored.  What remains is the k tail: elements k >= K of the last
// slab that lie inside the operand (row padding, or the start of the next
// row).  After that slab's copy lands, each lane zeroes those elements of the
// chunks it fetched (A and column-major B; row-major B's k-rows >= K are past
// its extent and already zero).
#pragma once

#include "epilogue.hpp"
#include "mfma_gemm.hpp"

namespace gemmf32 {

// PRIO: raise the wavefront priority for the matrix-core part of each slab.
// Measured at 4096^3: +0.4-0.8 % with 256x128 tiles (two workgroups per CU)
// and 64x64 tiles, but 128x128 tiles with three workgroups per CU lose 18 %
// with it (115.8 against 142.0 TFLOPS), so those variants leave it off.
template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int STAGES_, bool PRIO_ = true>
struct DmaTile : MfmaTile<BM_, BN_, BK_, WAVES_M_, WAVES_N_> {
    using Base = MfmaTile<BM_, BN_, BK_, WAVES_M_, WAVES_N_>;
    static constexpr int STAGES = STAGES_;
    static constexpr bool PRIO = PRIO_;
    static constexpr int PIECES = Base::A_PER_T + Base::B_PER_T;   // 16-byte copies per lane per slab
    static constexpr int LDS_BYTES = STAGES * (Base::A_CHUNKS + Base::B_CHUNKS) * 16;
    static_assert(STAGES >= 2 && STAGES <= 4, "2 to 4 LDS stages");
    static_assert(LDS_BYTES <= 160 * 1024, "fits the 160 KB LDS of a CU");
    static_assert((STAGES - 2) * PIECES <= 63, "outstanding copies fit the vmcnt counter");
};

typedef __attribute__((address_space(3))) void *lds_ptr_t;

// One 16-byte global -> LDS copy for wavefront-uniform LDS chunk `wave_chunk`
// (lane i lands at wave_chunk + i).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, f32x4 *wave_chunk)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)wave_chunk, 16, (int)byte_off, 0, 0, 0);
}

// Global element (row, k-chunk) of piece j, and the LDS chunk it lands in.
template <class T, bool B_COL>
struct DmaPiece {
    int lds_chunk;   // chunk index inside the operand's stage region
    bool is_a;
    int row;         // A row / B k-row (row-major) / B column (column-major) inside the tile
    int kc;          // logical 16-byte k-chunk (A and column-major B), n-chunk for row-major B
};

template <class T, bool B_COL, bool A_COL = false>
__device__ __forceinline__ DmaPiece<T, B_COL> dma_piece(int j, int tid)
{
    DmaPiece<T, B_COL> d;
    if (j < T::A_PER_T) {
        const int c = tid + j * T::THREADS;
        d.lds_chunk = c;
        d.is_a = true;
        if constexpr (A_COL) {
            d.row = c / (T::BM / 4);     // k-row
            d.kc = c % (T::BM / 4);      // m-chunk
        } else {
            d.row = c / T::ACH;
            d.kc = (c % T::ACH) ^ swz_a<T::ACH>(d.row);
        }
    } else {
        const int c = tid + (j - T::A_PER_T) * T::THREADS;
        d.lds_chunk = c;
        d.is_a = false;
        if constexpr (!B_COL) {
            d.row = c / T::BCH;
            d.kc = c % T::BCH;
        } else {
            d.row = c / T::ACH;
            d.kc = (c % T::ACH) ^ swz_a<T::ACH>(d.row);
        }
    }
    return d;
}

// Per-lane global offsets of a tile's copies at slab 0, computed once per
// tile; a slab adds a uniform k term (no per-copy multiply).  Pieces whose
// rows run along k (column-major A, row-major B) add k0 * ld and drop rows
// at or past K (only the tail slab has any; their offsets could also wrap);
// pieces whose 16-byte chunks run along k (row-major A, column-major B) add
// k0 and carry the out-of-range offset for rows past M (columns past N),
// which stays out of range after the add.
template <class T, bool B_COL, bool A_COL = false>
struct DmaBases {
    uint32_t off[T::PIECES];
};

template <class T, bool B_COL, bool A_COL = false>
__device__ __forceinline__ DmaBases<T, B_COL, A_COL> dma_bases(const GemmArgs &g, int row0, int col0, int tid)
{
    DmaBases<T, B_COL, A_COL> b;
#pragma unroll
    for (int j = 0; j < T::PIECES; ++j) {
        const DmaPiece<T, B_COL> d = dma_piece<T, B_COL, A_COL>(j, tid);
        if (A_COL && d.is_a) {
            // (wraps harmlessly for rows at or past K, which are dropped)
            b.off[j] = ((uint32_t)d.row * (uint32_t)g.lda + (uint32_t)(row0 + 4 * d.kc)) * 4u;
        } else if (d.is_a) {
            const int gr = row0 + d.row;
            b.off[j] = elem_off(gr < g.m, gr, g.lda, 4 * d.kc);
        } else if (!B_COL) {
            b.off[j] = ((uint32_t)d.row * (uint32_t)g.ldb + (uint32_t)(col0 + 4 * d.kc)) * 4u;
        } else {
            const int gn = col0 + d.row;
            b.off[j] = elem_off(gn < g.n, gn, g.ldb, 4 * d.kc);
        }
    }
    return b;
}

// KCHECK: drop the k-rows at or past K (needed only for the last slab when
// K is not a multiple of BK; every other slab's k-rows are all below K).
template <class T, bool B_COL, bool A_COL = false, bool KCHECK = true>
__device__ __forceinline__ void dma_issue(int j, const GemmArgs &g, const DmaBases<T, B_COL, A_COL> &bases,
                                          __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb, int kt, int tid,
                                          int wave, f32x4 *As, f32x4 *Bs)
{
    const DmaPiece<T, B_COL> d = dma_piece<T, B_COL, A_COL>(j, tid);
    const int k0 = kt * T::BK;
    const int wave_base = (j < T::A_PER_T ? j : j - T::A_PER_T) * T::THREADS + wave * 64;
    const bool krows = d.is_a ? A_COL : !B_COL;      // rows of the piece run along k
    uint32_t off;
    if (krows) {
        const int ld = d.is_a ? g.lda : g.ldb;
        off = (!KCHECK || d.row < g.k - k0) ? bases.off[j] + (uint32_t)(k0 * ld) * 4u : kOobOffset;
    } else {
        off = bases.off[j] + (uint32_t)k0 * 4u;
    }
    dma16(d.is_a ? ra : rb, off, d.is_a ? As + wave_base : Bs + wave_base);
}

// Zero the elements k >= K of this lane's chunks of the last slab (A and
// column-major B).  Runs after the lane's copies of that slab have landed.
template <class T, bool B_COL, bool A_COL = false>
__device__ __forceinline__ void dma_fix_tail(const GemmArgs &g, int kt, int tid, f32x4 *As, f32x4 *Bs)
{
    const int k0 = kt * T::BK;
#pragma unroll
    for (int j = 0; j < T::PIECES; ++j) {
        const DmaPiece<T, B_COL> d = dma_piece<T, B_COL, A_COL>(j, tid);
        if (d.is_a ? A_COL : !B_COL) continue;   // k-rows past K already read as zero
        float *p = reinterpret_cast<float *>((d.is_a ? As : Bs) + d.lds_chunk);
        const int gk = k0 + 4 * d.kc;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (gk + q >= g.k) p[q] = 0.0f;
    }
}

// vmcnt wait with every other counter left alone (gfx9 encoding: vmcnt bits
// 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// The slab ring's workgroup barrier: this wavefront's LDS reads and writes
// complete and at most N of its copies still in flight, then s_barrier.
// __syncthreads() would add a workgroup-scope release fence, and since the
// copies write LDS through the vector memory counter the fence waits for all
// of them (vmcnt(0)), copies of the slab after next included: the ring then
// drains every slab.  The "memory" clobber keeps the compiler from moving LDS
// accesses across the barrier; the explicit counts give the ordering the
// fence would: the next slab's copies have landed (vmcnt), and no LDS read of
// the stage about to be refilled is still pending (lgkmcnt(0)).
template <int N>
__device__ __forceinline__ void ring_barrier()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
    asm volatile("s_barrier" ::: "memory");
}

// How many k-steps ahead of its first use a fragment is read from LDS.  One
// step is enough for most tile/layout pairs; two paid where both operands
// are read one k-step at a time or the CU runs three workgroups (4096^3, one
// MI355X, distance 1 -> 2: 256x128 with column-major A and row-major B 139.0
// -> 142.5 TFLOPS, 128x128 row-major 140.7 -> 142.6).  Elsewhere two steps
// measured the same within 0.5 %, or slower (256x128 row-major 145.7 ->
// 144.5, 128x128 with column-major B 127 -> 119.5), so they keep one.
template <class T, bool B_COL, bool A_COL>
constexpr int prefetch_distance()
{
    return ((T::BM == 256 && T::BN == 128 && A_COL && !B_COL) || (T::BM == 128 && T::BN == 128 && !A_COL && !B_COL))
               ? 2
               : 1;
}

// Fragments of one wavefront for one slab.  A (and column-major B) come as
// 16-byte k-chunks, double-buffered per chunk (a chunk covers four k-steps,
// more than the prefetch distance); row-major B and column-major A as one
// read per k-step, in a ring of 2 x distance registers sets (so that a slab
// of KH = 8 k-steps maps each k-step to the same set in every slab).
template <class T, bool B_COL, bool A_COL = false>
struct DmaFrags {
    static constexpr int D = prefetch_distance<T, B_COL, A_COL>();
    static constexpr int FB = 2 * D;
    static_assert(T::KH % FB == 0 && D <= 4, "k-step ring and chunk buffers");
    f32x4 af[2][T::MB];
    f32x4 bk[2][T::NB];        // column-major B: k-chunk q of block nb in bk[q & 1][nb]
    BFrag<T::NB> bf[FB];       // row-major B: k-step p in bf[p % FB]
    BFrag<T::MB> am[FB];       // column-major A: k-step p in am[p % FB]
};

template <class T>
__device__ __forceinline__ void read_bk(const f32x4 *Bs, int wc, int l32, int half, int q, f32x4 (&bk)[T::NB])
{
#pragma unroll
    for (int nb = 0; nb < T::NB; ++nb) {
        const int n = wc * T::WN + nb * 32 + l32;
        const int kc = half * T::AQ + q;
        bk[nb] = Bs[n * T::ACH + (kc ^ swz_a<T::ACH>(n))];
    }
}

// Row-major B without a swizzle (the copy lands n-contiguous).
template <class T>
__device__ __forceinline__ void read_bn(const f32x4 *Bs, int wc, int l32, int half, int p, BFrag<T::NB> &bf)
{
    const int kr = half * T::KH + p;
    const f32x4 *brow = Bs + kr * T::BCH;
    if constexpr (T::NB == 4) {
        const f32x4 t = brow[wc * (T::WN / 4) + l32];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) bf.v[nb] = t[nb];
    } else if constexpr (T::NB == 2) {
        const float *cp = reinterpret_cast<const float *>(brow + wc * (T::WN / 4) + (l32 >> 1));
        const f32x2 t = *reinterpret_cast<const f32x2 *>(cp + 2 * (l32 & 1));
        bf.v[0] = t[0];
        bf.v[1] = t[1];
    } else {
        const float *cp = reinterpret_cast<const float *>(brow + wc * (T::WN / 4) + (l32 >> 2));
        bf.v[0] = cp[l32 & 3];
    }
}

// Column-major A without a swizzle (the copy lands m-contiguous).
template <class T>
__device__ __forceinline__ void read_am(const f32x4 *As, int wr, int l32, int half, int p, BFrag<T::MB> &af)
{
    const int kr = half * T::KH + p;
    const f32x4 *arow = As + kr * (T::BM / 4);
    if constexpr (T::MB == 4) {
        const f32x4 t = arow[wr * (T::WM / 4) + l32];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) af.v[mb] = t[mb];
    } else if constexpr (T::MB == 2) {
        const float *cp = reinterpret_cast<const float *>(arow + wr * (T::WM / 4) + (l32 >> 1));
        const f32x2 t = *reinterpret_cast<const f32x2 *>(cp + 2 * (l32 & 1));
        af.v[0] = t[0];
        af.v[1] = t[1];
    } else {
        const float *cp = reinterpret_cast<const float *>(arow + wr * (T::WM / 4) + (l32 >> 2));
        af.v[0] = cp[l32 & 3];
    }
}

template <class T, bool B_COL, bool A_COL = false>
__device__ __forceinline__ void dma_mfma_one(int i, int p, const DmaFrags<T, B_COL, A_COL> &f,
                                             f32x16 (&acc)[T::MB][T::NB])
{
    const int mb = i / T::NB, nb = i % T::NB;
    constexpr int FB = DmaFrags<T, B_COL, A_COL>::FB;
    const float a = A_COL ? f.am[p % FB].v[mb] : f.af[(p >> 2) & 1][mb][p & 3];
    float b;
    if constexpr (B_COL) b = f.bk[(p >> 2) & 1][nb][p & 3];
    else b = f.bf[p % FB].v[nb];
    acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[mb][nb], 0, 0, 0);
}

// Reads for k-step p_next: issued in k-step p_next - D (at its top, or
// after its first MFMA), or after the barrier for the first D k-steps of
// the next slab.
template <class T, bool B_COL, bool A_COL = false>
__device__ __forceinline__ void dma_prefetch(int p_next, const f32x4 *As, const f32x4 *Bs, int wr, int wc, int l32,
                                             int half, DmaFrags<T, B_COL, A_COL> &f)
{
    if ((p_next & 3) == 0) {
        const int q = p_next >> 2;
        if constexpr (!A_COL) read_a<T>(As, wr, l32, half, q, f.af[q & 1]);
        if constexpr (B_COL) read_bk<T>(Bs, wc, l32, half, q, f.bk[q & 1]);
    }
    constexpr int FB = DmaFrags<T, B_COL, A_COL>::FB;
    if constexpr (A_COL) read_am<T>(As, wr, l32, half, p_next, f.am[p_next % FB]);
    if constexpr (!B_COL) read_bn<T>(Bs, wc, l32, half, p_next, f.bf[p_next % FB]);
}

// One slab kt on stage kt % STAGES.  copy: issue the copies of slab
// kt + STAGES - 1 (one per two MFMAs from the start of the slab; uniform
// flag).  WAIT: the vmcnt allowance when waiting for slab kt+1's copies at the
// end (-1: slab kt is the last one).  fix: zero the k tail of slab kt+1 after
// it lands (uniform flag).  The barrier precedes the last D k-steps (D = the
// prefetch distance), whose MFMAs cover the first LDS reads of slab kt+1.
template <class T, bool B_COL, int WAIT, bool A_COL = false, bool KCHECK = true>
__device__ __forceinline__ void dma_slab(const GemmArgs &g, f32x4 *lds_a, f32x4 *lds_b, __amdgpu_buffer_rsrc_t ra,
                                         __amdgpu_buffer_rsrc_t rb, const DmaBases<T, B_COL, A_COL> &bases,
                                         int kt, bool copy, bool fix,
                                         int tid, int wave, int wr, int wc, int l32, int half,
                                         DmaFrags<T, B_COL, A_COL> &f, f32x16 (&acc)[T::MB][T::NB])
{
    constexpr int NM = T::MB * T::NB;
    constexpr int D = DmaFrags<T, B_COL, A_COL>::D;
    constexpr int GAP = 2 * T::PIECES <= (T::KH - D) * NM ? 2 : 1;
    static_assert(T::PIECES * GAP <= (T::KH - D) * NM, "copies fit before the barrier");
    const int cur = kt % T::STAGES;
    const int nxt = (kt + 1) % T::STAGES;
    const int cpy = (kt + T::STAGES - 1) % T::STAGES;
    const f32x4 *As = lds_a + cur * T::A_CHUNKS;
    const f32x4 *Bs = lds_b + cur * T::B_CHUNKS;
    // With PRIO the matrix-core part of the slab issues at a raised priority
    // and the wait for the next slab and the barrier at the normal one, so a
    // wavefront that is ready to multiply goes ahead of one about to wait.
    if constexpr (T::PRIO) __builtin_amdgcn_s_setprio(1);
    // With four or more MFMAs per k-step the reads for k-step p + D go out
    // after the step's first MFMA: that MFMA then waits only for reads
    // issued a whole k-step earlier (issued before it, the read for the
    // next step is caught by the in-order LDS counter wait as well).  With
    // one or two MFMAs per step the reads go first, so that both MFMAs
    // cover them.
    constexpr bool READ_AFTER_FIRST = NM >= 4;
#pragma unroll
    for (int p = 0; p < T::KH - D; ++p) {
        if constexpr (!READ_AFTER_FIRST) {
            dma_prefetch<T, B_COL, A_COL>(p + D, As, Bs, wr, wc, l32, half, f);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            dma_mfma_one<T, B_COL, A_COL>(i, p, f, acc);
            if (READ_AFTER_FIRST && i == 0) {
                __builtin_amdgcn_sched_barrier(0);
                dma_prefetch<T, B_COL, A_COL>(p + D, As, Bs, wr, wc, l32, half, f);
            }
            const int t = p * NM + i;
            if ((t + 1) % GAP == 0 && (t + 1) / GAP - 1 < T::PIECES && copy)
                dma_issue<T, B_COL, A_COL, KCHECK>((t + 1) / GAP - 1, g, bases, ra, rb, kt + T::STAGES - 1, tid,
                                                   wave, lds_a + cpy * T::A_CHUNKS, lds_b + cpy * T::B_CHUNKS);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    if constexpr (T::PRIO) __builtin_amdgcn_s_setprio(0);
    if constexpr (WAIT >= 0) {
        wait_vmcnt<WAIT>();
        if (fix) dma_fix_tail<T, B_COL, A_COL>(g, kt + 1, tid, lds_a + nxt * T::A_CHUNKS, lds_b + nxt * T::B_CHUNKS);
    }
    // (WAIT < 0: no copies of this range remain; the barrier only orders the
    // LDS reads before the next range's copies.)
    ring_barrier<(WAIT < 0 ? 63 : WAIT)>();
    // Fenced: left alone the scheduler moved most of these MFMAs ahead of
    // the reads (one even above the barrier), and the next slab's first
    // MFMA waited for LDS.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int d = 0; d < D; ++d) {
        if constexpr (WAIT >= 0)
            dma_prefetch<T, B_COL, A_COL>(d, lds_a + nxt * T::A_CHUNKS, lds_b + nxt * T::B_CHUNKS, wr, wc, l32, half,
                                          f);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NM; ++i) dma_mfma_one<T, B_COL, A_COL>(i, T::KH - D + d, f, acc);
    }
}

// Slabs [kt0, kt1) of one tile, accumulated into acc.  The ring stage of
// slab kt is kt % STAGES.  Every LDS read of the range happens before its
// last barrier, so the next range may start copying at once.
template <class T, bool B_COL, bool A_COL = false>
__device__ __forceinline__ void dma_range(const GemmArgs &g, f32x4 *lds_a, f32x4 *lds_b, __amdgpu_buffer_rsrc_t ra,
                                          __amdgpu_buffer_rsrc_t rb, int row0, int col0, int kt0, int kt1, int tid,
                                          int wave, int wr, int wc, int l32, int half,
                                          f32x16 (&acc)[T::MB][T::NB])
{
    const int KT = g.k_tiles;
    const bool ktail = g.k % T::BK != 0;
    DmaFrags<T, B_COL, A_COL> f;
    const DmaBases<T, B_COL, A_COL> bases = dma_bases<T, B_COL, A_COL>(g, row0, col0, tid);

    // Prologue: copies of slabs kt0 .. kt0+STAGES-2, wait for slab kt0.
#pragma unroll
    for (int s = 0; s < T::STAGES - 1; ++s)
        if (kt0 + s < kt1) {
            const int st = (kt0 + s) % T::STAGES;
#pragma unroll
            for (int j = 0; j < T::PIECES; ++j)
                dma_issue<T, B_COL, A_COL>(j, g, bases, ra, rb, kt0 + s, tid, wave, lds_a + st * T::A_CHUNKS,
                                    lds_b + st * T::B_CHUNKS);
        }
    // Wait for slab kt0's copies only: those of the later prologue slabs
    // were issued after them and may stay in flight.
    const int st0 = kt0 % T::STAGES;
    const int n_pro = kt1 - kt0 < T::STAGES - 1 ? kt1 - kt0 : T::STAGES - 1;
    if (n_pro == 1) {
        wait_vmcnt<0>();
        if (kt0 + 1 == kt1 && kt1 == KT && ktail)
            dma_fix_tail<T, B_COL, A_COL>(g, kt0, tid, lds_a + st0 * T::A_CHUNKS, lds_b + st0 * T::B_CHUNKS);
        ring_barrier<0>();
    } else if (T::STAGES >= 4 && n_pro == 3) {
        ring_barrier<(T::STAGES >= 4 ? 2 : 0) * T::PIECES>();
    } else {
        ring_barrier<T::PIECES>();
    }
#pragma unroll
    for (int d = 0; d < DmaFrags<T, B_COL, A_COL>::D; ++d)
        dma_prefetch<T, B_COL, A_COL>(d, lds_a + st0 * T::A_CHUNKS, lds_b + st0 * T::B_CHUNKS, wr, wc, l32, half, f);

    // Steady state: slab kt+1 is not the last one and slab kt+STAGES-1
    // exists, so STAGES-2 slabs' copies may stay in flight while waiting for
    // slab kt+1; first while the slab being copied lies wholly below K (no
    // k check on the copies), then for the copy of a partial last slab.
    // Then the drain: copies only while slabs remain, every wait complete,
    // the k tail fixed when slab kt+1 is the tile's last.
    int kt = kt0;
    const int unchecked_end = ktail ? KT - 1 : KT;   // slabs below this copy without a k check
    for (; kt + T::STAGES - 1 < kt1 && kt + 2 < kt1 && kt + T::STAGES - 1 < unchecked_end; ++kt)
        dma_slab<T, B_COL, (T::STAGES - 2) * T::PIECES, A_COL, false>(g, lds_a, lds_b, ra, rb, bases, kt, true,
                                                                      false, tid, wave, wr, wc, l32, half, f, acc);
    for (; kt + T::STAGES - 1 < kt1 && kt + 2 < kt1; ++kt)
        dma_slab<T, B_COL, (T::STAGES - 2) * T::PIECES, A_COL>(g, lds_a, lds_b, ra, rb, bases, kt, true, false, tid,
                                                         wave, wr, wc, l32, half, f, acc);
    for (; kt + 1 < kt1; ++kt)
        dma_slab<T, B_COL, 0, A_COL>(g, lds_a, lds_b, ra, rb, bases, kt, kt + T::STAGES - 1 < kt1,
                              ktail && kt + 2 == KT, tid, wave, wr, wc, l32, half, f, acc);
    dma_slab<T, B_COL, -1, A_COL>(g, lds_a, lds_b, ra, rb, bases, kt, false, false, tid, wave, wr, wc, l32, half, f,
                           acc);
}

// Accumulators -> C.  Lane (l32, half), element v of block (mb, nb) is row
// i = 8*(v/4) + 4*half + v%4 of the block: tile row mb*32 + i of the
// wavefront tile (row-major A) or MB*i + mb (column-major A, interleaved
// rows); its column is NB*l32 + nb (row-major B) or nb*32 + l32
// (column-major B).  Range-checked stores.  Column-major B: per
// instruction, 32 lanes write one 128-byte row segment.  Row-major B: lane
// l32 holds the NB adjacent columns NB*l32 .. NB*l32+NB-1 of each row; with
// WIDE (a separate kernel, chosen by the plan when N is a multiple of NB, so
// that no group straddles column N) they go out as one 8- or 16-byte store,
// 32 lanes covering NB*128 contiguous bytes, else one store per element.
// At 4096^3 the 8-byte stores cut the store phase (64 MB of C) from 15.3 to
// 10.6 us and the launch by 0.45 %.  The choice is a template parameter, not
// a branch: with both store loops in one kernel the register allocator moved
// the accumulators around (256x128: 166 VGPRs, one workgroup per CU; 256x256
// spilled).
//
// EPI: the linear-layer epilogue act(alpha * acc + beta * C + bias[col]),
// with C read only when beta != 0.  The C values of one block are loaded
// together before any is used, so the epilogue pays one memory latency per
// block.
template <class T, bool B_COL, bool A_COL = false, bool EPI = false, bool WIDE = false>
__device__ __forceinline__ void dma_store_c(const GemmArgs &g, __amdgpu_buffer_rsrc_t rc, int row0, int col0, int wr,
                                            int wc, int l32, int half, const f32x16 (&acc)[T::MB][T::NB])
{
    auto row_of = [&](int mb, int v) {
        const int i = 8 * (v >> 2) + 4 * half + (v & 3);
        return row0 + wr * T::WM + (A_COL ? T::MB * i + mb : mb * 32 + i);
    };
    auto col_of = [&](int nb) {
        return B_COL ? col0 + wc * T::WN + nb * 32 + l32 : col0 + wc * T::WN + T::NB * l32 + nb;
    };
    static_assert(!WIDE || (!B_COL && (T::NB == 2 || T::NB == 4)), "wide stores: row-major B, NB of 2 or 4");
    if constexpr (WIDE && !EPI) {
#pragma unroll
        for (int mb = 0; mb < T::MB; ++mb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = row_of(mb, v);
                const int c = col_of(0);
                const uint32_t off = elem_off(r < g.m && c < g.n, r, g.ldc, c);
                if constexpr (T::NB == 2)
                    buf_store_x2(acc[mb][0][v], acc[mb][1][v], rc, off);
                else
                    buf_store_x4(f32x4{acc[mb][0][v], acc[mb][1][v], acc[mb][2][v], acc[mb][3][v]}, rc, off);
            }
    } else if constexpr (!EPI) {
#pragma unroll
        for (int mb = 0; mb < T::MB; ++mb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = row_of(mb, v);
#pragma unroll
                for (int nb = 0; nb < T::NB; ++nb) {
                    const int c = col_of(nb);
                    buf_store_x1(acc[mb][nb][v], rc, elem_off(r < g.m && c < g.n, r, g.ldc, c));
                }
            }
    } else if constexpr (WIDE) {
        // As below, NB adjacent columns per load and store (N a multiple of
        // NB, so the group is inside the row when its first column is).
        const __amdgpu_buffer_rsrc_t rbias = make_rsrc(g.bias, g.bias ? (uint32_t)g.n * 4u : 0u);
        const float lo = g.act == 1 ? 0.0f : -__builtin_inff();
        const bool gelu = g.act == 2;
        const int c = col_of(0);
        float bias[T::NB];
        if constexpr (T::NB == 2) {
            const f32x2 t = buf_load_x2(rbias, elem_off(c < g.n, 0, 0, c));
            bias[0] = t[0];
            bias[1] = t[1];
        } else {
            const f32x4 t = buf_load_x4(rbias, elem_off(c < g.n, 0, 0, c));
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) bias[nb] = t[nb];
        }
#pragma unroll
        for (int mb = 0; mb < T::MB; ++mb) {
            float cold[16][T::NB];
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = row_of(mb, v);
                const uint32_t off = elem_off(g.use_beta && r < g.m && c < g.n, r, g.ldc, c);
                if constexpr (T::NB == 2) {
                    const f32x2 t = buf_load_x2(rc, off);
                    cold[v][0] = t[0];
                    cold[v][1] = t[1];
                } else {
                    const f32x4 t = buf_load_x4(rc, off);
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb) cold[v][nb] = t[nb];
                }
            }
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = row_of(mb, v);
                float x[T::NB];
#pragma unroll
                for (int nb = 0; nb < T::NB; ++nb) {
                    x[nb] = g.alpha * acc[mb][nb][v] + g.beta * cold[v][nb] + bias[nb];
                    x[nb] = fmaxf(x[nb], lo);
                    x[nb] = gelu ? gelu_erf(x[nb]) : x[nb];
                }
                const uint32_t off = elem_off(r < g.m && c < g.n, r, g.ldc, c);
                if constexpr (T::NB == 2)
                    buf_store_x2(x[0], x[1], rc, off);
                else
                    buf_store_x4(f32x4{x[0], x[1], x[2], x[3]}, rc, off);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
        // Branch-free over the elements: C reads as zero when beta == 0 (an
        // out-of-range offset), ReLU is max(x, lo) with lo = -inf when off,
        // GELU is selected.  A branch per element splits the block into
        // pieces the scheduler cannot see across.
        const __amdgpu_buffer_rsrc_t rbias = make_rsrc(g.bias, g.bias ? (uint32_t)g.n * 4u : 0u);
        const float lo = g.act == 1 ? 0.0f : -__builtin_inff();
        const bool gelu = g.act == 2;
#pragma unroll
        for (int mb = 0; mb < T::MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < T::NB; ++nb) {
                const int c = col_of(nb);
                const float bias = buf_load_x1(rbias, elem_off(c < g.n, 0, 0, c));
                float cold[16];
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int r = row_of(mb, v);
                    cold[v] = buf_load_x1(rc, elem_off(g.use_beta && r < g.m && c < g.n, r, g.ldc, c));
                }
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int r = row_of(mb, v);
                    float x = g.alpha * acc[mb][nb][v] + g.beta * cold[v] + bias;
                    x = fmaxf(x, lo);
                    x = gelu ? gelu_erf(x) : x;
                    buf_store_x1(x, rc, elem_off(r < g.m && c < g.n, r, g.ldc, c));
                }
                // One block at a time, so its loads are the only ones in flight.
                __builtin_amdgcn_sched_barrier(0);
            }
    }
}

// Stream-K bookkeeping.  The slab iterations of all tiles, I = tiles * KT in
// tile order, are cut into P = sk_wgs equal ranges; range p is
// [p*I/P, (p+1)*I/P).
struct StreamK {
    long long iters;
    int wgs;
    __device__ long long start(int p) const { return (long long)p * iters / wgs; }
    // The range that holds iteration x.
    __device__ int owner(long long x) const { return (int)(((x + 1) * wgs - 1) / iters); }
};

// A tile whose slabs are shared by several ranges ("segments", in k order)
// is finished by the last segment to arrive.  Every segment publishes its
// partial sums as epoch-tagged 64-bit words in a slot of its own range (two
// slots per range: its first and its last tile), then counts itself in; the
// last one reads all segments back and adds them in k order, so the sum does
// not depend on who arrives last, and writes the tile to C.  (The last one
// could keep its own part in its accumulators, but adding vector-ALU
// results to the accumulators makes the compiler hold all of them in vector
// registers, which halves the occupancy of the whole kernel.)  Word w of a
// slot belongs to lane w % THREADS, so each access instruction covers
// consecutive words; the words go through a buffer descriptor with the
// device-scope cache policy, with the lane's offset in one register and the
// slot and block in the scalar offset, and are read back eight per lane at
// a time, so the fix-up needs few registers beyond the main loop's.
template <class T, bool B_COL, bool EPI = false>
__device__ __forceinline__ void dma_fixup(const GemmArgs &g, __amdgpu_buffer_rsrc_t rc, const StreamK &sk, int t,
                                          int p, int tid, int row0, int col0, int wr, int wc, int l32, int half,
                                          int *last_flag, unsigned epoch, const f32x16 (&acc)[T::MB][T::NB])
{

    const long long t0 = (long long)t * g.k_tiles;
    const int p_lo = sk.owner(t0), p_hi = sk.owner(t0 + g.k_tiles - 1);
    const int nseg = p_hi - p_lo + 1;
    constexpr uint32_t SLOT = (uint32_t)T::BM * T::BN;   // words
    // Slot of range q's segment of this tile: 2q for a range that starts in
    // the tile (the tile is its first), 2q + 1 for one that starts before.
    auto slot = [&](int q) { return (uint32_t)(2 * q + (sk.start(q) < t0 ? 1 : 0)) * SLOT; };
    // Word of (block, element v) relative to the lane's first word.
    auto word = [](int mb, int nb, int v) { return (uint32_t)(((mb * T::NB + nb) * 16 + v) * T::THREADS); };

    const __amdgpu_buffer_rsrc_t rp = make_rsrc(g.partial, g.partial_bytes);
    const uint32_t lane_off = (uint32_t)tid * 8u;
    const uint32_t mine = slot(p);
#pragma unroll
    for (int mb = 0; mb < T::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < T::NB; ++nb) {
#pragma unroll
            for (int v = 0; v < 16; ++v)
                buf_store_tagged(acc[mb][nb][v], epoch, rp, lane_off, (mine + word(mb, nb, v)) * 8u);
            // One block at a time: keeps the scheduler from pulling all
            // accumulators into vector registers at once.
            __builtin_amdgcn_sched_barrier(0);
        }

    // Every wavefront has issued its words before the segment counts itself
    // in, so the last segment to arrive finds every word of the others at
    // least in flight.
    issue_barrier();
    if (tid == 0) {
        const unsigned before = __hip_atomic_fetch_add(g.arrivals + t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = before == (unsigned)(nseg - 1);
        if (last) {
            // Every other segment has counted itself in: reset for the next
            // run, and count one more tile this workgroup finishes (a
            // word-tagged launch reports them at the kernel's end).
            __hip_atomic_store(g.arrivals + t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            ++last_flag[1];
        }
        *last_flag = last;
    }
    __syncthreads();
    if (!*last_flag) return;
    int budget = g.wait_budget;
    const unsigned want = epoch ^ g.epoch_xor;

    constexpr int H = 8;   // words per lane in flight
#pragma unroll
    for (int mb = 0; mb < T::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < T::NB; ++nb)
#pragma unroll
            for (int v0 = 0; v0 < 16; v0 += H) {
                float sum[H];
                for (int jj = 0; jj < nseg; ++jj) {
                    const uint32_t base = slot(p_lo + jj);
                    unsigned long long w[H];
#pragma unroll
                    for (int v = 0; v < H; ++v) w[v] = buf_load_tagged(rp, lane_off, (base + word(mb, nb, v0 + v)) * 8u);
#pragma unroll
                    for (int v = 0; v < H; ++v) {
                        // The word's address is formed only if it has not arrived yet.
                        const float x = (unsigned)(w[v] >> 32) == want
                                            ? __uint_as_float((unsigned)w[v])
                                            : wait_tagged_word(g.partial + base + word(mb, nb, v0 + v) + tid, w[v],
                                                               want, budget);
                        sum[v] = jj == 0 ? x : sum[v] + x;
                    }
                }
#pragma unroll
                for (int v = 0; v < H; ++v) {
                    const int e = v0 + v;
                    const int r = row0 + wr * T::WM + mb * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
                    const int c = B_COL ? col0 + wc * T::WN + nb * 32 + l32 : col0 + wc * T::WN + T::NB * l32 + nb;
                    const bool in = r < g.m && c < g.n;
                    float y = sum[v];
                    if constexpr (EPI) {
                        if (in) y = linear_epilogue(g, y, r, c);
                    }
                    buf_store_x1(y, rc, elem_off(in, r, g.ldc, c));
                }
                __builtin_amdgcn_sched_barrier(0);
            }
    record_give_up(budget, g.status);
}

// One whole tile per workgroup.  A_COL: column-major A; EPI: the
// linear-layer epilogue; WIDE_C: row-major B, N a multiple of T::NB, C
// stored NB adjacent columns per instruction.  `lds`: the copy ring,
// T::STAGES * (T::A_CHUNKS + T::B_CHUNKS) chunks.
template <class T, bool B_COL, bool A_COL = false, bool EPI = false, bool WIDE_C = false>
__device__ __forceinline__ void dma_whole_tile(const GemmArgs &g, f32x4 *lds)
{
    f32x4 *const lds_a = lds;                                // [STAGES][A_CHUNKS]
    f32x4 *const lds_b = lds + T::STAGES * T::A_CHUNKS;      // [STAGES][B_CHUNKS]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wave % T::WAVES_M, wc = wave / T::WAVES_M;
    const int l32 = lane & 31, half = lane >> 5;
    // (Not in the epilogue kernels, which share the copy ring with the plain
    // ones: there the test branch cost one of them occupancy.)
    if constexpr (!EPI)
        if (g.poison_lds) poison_lds(lds, T::STAGES * (T::A_CHUNKS + T::B_CHUNKS), tid, T::THREADS);

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
    dma_range<T, B_COL, A_COL>(g, lds_a, lds_b, ra, rb, row0, col0, 0, g.k_tiles, tid, wave, wr, wc, l32, half, acc);
    dma_store_c<T, B_COL, A_COL, EPI, WIDE_C>(g, rc, row0, col0, wr, wc, l32, half, acc);
}

template <class T, bool B_COL, bool A_COL = false, bool EPI = false, bool WIDE_C = false>
__global__ __launch_bounds__(T::THREADS) void gemm_mfma_dma_kernel(GemmArgs g)
{
    __shared__ f32x4 lds[T::STAGES * (T::A_CHUNKS + T::B_CHUNKS)];
    dma_whole_tile<T, B_COL, A_COL, EPI, WIDE_C>(g, lds);
}

// Stream-K ("GEMM 性能优化", Wave 模型: a last, partly filled wave of tiles
// idles most of the GPU).  The grid's first sk_wgs workgroups share the slab
// iterations of tiles [0, sk_tiles) evenly; the workgroups after them take
// one whole tile each of the rest.  With sk_wgs = S * sk_tiles every shared
// tile is split into S k-segments run side by side, which keeps workgroups
// at the same k (and in the same L2 lines) as their neighbours.  The shared
// tiles come first, so their fix-ups overlap the whole-tile work that
// follows.  Range p covers the tail of its first tile, whole tiles, and the
// head of its last tile; the two partial segments run first.
// Wavefronts per SIMD the stream-K kernel is register-budgeted for: as many
// workgroups per CU as the whole-tile kernel of the tile holds (its LDS ring
// and registers allow 8 of 64x64, 5 of 64x128 and 128x64, 3 of 128x128),
// since a plan that shares only some tiles runs all of them in this kernel.
// The larger tiles are held to their count by LDS alone.
template <class T>
constexpr int sk_waves_per_simd()
{
    constexpr int lds_cap = 163840 / (T::LDS_BYTES + 16);
    constexpr int reg_cap = T::BM * T::BN <= 4096 ? 8 : T::BM * T::BN <= 8192 ? 5 : T::BM * T::BN <= 16384 ? 3 : 1;
    return lds_cap < reg_cap ? lds_cap : reg_cap;
}

// EPI: C gets the linear-layer epilogue, in the whole tiles' stores and in
// the fix-up's (linear_epilogue, per element).
template <class T, bool B_COL, bool EPI>
__device__ __forceinline__ void dma_sk_body(const GemmArgs &g)
{
    // The fix-up's flag lives in one extra chunk of the ring's array: with a
    // second LDS variable the compiler can no longer tell the ring's copies
    // from the fragment reads, and waits for every copy before each read.
    __shared__ f32x4 lds[T::STAGES * (T::A_CHUNKS + T::B_CHUNKS) + 1];
    int *const last_flag = reinterpret_cast<int *>(lds + T::STAGES * (T::A_CHUNKS + T::B_CHUNKS));
    f32x4 *const lds_a = lds;                                // [STAGES][A_CHUNKS]
    f32x4 *const lds_b = lds + T::STAGES * T::A_CHUNKS;      // [STAGES][B_CHUNKS]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wave % T::WAVES_M, wc = wave / T::WAVES_M;
    const int l32 = lane & 31, half = lane >> 5;
    if (g.poison_lds) poison_lds(lds, T::STAGES * (T::A_CHUNKS + T::B_CHUNKS), tid, T::THREADS);

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.A, g.a_bytes);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(g.B, g.b_bytes);
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(g.C, g.c_bytes);
    const int KT = g.k_tiles;

    f32x16 acc[T::MB][T::NB];
    if ((int)blockIdx.x >= g.sk_wgs) {
        // One whole tile of [sk_tiles, tiles).
        const int whole = g.tiles_m * g.tiles_n - g.sk_tiles;
        int tm, tn;
        grouped_tile(g.sk_tiles + xcd_contiguous(blockIdx.x - g.sk_wgs, whole, g.num_xcd), g, tm, tn);
        const int row0 = tm * T::BM, col0 = tn * T::BN;
#pragma unroll
        for (int mb = 0; mb < T::MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < T::NB; ++nb) acc[mb][nb] = f32x16{};
        dma_range<T, B_COL>(g, lds_a, lds_b, ra, rb, row0, col0, 0, KT, tid, wave, wr, wc, l32, half, acc);
        dma_store_c<T, B_COL, false, EPI>(g, rc, row0, col0, wr, wc, l32, half, acc);
        return;
    }

    const StreamK sk{(long long)g.sk_tiles * KT, g.sk_wgs};
    const int p = xcd_contiguous(blockIdx.x, g.sk_wgs, g.num_xcd);
    // This run's tag, in a scalar register: the argument, or for a
    // word-tagged launch the epoch word's (read here, before the copies).
    unsigned epoch = g.epoch;
    if (g.epoch_word) epoch = __builtin_amdgcn_readfirstlane(load_run_epoch(g));
    if (tid == 0) last_flag[1] = 0;   // split tiles this workgroup finishes (thread 0's count)
    const long long i0 = sk.start(p), i1 = sk.start(p + 1);
    if (i0 >= i1) return;
    const int t_first = (int)(i0 / KT), t_last = (int)((i1 - 1) / KT);
    const int head0 = (int)(i0 - (long long)t_first * KT);           // first slab in t_first
    const int tail1 = (int)(i1 - (long long)t_last * KT);            // end slab in t_last
    // Work items in order: partial first tile, partial last tile, whole tiles.
    const bool first_partial = head0 != 0 || (t_first == t_last && tail1 != KT);
    const bool last_partial = t_last != t_first && tail1 != KT;
    const int n_part = (first_partial ? 1 : 0) + (last_partial ? 1 : 0);
    const int full0 = first_partial ? t_first + 1 : t_first;
    const int n_items = n_part + max(0, (last_partial ? t_last : t_last + 1) - full0);

    for (int it = 0; it < n_items; ++it) {
        int t = full0 + it - n_part, kt0 = 0, kt1 = KT;
        if (it == 0 && first_partial) {
            t = t_first; kt0 = head0; kt1 = t_first == t_last ? tail1 : KT;
        } else if (it < n_part) {
            t = t_last; kt1 = tail1;
        }
        int tm, tn;
        grouped_tile(t, g, tm, tn);
        const int row0 = tm * T::BM, col0 = tn * T::BN;
        // The lane's position, opaque to the compiler once per work item:
        // otherwise every per-lane offset of the copies, fragment reads,
        // stores and fix-up is hoisted out of this loop and held in
        // registers across all of it.
        int tid_i = tid;
        asm volatile("" : "+v"(tid_i));
        const int l32_i = tid_i & 31, half_i = (tid_i >> 5) & 1;
#pragma unroll
        for (int mb = 0; mb < T::MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < T::NB; ++nb) acc[mb][nb] = f32x16{};
        dma_range<T, B_COL>(g, lds_a, lds_b, ra, rb, row0, col0, kt0, kt1, tid_i, wave, wr, wc, l32_i, half_i, acc);
        if (kt0 == 0 && kt1 == KT)
            dma_store_c<T, B_COL, false, EPI>(g, rc, row0, col0, wr, wc, l32_i, half_i, acc);
        else
            dma_fixup<T, B_COL, EPI>(g, rc, sk, t, p, tid_i, row0, col0, wr, wc, l32_i, half_i, last_flag, epoch,
                                     acc);
    }
    // A word-tagged launch counts the split tiles this workgroup finished
    // (here, where the registers are free, rather than in the fix-up).
    if (g.epoch_word && tid == 0 && last_flag[1] > 0) {
        const int finished = last_flag[1];
        advance_epoch(g, count_split_tiles(g, finished), epoch, finished);
    }
}

template <class T, bool B_COL>
__global__ __launch_bounds__(T::THREADS, sk_waves_per_simd<T>()) void gemm_mfma_dma_sk_kernel(GemmArgs g)
{
    dma_sk_body<T, B_COL, false>(g);
}

// The same with the linear-layer epilogue (row-major A).  Held to four
// wavefronts per SIMD (the epilogue's registers spilled at eight; the
// stream-K plans run at most three workgroups per CU).
template <class T, bool B_COL>
__global__ __launch_bounds__(T::THREADS, sk_waves_per_simd<T>() < 4 ? sk_waves_per_simd<T>() : 4) void
gemm_mfma_dma_sk_epi_kernel(GemmArgs g)
{
    dma_sk_body<T, B_COL, true>(g);
}

}  // namespace gemmf32

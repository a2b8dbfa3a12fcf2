// Few-row FP32 GEMM (M <= 32): the bandwidth-bound shape.
//
// With M = 16 the product does ~8 FLOP per byte of B, below the MI355X ridge
// point of ~19.7 FLOP/B ("GEMM 性能优化", Roofline 与平衡点: below the ridge
// the kernel is bandwidth-limited), so the goal is to stream B from HBM once
// at full bandwidth.  Every element of B is used by all M rows in a single
// v_mfma_f32_16x16x4_f32 and never again, so B goes straight from HBM into
// MFMA operand registers (no LDS), and enough wavefronts with enough loads
// each stay in flight to cover the memory latency ("GPU 算子优化中的数据复用",
// 11.1: memory-bound kernels need parallelism to hide latency; "PMPP Chapter
// 06", section 2: many concurrent requests).
//
// MFMA 16x16x4 (f32): lane l supplies A[i = l%16][kk = l/16] and
// B[kk = l/16][j = l%16]; the 16x16 result sits as 4 values per lane at row
// 4*(l/16) + v, column l%16.  Lane group h = l/16 walks the k-run
// kq + 4h + t (t = 0..3) of each 16-k group, so one 16-byte load of A gives a
// lane its A values for 4 k-steps.
//
// Tile widths.  BN = 64: four MFMA blocks with interleaved columns (lane
// column j stands for column 4*j + nb of block nb), so one 16-byte load of
// row-major B feeds all 4 blocks of a k-step; column-major B is loaded as 16
// bytes along k of one column.  BN = 32: two interleaved blocks, 8-byte
// loads of row-major B.  BN = 16: one block; row-major B is loaded one
// element per k-step (16 lanes still read 64 contiguous bytes of a row),
// column-major B as 16 bytes along k.  The narrow tile gives N/16 workgroups,
// enough to cover the CUs without splitting k across workgroups.
//
// Within a workgroup the WAVES wavefronts take contiguous shares of the
// workgroup's k-range, and the shares are added in LDS in wavefront order.
// When k is also split across workgroups, each split's partial sums go to
// the plan's workspace and the last workgroup of a tile to finish adds the
// splits in split order.  Both orders are fixed, so results are
// reproducible run to run.  (Splitting
// k is the partial-result-then-merge pattern the checklist of "PMPP Chapter
// 06", section 4, calls privatization.)
#pragma once

#include "device_common.hpp"
#include "epilogue.hpp"

namespace gemmf32 {

template <int WAVES_, int DEPTH_, int BN_, int RT_ = 1>
struct SkinnyTile {
    static_assert(BN_ == 16 || BN_ == 32 || BN_ == 64, "one MFMA block, or two or four interleaved ones");
    static_assert(RT_ == 1 || RT_ == 2, "16 or 32 rows");
    static constexpr int WAVES = WAVES_;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int RT = RT_;                    // 16-row MFMA blocks per tile (rows of A per lane)
    static constexpr int BM = 16 * RT, BN = BN_, KQ = 16;  // rows, columns, k per load group
    static constexpr int NB = BN / 16;                // MFMA blocks per tile row
    static constexpr int DEPTH = DEPTH_;              // k groups in flight per wavefront
    // LDS floats per wavefront in the reduction (one past red_index's largest value).
    static constexpr int RED = BN == 64   ? (BM - 1) * 65 + 64 + 2 * ((BM - 1) >> 2) + 1
                               : BN == 32 ? 33 * BM
                                          : (BM - 1) * 16 + 16 + 16 * ((BM - 1) >> 2);
};

// LDS position of element (r, c) of a wavefront's BM x BN share in the
// reduction (each 16-row block placed as the first).  An accumulator write puts lanes (h, j) = (l / 16, l % 16) at
// row 4h + v, column NB*j + nb, and LDS serves 32 lanes per cycle from 32
// banks: for BN = 16 the 16 columns of two row groups land 16 banks apart;
// for BN = 64 (rows 65 floats apart) the columns 4j (8 banks, twice) are
// skewed by one bank from column 32 on and the row groups by two more.  The
// reads, consecutive c of one row, stay on distinct banks.
template <class T>
constexpr __host__ __device__ int red_index(int r, int c)
{
    if constexpr (T::BN == 64) return r * 65 + c + (c >> 5) + 2 * (r >> 2);
    else if constexpr (T::BN == 32) return r * 33 + c + ((r >> 2) & 1);
    else return r * 16 + c + 16 * (r >> 2);
}

// Every element of the tile has a position of its own inside RED.
template <class T>
constexpr bool red_index_one_to_one()
{
    bool used[T::RED] = {};
    for (int r = 0; r < T::BM; ++r)
        for (int c = 0; c < T::BN; ++c) {
            const int x = red_index<T>(r, c);
            if (x < 0 || x >= T::RED || used[x]) return false;
            used[x] = true;
        }
    return true;
}

// Loads of one 16-k group for lane (j, h): A[row + 16r][kq+4h .. +3] for
// each 16-row block r of the tile and the B values of the 4 k-steps.  NB = 4: b[t][nb] (row-major B) or b[nb][t]
// (column-major B) is column 4j + nb; NB = 2: b[nb][t] is column 2j + nb; NB = 1: b[0][t] is column j.  Element
// checks only when the group is not whole (tail of a range, or k past K).
// Columns at or past N may read other elements of B: they only feed columns
// of C that are never stored.  A_COL: column-major A, read one element per
// k-step (16 lanes read 64 contiguous bytes of a column; A is small and read
// from the L2).
template <class T, bool B_COL, bool A_COL = false>
__device__ __forceinline__ void skinny_load(const GemmArgs &g, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                            int row, int col0, int j, int h, int kq, int kend, bool whole,
                                            bool live, f32x4 (&a)[T::RT], f32x4 (&b)[T::NB])
{
    const int ka = kq + 4 * h;
    if (whole) {
        // A group that is not live reads zeros (out-of-range offsets).
#pragma unroll
        for (int r = 0; r < T::RT; ++r) {
            if constexpr (A_COL) {
                // One lane offset for the 4 k-steps; the steps' distance,
                // lda elements, is uniform and goes in the scalar offset.
                const uint32_t off = elem_off(live && row + 16 * r < g.m, ka, g.lda, row + 16 * r);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    a[r][q] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ra, (int)off, q * g.lda * 4, 0));
            } else {
                a[r] = buf_load_x4(ra, elem_off(live && row + 16 * r < g.m, row + 16 * r, g.lda, ka));
            }
        }
        if constexpr (T::NB == 4 && !B_COL) {
#pragma unroll
            for (int t = 0; t < 4; ++t) b[t] = buf_load_x4(rb, elem_off(live, ka + t, g.ldb, col0 + 4 * j));
        } else if constexpr (T::NB == 2 && !B_COL) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const f32x2 v = buf_load_x2(rb, elem_off(live, ka + t, g.ldb, col0 + 2 * j));
                b[0][t] = v[0];
                b[1][t] = v[1];
            }
        } else if constexpr (!B_COL) {
#pragma unroll
            for (int t = 0; t < 4; ++t) b[0][t] = buf_load_x1(rb, elem_off(live, ka + t, g.ldb, col0 + j));
        } else {
#pragma unroll
            for (int nb = 0; nb < T::NB; ++nb) {
                const int col = col0 + T::NB * j + nb;
                b[nb] = buf_load_x4(rb, elem_off(live && col < g.n, col, g.ldb, ka));
            }
        }
    } else {
#pragma unroll
        for (int r = 0; r < T::RT; ++r)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                a[r][q] = buf_load_x1(ra, A_COL ? elem_off(row + 16 * r < g.m && ka + q < kend, ka + q, g.lda, row + 16 * r)
                                                : elem_off(row + 16 * r < g.m && ka + q < kend, row + 16 * r, g.lda, ka + q));
#pragma unroll
        for (int x = 0; x < T::NB; ++x)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                // (x, q) = (block, k-step) for column-major B and NB = 1;
                // (k-step, block) for row-major B with NB = 4.
                const int kk = (T::NB == 4 && !B_COL) ? x : q;
                const int nb = (T::NB == 4 && !B_COL) ? q : x;
                const int col = col0 + T::NB * j + nb;
                const bool ok = ka + kk < kend && col < g.n;
                b[x][q] = buf_load_x1(rb, B_COL ? elem_off(ok, col, g.ldb, ka + kk) : elem_off(ok, ka + kk, g.ldb, col));
            }
    }
}

template <class T, bool B_COL>
__device__ __forceinline__ void skinny_mfma(const f32x4 (&a)[T::RT], const f32x4 (&b)[T::NB],
                                            f32x4 (&acc)[T::RT][T::NB])
{
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int nb = 0; nb < T::NB; ++nb) {
            const float bv = (T::NB == 4 && !B_COL) ? b[t][nb] : b[nb][t];
#pragma unroll
            for (int r = 0; r < T::RT; ++r)
                acc[r][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r][t], bv, acc[r][nb], 0, 0, 0);
        }
}

// Grid: tiles_m * tiles_n * split_k workgroups.  With one split the
// workgroup writes its tile of C; otherwise the splits meet through
// g.partial[split][m][n] (epoch-tagged words) and g.arrivals[tile].
// EPI: C gets the linear-layer epilogue (linear_epilogue) where it is written.
// A_COL: column-major A.
template <class T, bool B_COL, bool EPI, bool A_COL = false>
__device__ __forceinline__ void skinny_body(const GemmArgs &g)
{
    static_assert(red_index_one_to_one<T>(), "reduction layout");
    __shared__ float red[T::WAVES][T::RED];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15, h = lane >> 4;

    // Workgroups on one XCD take neighbouring tiles of one split, row tiles
    // first: the row tiles of one column of tiles read the same B at about
    // the same time, through that XCD's L2.
    const int per_split = g.tiles_m * g.tiles_n;
    const int wg = xcd_contiguous(blockIdx.x, per_split * g.split_k, g.num_xcd);
    const int split = wg / per_split;
    const int rest = wg - split * per_split;
    const int tn = rest / g.tiles_m, tm = rest - (rest / g.tiles_m) * g.tiles_m;
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

    const int row = row0 + j;    // A row this lane supplies (and row + 16r for block r)
    f32x4 acc[T::RT][T::NB];
#pragma unroll
    for (int r = 0; r < T::RT; ++r)
#pragma unroll
        for (int nb = 0; nb < T::NB; ++nb) acc[r][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Split plans: the workgroups of a tile count themselves in on the
    // tile's arrival counter as soon as thread 0's wavefront has issued its
    // last loads, so the count's round trip overlaps the stream; the last to
    // count in adds the splits.  Every workgroup counted in is resident and
    // in its last pass (its other wavefronts stream alongside thread 0's),
    // with only the sums and its stores after it, so the last one's wait for
    // their words is short (and bounded in any case).  A
    // word-tagged launch (captured in a graph) reads its tag first, so that
    // when the run's last split tile advances the epoch word every workgroup
    // has read it.
    __shared__ unsigned run_epoch;
    const bool word_tag = g.epoch_word != nullptr && g.split_k > 1;
    unsigned word_read = 0, tag_read = 0, before = 0;
    if (word_tag && tid == 0) word_read = load_epoch_word(g);   // waited for at the count
    auto count_in = [&]() {
        if (g.split_k > 1 && tid == 0) {
            int slot = rest;
            if (word_tag) {
                // The count goes out only once the word has come back: the
                // empty asm takes the word here (not earlier) and makes the
                // counter's index depend on it.
                unsigned w = word_read;
                asm volatile("" : "+v"(w), "+v"(slot));
                tag_read = run_epoch_of(w);
                run_epoch = tag_read;
            }
            before = __hip_atomic_fetch_add(g.arrivals + slot, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    };

    // Whole 16-k groups stream through a ring of DEPTH register slots: the
    // loads of group q + DEPTH are issued as soon as group q has been
    // multiplied, so DEPTH groups (5 * DEPTH loads) stay in flight.  The ring
    // runs a whole number of passes; the groups past the range load zeros,
    // so every load is unconditional and in group order, and the counter
    // wait before each group's MFMAs lets the DEPTH - 1 later groups fly.
    // Only the last pass can hold such groups, and their MFMAs are skipped
    // (a wavefront-uniform branch): with short k-shares (16 k per wavefront
    // at 256^3) they would be most of the matrix-core work.
    constexpr int D = T::DEPTH;
    const int kspan = max(0, kw1 - kw0);
    const int G = kspan / T::KQ;
    const int passes = (G + D - 1) / D;
    if (passes > 0) {
        f32x4 a[D][T::RT], b[D][T::NB];
#pragma unroll
        for (int u = 0; u < D; ++u) {
            skinny_load<T, B_COL, A_COL>(g, ra, rb, row, col0, j, h, kw0 + u * T::KQ, kw1, true, u < G, a[u], b[u]);
            __builtin_amdgcn_sched_barrier(0);
        }
        for (int p = 1; p < passes; ++p) {
#pragma unroll
            for (int u = 0; u < D; ++u) {
                const int q = p * D + u;
                skinny_mfma<T, B_COL>(a[u], b[u], acc);
                __builtin_amdgcn_sched_barrier(0);
                skinny_load<T, B_COL, A_COL>(g, ra, rb, row, col0, j, h, kw0 + q * T::KQ, kw1, true, q < G, a[u], b[u]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        count_in();
        __builtin_amdgcn_sched_barrier(0);
        const int last0 = (passes - 1) * D;
        if (last0 + D <= G) {
#pragma unroll
            for (int u = 0; u < D; ++u) skinny_mfma<T, B_COL>(a[u], b[u], acc);
        } else {
#pragma unroll
            for (int u = 0; u < D; ++u)
                if (last0 + u < G) skinny_mfma<T, B_COL>(a[u], b[u], acc);
        }
    } else {
        count_in();
    }
    // The partial group at the end of the range, element by element.
    if (G * T::KQ < kspan) {
        f32x4 at[T::RT], bt[T::NB];
        skinny_load<T, B_COL, A_COL>(g, ra, rb, row, col0, j, h, kw0 + G * T::KQ, kw1, false, true, at, bt);
        skinny_mfma<T, B_COL>(at, bt, acc);
    }

    // Add the wavefronts' shares in wavefront order (element (r, c) of the
    // BM x BN tile: r = 16*rt + 4*h + v, c = NB*j + nb; LDS positions by
    // red_index, free of bank conflicts).
#pragma unroll
    for (int rt = 0; rt < T::RT; ++rt)
#pragma unroll
        for (int nb = 0; nb < T::NB; ++nb)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                red[wave][red_index<T>(16 * rt + 4 * h + v, T::NB * j + nb)] = acc[rt][nb][v];
    __shared__ int last;
    if (g.split_k > 1 && tid == 0) {
        last = before == (unsigned)(g.split_k - 1);
        if (last) {
            // Every split of this tile has counted itself in: reset the
            // counter for the next run; a word-tagged launch counts the tile
            // finished.
            __hip_atomic_store(g.arrivals + rest, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (word_tag) advance_epoch(g, count_split_tiles(g), tag_read);
        }
    }
    __syncthreads();
    // This run's tag for the partial sums.
    const unsigned epoch = word_tag ? __builtin_amdgcn_readfirstlane(run_epoch) : g.epoch;

    constexpr int ELEMS = T::BM * T::BN;
    constexpr int EPT = (ELEMS + T::THREADS - 1) / T::THREADS;   // elements per thread
    float own[EPT];
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
        const int e = tid + q * T::THREADS;
        float s = 0.0f;
        if (e < ELEMS) {
            const int x = red_index<T>(e / T::BN, e % T::BN);
            s = red[0][x];
#pragma unroll
            for (int w = 1; w < T::WAVES; ++w) s += red[w][x];
        }
        own[q] = s;
    }
    if (g.split_k == 1) {
#pragma unroll
        for (int q = 0; q < EPT; ++q) {
            const int e = tid + q * T::THREADS;
            const int r = row0 + e / T::BN, c = col0 + e % T::BN;
            if (e < ELEMS && r < g.m && c < g.n)
                g.C[(size_t)r * g.ldc + c] = EPI ? linear_epilogue(g, own[q], r, c) : own[q];
        }
        return;
    }

    // k is split across workgroups.  Each split but the last to count in
    // publishes its partial sums as 64-bit words {value, epoch}, written
    // whole, so a reader that sees this run's epoch in a word also sees the
    // value beside it (no fence needed).  The last to count in adds the
    // splits in split order and writes C.
    const size_t plane = (size_t)g.m * g.n;
    const unsigned long long tag = (unsigned long long)epoch << 32;
    if (!last) {
#pragma unroll
        for (int q = 0; q < EPT; ++q) {
            const int e = tid + q * T::THREADS;
            const int r = row0 + e / T::BN, c = col0 + e % T::BN;
            if (e < ELEMS && r < g.m && c < g.n)
                store_tagged_word(g.partial + split * plane + (size_t)r * g.n + c, own[q], epoch);
        }
        return;
    }
    int budget = g.wait_budget;
    const unsigned want = epoch ^ g.epoch_xor;

#pragma unroll
    for (int q = 0; q < EPT; ++q) {
        const int e = tid + q * T::THREADS;
        const int r = row0 + e / T::BN, c = col0 + e % T::BN;
        if (!(e < ELEMS && r < g.m && c < g.n)) continue;
        const unsigned long long *p = g.partial + (size_t)r * g.n + c;
        float sum = 0.0f;
        // The words of up to 8 splits are loaded together, then checked.
        for (int s0 = 0; s0 < g.split_k; s0 += 8) {
            unsigned long long w[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                w[u] = (s0 + u < g.split_k && s0 + u != split)
                           ? load_tagged_word(p + (s0 + u) * plane)
                           : tag;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int sp = s0 + u;
                if (sp >= g.split_k) break;
                const float v = sp == split ? own[q] : wait_tagged_word(p + sp * plane, w[u], want, budget);
                sum = sp == 0 ? v : sum + v;
            }
        }
        g.C[(size_t)r * g.ldc + c] = EPI ? linear_epilogue(g, sum, r, c) : sum;
    }
    record_give_up(budget, g.status);
}

template <class T, bool B_COL>
__global__ __launch_bounds__(T::THREADS) void gemm_skinny_kernel(GemmArgs g)
{
    skinny_body<T, B_COL, false>(g);
}

// The same with the linear-layer epilogue (row-major A).
template <class T, bool B_COL>
__global__ __launch_bounds__(T::THREADS) void gemm_skinny_epi_kernel(GemmArgs g)
{
    skinny_body<T, B_COL, true>(g);
}

// Column-major A, without and with the epilogue.
template <class T, bool B_COL>
__global__ __launch_bounds__(T::THREADS) void gemm_skinny_acol_kernel(GemmArgs g)
{
    skinny_body<T, B_COL, false, true>(g);
}

template <class T, bool B_COL>
__global__ __launch_bounds__(T::THREADS) void gemm_skinny_acol_epi_kernel(GemmArgs g)
{
    skinny_body<T, B_COL, true, true>(g);
}

}  // namespace gemmf32

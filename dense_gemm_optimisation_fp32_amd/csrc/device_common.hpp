// Device-side helpers shared by the GEMM kernels: vector types, raw buffer
// descriptors with hardware range checking, and the launch argument block.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gemmf32 {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Word 3 of a gfx9-family raw buffer descriptor: 32-bit data format, no
// swizzle, no stride.  Loads whose byte offset is at or past num_records
// return zero and such stores are dropped, so boundary tiles need no branch:
// an out-of-range element gets the offset kOobOffset instead of its address.
constexpr int kRawBufferWord3 = 0x00020000;
// Every operand's byte extent is validated to be below 2^31, so this offset
// is always out of range.
constexpr uint32_t kOobOffset = 0x80000000u;

// Launch arguments, identical for every kernel family.  Sizes in elements;
// *_bytes are the operands' byte extents (num_records of the descriptors).
struct GemmArgs {
    const float *A;
    const float *B;
    float *C;
    int m, n, k;
    int lda, ldb, ldc;
    int tiles_m, tiles_n;  // output tiles along M and N
    int k_tiles;           // ceil(k / BK)
    int group_m;           // tile-rows per rasterisation group
    int num_xcd;           // dispatch round-robins workgroups over this many XCDs
    uint32_t a_bytes, b_bytes, c_bytes;
    unsigned long long *partial;  // partial sums of split tiles, epoch-tagged words
    uint32_t partial_bytes;       // byte extent of the stream-K partial-sum words (< 2^31)
    unsigned *arrivals;           // per-tile arrival counters for split tiles
    unsigned epoch;               // tag of this run's partial sums (bit 31 clear, never 0), unless:
    unsigned *epoch_word;         // non-NULL: the run takes its tag from this workspace word
                                  // (launches captured in a graph; see load_run_epoch)
    unsigned *done_tiles;         // workspace counter of the run's finished split tiles
    int split_tiles;              // tiles that workgroups share (finished by a last arriver)
    int sk_wgs;            // stream-K: workgroups sharing the first sk_tiles tiles' slabs (0: none)
    int sk_tiles;          // stream-K: tiles [0, sk_tiles) are shared; the rest get a workgroup each
    int split_k;           // number of k-splits (skinny path), else 1
    int k_per_split;       // k values per split (multiple of the k tile)
    int masked_loads;      // 1: check every element in every slab (tiny ldb)
    // Linear-layer epilogue (kernels built with it): act(alpha * AB + beta * C + bias[col]).
    float alpha, beta;
    const float *bias;     // N values, or NULL
    int use_beta;          // beta != 0: C is read
    int act;               // 0 none, 1 ReLU, 2 GELU (x * Phi(x))
    // Waits for partial sums (split-k and stream-K plans).
    unsigned *status;      // workspace word set to 1 when a wait gave up (a NaN went to C), or NULL
    int wait_budget;       // polls one thread may spend waiting for partial sums
    unsigned epoch_xor;    // readers wait for the tag (this run's epoch) ^ epoch_xor (0; a test sets
                           // it so that no word ever matches and every wait gives up)
    int poison_lds;        // 1: fill LDS with NaN before the first copy (a test of the waits)
    // Column sliver carried by a whole-tile launch (gemm_mfma_dma_sliver_kernel):
    // workgroups from sliver_wg0 on compute the sliver_cols columns after
    // the tiles' n with the few-column method.
    int sliver_wg0;        // first workgroup of the sliver (the tiles' count)
    int sliver_cols;
    const float *sliver_B; // B at the sliver's first column
    uint32_t sliver_b_bytes;
    float *sliver_C;       // C at the sliver's first column
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                             kRawBufferWord3);
}

__device__ __forceinline__ f32x4 buf_load_x4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off)
{
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0));
}

__device__ __forceinline__ f32x2 buf_load_x2(__amdgpu_buffer_rsrc_t r, uint32_t byte_off)
{
    return __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)byte_off, 0, 0));
}

__device__ __forceinline__ float buf_load_x1(__amdgpu_buffer_rsrc_t r, uint32_t byte_off)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)byte_off, 0, 0));
}

__device__ __forceinline__ void buf_store_x4(f32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t byte_off)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)byte_off, 0, 0);
}

__device__ __forceinline__ void buf_store_x2(float a, float b, __amdgpu_buffer_rsrc_t r, uint32_t byte_off)
{
    __builtin_amdgcn_raw_buffer_store_b64(
        u32x2{__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b)}, r, (int)byte_off, 0, 0);
}

__device__ __forceinline__ void buf_store_x1(float v, __amdgpu_buffer_rsrc_t r, uint32_t byte_off)
{
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, (int)byte_off, 0, 0);
}

// Byte offset of element (row, col) of a row-major operand, or the
// out-of-range offset when the element is outside the logical matrix.
__device__ __forceinline__ uint32_t elem_off(bool valid, uint32_t row, uint32_t ld, uint32_t col)
{
    return valid ? (row * ld + col) * 4u : kOobOffset;
}

// Workgroup id -> output tile (tm, tn).
//
// Step 1 undoes the hardware's round-robin dispatch of consecutive workgroup
// ids over the XCDs (each with its own L2): the workgroups that land on one
// XCD get a contiguous range of logical tile ids, so neighbouring tiles share
// that XCD's L2.  Step 2 walks the logical ids in groups of `group_m`
// tile-rows, column by column inside a group, so the tiles resident at one
// time reuse a few A row-panels and B column-panels instead of one full
// row of tiles ("GEMM 性能优化", Wave 模型与 L2 命中率: the block order alone
// changes the L2 hit rate).  Runs once per workgroup.
__device__ __forceinline__ int xcd_contiguous(int wg, int total, int num_xcd)
{
    const int x = wg % num_xcd;
    const int i = wg / num_xcd;
    const int per = total / num_xcd;
    const int rem = total % num_xcd;
    return x * per + (x < rem ? x : rem) + i;
}

__device__ __forceinline__ void grouped_tile(int logical, const GemmArgs &a, int &tm, int &tn)
{
    const int width = a.group_m * a.tiles_n;
    const int group = logical / width;
    const int first_m = group * a.group_m;
    const int rows_left = a.tiles_m - first_m;
    const int gsize = rows_left < a.group_m ? rows_left : a.group_m;
    const int r = logical - group * width;
    tm = first_m + r % gsize;
    tn = r / gsize;
}

__device__ __forceinline__ void raster_tile(int wg, const GemmArgs &a, int &tm, int &tn)
{
    grouped_tile(xcd_contiguous(wg, a.tiles_m * a.tiles_n, a.num_xcd), a, tm, tn);
}

// Value of a 64-bit partial-sum word {float bits, epoch} written by another
// workgroup, once it carries the epoch `want`.  `w` is a first load already
// in hand.  A writer counts itself in on the tile only when all it has
// left is to finish and issue its words (the stream-K kernel once they are
// issued, the few-row kernel once its last loads are), and the reader is
// the last to count in, so the wait ends; `budget` (polls
// left for the caller, shared by all its waits) only keeps a lost word from
// hanging the kernel: once it is spent, missing elements read as NaN at once
// and the budget is left negative, which the caller records in the plan's
// status word when it is done (record_give_up; gemm_f32_plan_check reports
// it).  The status store stays out of the wait so that its address is not
// held in registers across the reads.
constexpr int kTaggedWaitBudget = 1 << 16;

__device__ __forceinline__ float wait_tagged_word(const unsigned long long *p, unsigned long long w, unsigned want,
                                                  int &budget)
{
    while ((unsigned)(w >> 32) != want) {
        if (budget <= 0) {
            budget = -1;
            return __builtin_nanf("");
        }
        --budget;
        __builtin_amdgcn_s_sleep(1);
        w = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return __uint_as_float((unsigned)w);
}

// Tags of partial-sum words.  A launch made outside graph capture carries
// its tag as an argument, a fresh one per run (bit 31 clear).  A launch
// captured in a graph would replay the argument it was recorded with, so a
// replay could take the previous replay's words for its own; such launches
// take the tag from a word of the workspace instead, which the run's last
// split tile advances: one past the word's count, bit 31 set (so the two
// kinds never meet, and no tag is 0, the tag of words never written).
// Every workgroup that shares a tile reads the word before it tags a word.
__device__ __forceinline__ unsigned load_epoch_word(const GemmArgs &g)
{
    return __hip_atomic_load(g.epoch_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned run_epoch_of(unsigned epoch_word)
{
    return ((epoch_word + 1u) & 0x7fffffffu) | 0x80000000u;
}

__device__ __forceinline__ unsigned load_run_epoch(const GemmArgs &g)
{
    return run_epoch_of(load_epoch_word(g));
}

// Counts split tiles finished (one thread of their last arriver,
// word-tagged launches only); returns the count before them.  The run's last split tile
// then stores the run's count in the epoch word (advance_epoch): by that
// time every workgroup that tags words has read the old value (it reads it
// before it counts itself in on its tile), and the next run, on the same
// stream, starts after this one.
__device__ __forceinline__ unsigned count_split_tiles(const GemmArgs &g, int tiles = 1)
{
    return __hip_atomic_fetch_add(g.done_tiles, (unsigned)tiles, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void advance_epoch(const GemmArgs &g, unsigned done_before, unsigned epoch, int tiles = 1)
{
    if (done_before + (unsigned)tiles == (unsigned)g.split_tiles) {
        __hip_atomic_store(g.done_tiles, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(g.epoch_word, epoch & 0x7fffffffu, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

__device__ __forceinline__ void record_give_up(int budget, unsigned *status)
{
    if (budget < 0 && status) __hip_atomic_store(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroup barrier without a memory fence: every wavefront has issued all
// it did before the barrier, and nothing is waited for.  Used before a
// split tile's arrival count: the partial-sum words need only be issued
// (their readers wait for each word's tag), so the store round trip a
// fence would add stays off the critical path.
__device__ __forceinline__ void issue_barrier()
{
    asm volatile("s_barrier" ::: "memory");
}

// Test hook: fill `chunks` 16-byte LDS chunks with NaN before a kernel's
// first copy, so that a read of LDS that no copy or store has written yet
// (a missing wait or barrier) puts NaN into C.
__device__ __forceinline__ void poison_lds(f32x4 *lds, int chunks, int tid, int threads)
{
    const float nan = __builtin_nanf("");
    for (int i = tid; i < chunks; i += threads) lds[i] = f32x4{nan, nan, nan, nan};
    __syncthreads();
}

// GELU(x) = x * Phi(x) = x/2 * (1 + erf(x / sqrt(2))).  erf by Abramowitz
// and Stegun, formula 7.1.26 (|error| <= 1.5e-7 on z >= 0): with
// t = 1 / (1 + p z) and y = t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) e^(-z^2),
// erf(z) = 1 - y.  erf is odd, so 1 + erf(z) = 2 - y for z >= 0 and y(|z|)
// for z < 0: no cancellation on the negative side.  A handful of registers,
// where the library erff, unrolled over a block of outputs, took a hundred.
__device__ __forceinline__ float gelu_erf(float x)
{
    const float z = fabsf(x) * 0.70710678118654752f;
    const float t = 1.0f / (1.0f + 0.3275911f * z);
    const float poly =
        t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
    const float y = poly * __expf(-z * z);
    return 0.5f * x * (x >= 0.0f ? 2.0f - y : y);
}

__device__ __forceinline__ unsigned long long load_tagged_word(const unsigned long long *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_tagged_word(unsigned long long *p, float v, unsigned epoch)
{
    __hip_atomic_store(p, ((unsigned long long)epoch << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// The same device-scope accesses through a buffer descriptor.  A relaxed
// agent-scope 64-bit atomic load or store is an ordinary 64-bit access with
// the sc1 cache policy on gfx950; issued as a buffer access it takes a
// per-lane offset plus a wavefront-uniform scalar offset, so a lane's words
// spread over a tile need one address register in all instead of a 64-bit
// address each.
constexpr int kAgentScopePolicy = 16;  // sc1

__device__ __forceinline__ unsigned long long buf_load_tagged(__amdgpu_buffer_rsrc_t r, uint32_t lane_off,
                                                              uint32_t uniform_off)
{
    const u32x2 w = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)lane_off, (int)uniform_off, kAgentScopePolicy));
    return ((unsigned long long)w.y << 32) | w.x;
}

__device__ __forceinline__ void buf_store_tagged(float v, unsigned epoch, __amdgpu_buffer_rsrc_t r, uint32_t lane_off,
                                                 uint32_t uniform_off)
{
    const u32x2 w = {__float_as_uint(v), epoch};
    __builtin_amdgcn_raw_buffer_store_b64(w, r, (int)lane_off, (int)uniform_off, kAgentScopePolicy);
}

}  // namespace gemmf32

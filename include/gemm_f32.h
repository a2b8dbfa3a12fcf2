/*
 * gemm_f32.h - C ABI of the MI355X (gfx950) single-precision GEMM library
 * libgemm_f32.so.
 *
 * Operation (pages "GEMM 性能优化", section 指标与目标, and
 * "PMPP Chapter 06: Performance considerations", section 1, corner-turning
 * example): for 0 <= i < m and 0 <= j < n
 *
 *     C[i*ldc + j] = sum_{0 <= kk < k} A[i*lda + kk] * B(kk, j)
 *
 *     B(kk, j) = B[kk*ldb + j]   layout_b == GEMM_F32_ROW_MAJOR
 *              = B[j*ldb + kk]   layout_b == GEMM_F32_COL_MAJOR (column j contiguous)
 *
 * A (m x k) and C (m x n) are always row-major.  C is overwritten (no
 * alpha/beta, C is never read); the entries of C's row padding
 * (j >= n) are never written.  Arithmetic is IEEE float32 multiply-add with
 * float32 accumulation; the order of the k-sum is the library's (blocked
 * along k, as the block-matrix identity of "GEMM 性能优化" 台阶 1 allows)
 * and is fixed for a given plan: the same plan on the same inputs gives
 * bitwise identical results run after run (no floating-point atomics).
 *
 * Conventions for every entry point:
 *  - Return value: a gemm_f32_status code.  Nothing here throws, prints
 *    (unless GEMM_F32_LOG is set, see gemm_f32_create) or aborts.
 *  - Pointers A, B, C are device pointers (HIP device memory of the current
 *    device), owned by the caller.  C must not overlap A or B.
 *  - Sizes and leading dimensions are in elements (floats).
 *  - A plan is immutable after creation.  Plans of the tiled kernels with
 *    one tile per workgroup hold host state only and may be used from
 *    several host threads and streams at once.  Plans that split tiles
 *    along k own a device workspace (zeroed by create, freed by destroy):
 *    few-row plans with gemm_f32_info.split_k > 1 hold split_k * m * n
 *    partial sums, stream-K plans (gemm_f32_info.stream_k = P > 0: P
 *    workgroups share the k-slabs of gemm_f32_info.stream_k_tiles tiles,
 *    all of them or the partial last wave's) hold 2 * P partial tiles
 *    (bm * bn each), all as 8-byte words tagged with a per-run epoch, plus
 *    one 32-bit arrival counter per output tile and three more words (a
 *    status word, a count of finished split tiles, an epoch word).  A run
 *    launched outside graph capture takes a fresh tag from the plan (an
 *    atomic counter, so runs may be enqueued from several host threads); a
 *    launch captured in a HIP graph, whose arguments every replay repeats,
 *    takes its tag from the epoch word instead, which each such run advances
 *    when its last split tile is done, so every replay is tagged afresh.
 *    Two runs of such a plan must not execute at the same time on the device
 *    (they would share the workspace): use one plan per stream, or order the
 *    streams.
 *  - Execution is asynchronous on the caller's stream; a device-side fault
 *    is reported by the caller's next synchronisation, not by gemm_f32_run.
 */
#ifndef GEMM_F32_H
#define GEMM_F32_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct gemm_f32_plan_impl *gemm_f32_plan; /* opaque, library-owned */

/* Storage order of B (and, for the *_ex calls, of A; C is always row-major). */
enum gemm_f32_layout {
    GEMM_F32_ROW_MAJOR = 0, /* B(kk, j) = B[kk*ldb + j], needs ldb >= n; A(i, kk) = A[i*lda + kk], lda >= k */
    GEMM_F32_COL_MAJOR = 1  /* B(kk, j) = B[j*ldb + kk], needs ldb >= k; A(i, kk) = A[kk*lda + i], lda >= m */
};

enum gemm_f32_status {
    GEMM_F32_SUCCESS = 0,
    GEMM_F32_ERR_INVALID_VALUE = 1,       /* bad size, stride, layout, NULL or misaligned pointer */
    GEMM_F32_ERR_NO_DEVICE = 2,           /* no HIP device visible */
    GEMM_F32_ERR_UNSUPPORTED_DEVICE = 3,  /* current device is not gfx950 */
    GEMM_F32_ERR_HIP = 4,                 /* a HIP runtime call failed; see gemm_f32_last_hip_error */
    GEMM_F32_ERR_ALLOC = 5,               /* host allocation failed */
    GEMM_F32_ERR_SCRATCH_TOO_SMALL = 6    /* gemm_f32_run_noalloc: the partial sums exceed its scratch area */
};

/* Activation of the linear-layer epilogue (gemm_f32_run_ex). */
enum gemm_f32_activation {
    GEMM_F32_ACT_NONE = 0,  /* identity */
    GEMM_F32_ACT_RELU = 1,  /* max(x, 0) */
    GEMM_F32_ACT_GELU = 2   /* x * Phi(x) = x/2 * (1 + erf(x / sqrt(2))), Phi the normal distribution function */
};

/* Kernel families (gemm_f32_info.kind). */
enum gemm_f32_kind {
    GEMM_F32_KIND_MFMA = 0,   /* LDS-tiled, wavefront tiles on v_mfma_f32_32x32x2_f32 */
    GEMM_F32_KIND_VALU = 1,   /* LDS-tiled, per-thread register outer product on the vector ALU */
    GEMM_F32_KIND_SKINNY = 2, /* few-row path: M <= 32 (memory-bound), and shapes with few tiles */
    GEMM_F32_KIND_FEWCOL = 3  /* few-column (memory-bound, matrix-vector-like) path */
};

/* What a plan (or a variant) does; filled by gemm_f32_describe / gemm_f32_variant_info. */
struct gemm_f32_info {
    int variant;        /* index into the compiled variant table */
    int kind;           /* enum gemm_f32_kind */
    int bm, bn, bk;     /* workgroup tile (rows of C, columns of C, k per LDS stage) */
    int waves_m, waves_n; /* wavefront grid inside the workgroup */
    int wave_m, wave_n; /* output tile per wavefront */
    int threads;        /* threads per workgroup */
    int lds_bytes;      /* LDS per workgroup (all stages) */
    int stages;         /* LDS buffers along k */
    int split_k;        /* k-splits (1 = none) */
    int stream_k;       /* plan only: workgroups sharing the k-slabs of stream_k_tiles tiles evenly (stream-K), 0 = none */
    int stream_k_tiles; /* plan only: tiles whose k-slabs are shared; every other tile gets one workgroup */
    int layout_a;       /* plan only: storage order of A (enum gemm_f32_layout) */
    int epilogue;       /* plan only: 1 if built with the linear-layer epilogue */
    int aligned;        /* plan only: 1 if lda, ldb and ldc are multiples of 4 (informational) */
    int64_t tiles_m, tiles_n, k_tiles, grid; /* plan only: tile counts and workgroups launched */
    int group_m;        /* plan only: tile-rows per rasterisation group */
    int c_store_width;  /* plan only: C elements per store instruction of the whole-tile kernel
                           (2 or 4 with row-major B and N a multiple of it; else 1) */
    char name[64];      /* human-readable variant name */
    /* Resources of one kernel ("GPU 算子优化中的数据复用", section 9: spills;
     * section 12: resident workgroups are the minimum over the register, LDS
     * and wave limits), from the compiler's report of this build.  For a
     * plan: the kernel the plan launches.  For gemm_f32_variant_info: the
     * variant's whole-tile kernel for row-major A and B, except that
     * scratch_bytes is the largest over all of the variant's kernels. */
    int vgprs;              /* architectural vector registers per lane */
    int agprs;              /* accumulation vector registers per lane (MFMA accumulators) */
    int sgprs;              /* scalar registers per wavefront */
    int scratch_bytes;      /* private memory per lane for register spills (0: none) */
    int compiler_waves_per_simd; /* occupancy the compiler derives from registers and LDS */
    int workgroups_per_cu;  /* plan only: resident workgroups per CU (the HIP runtime's
                               occupancy calculator for the launched kernel) */
    int waves_per_simd;     /* plan only: workgroups_per_cu * wavefronts per workgroup / 4 */
    /* Column sliver (plan only): when the tile the dispatch picks would leave
     * a last tile-column at most an eighth full, the plan covers the first
     * n - sliver_cols columns (tiles_n, ... describe those tiles) and runs the
     * last sliver_cols columns with the few-column method: as a second launch
     * on the same stream, with a plan of its own (variant sliver_variant,
     * stream-K over sliver_stream_k workgroups), or, with sliver_fused = 1, as
     * further workgroups of the tiles' launch (grid counts them; they take the
     * slots a partly filled last wave of tiles leaves idle).  The two give
     * bitwise the same C.  sliver_cols = 0: one launch, no sliver. */
    int64_t sliver_cols;
    int sliver_variant;
    int sliver_stream_k;
    int sliver_fused;
    /* Plan only: 1 when the plan computes the transposed product
     * C^T = B^T . A^T (up to eight rows of C, column-major B: the caller's B
     * read as a row-major N x K matrix on a few-column kernel, whose loads
     * run along each column of B; "PMPP Chapter 06", section 1: the
     * corner-turning layout read along its contiguous direction), with or
     * without the linear-layer epilogue (row-major A).  The tile fields
     * then describe that product (tiles_m counts blocks of columns of C).
     * 0 otherwise. */
    int transposed;
};

/*
 * gemm_f32_validate: the pure argument check of gemm_f32_create (no HIP call).
 *   m, n, k >= 1 (a zero dimension is rejected, the pages never define it);
 *   lda >= k; ldb >= n (row-major B) or ldb >= k (column-major B); ldc >= n;
 *   layout_b in {0, 1}; every operand's byte extent below 2^31.
 * Returns GEMM_F32_SUCCESS or GEMM_F32_ERR_INVALID_VALUE.
 */
int gemm_f32_validate(int64_t m, int64_t n, int64_t k, int layout_b,
                      int64_t lda, int64_t ldb, int64_t ldc);

/*
 * gemm_f32_create: build a plan for C = A.B of the given shape, B layout and
 * leading dimensions, choosing the kernel variant by shape class.
 *   out: receives the plan (set to NULL on failure); must be non-NULL.
 * Errors: GEMM_F32_ERR_INVALID_VALUE (see gemm_f32_validate, or out == NULL),
 *         GEMM_F32_ERR_NO_DEVICE, GEMM_F32_ERR_UNSUPPORTED_DEVICE,
 *         GEMM_F32_ERR_HIP (including a failed workspace allocation),
 *         GEMM_F32_ERR_ALLOC.
 * Environment overrides, read when a plan is created (for measurement and
 * tuning; unset means the shape dispatch decides):
 *   GEMM_F32_VARIANT=<index>  force a kernel variant;
 *   GEMM_F32_GROUP_M=<rows>   tile-rows per rasterisation group (default 8);
 *   GEMM_F32_SPLIT_K=<count>  k splits of a few-row plan;
 *   GEMM_F32_SK_WGS=<P>       stream-K with P workgroups over the first
 *                             GEMM_F32_SK_TILES=<R> tiles (default all);
 *                             a partial-sum area of 2^31 bytes or more is
 *                             rejected with GEMM_F32_ERR_INVALID_VALUE;
 *   GEMM_F32_STREAMK=0        never choose stream-K automatically;
 *   GEMM_F32_SLIVER=0         never split off a column sliver (see
 *                             gemm_f32_info.sliver_cols);
 *   GEMM_F32_SLIVER_FUSE=0    run a sliver as a second launch, never in
 *                             the tiles' launch (gemm_f32_info.sliver_fused);
 *   GEMM_F32_TRANSPOSE=0      never compute a few rows of C with column-major
 *                             B as the transposed product (gemm_f32_info.transposed);
 *                             =2 (measurement) always, for up to eight rows;
 *   GEMM_F32_WIDE_C=0         store C one element at a time even where the
 *                             whole-tile kernel could store 2 or 4 (for measuring
 *                             gemm_f32_info.c_store_width);
 *   GEMM_F32_NUM_XCD=<count>  the XCD count the rasterisation undoes
 *                             (default: the device's; 1 turns the XCD
 *                             remap off, for measuring it);
 *   GEMM_F32_WAIT_BUDGET=<polls>  how long one thread waits for partial
 *                             sums before it gives up (gemm_f32_plan_check);
 *   GEMM_F32_TEST_LOST_WORDS=1  test hook: every wait for a partial sum
 *                             gives up (the split tiles of C become NaN);
 *   GEMM_F32_POISON_LDS=1     test hook: the tiled kernels fill LDS with NaN
 *                             before their first copy, so a read of LDS
 *                             before the copy that fills it lands shows up
 *                             as NaN in C;
 *   GEMM_F32_LOG=1 (or 2)     print the plan (and the dispatch's estimates)
 *                             to stderr, the one exception to "nothing
 *                             prints".
 */
int gemm_f32_create(gemm_f32_plan *out, int64_t m, int64_t n, int64_t k, int layout_b,
                    int64_t lda, int64_t ldb, int64_t ldc);

/*
 * gemm_f32_create_variant: as gemm_f32_create with an explicit variant index
 * in [0, gemm_f32_num_variants()).  Used by the tile/occupancy sweep.
 * Errors: as gemm_f32_create; an out-of-range variant is INVALID_VALUE.
 */
int gemm_f32_create_variant(gemm_f32_plan *out, int variant, int64_t m, int64_t n, int64_t k,
                            int layout_b, int64_t lda, int64_t ldb, int64_t ldc);

/*
 * gemm_f32_run: enqueue C = A.B on `stream` (a hipStream_t; NULL = the null
 * stream).  A, B, C: device pointers, 4-byte aligned, non-NULL.  Runs of 4
 * consecutive elements inside the matrices move with 16-byte accesses at any
 * 4-byte alignment; the k tail and the edge columns move element by element.
 * Odd leading dimensions and pointers that are not 16-byte aligned are not
 * errors.
 * Errors: GEMM_F32_ERR_INVALID_VALUE (NULL plan/pointer, pointer not 4-byte
 *         aligned), GEMM_F32_ERR_HIP (launch failed).  Never synchronises.
 */
int gemm_f32_run(gemm_f32_plan plan, const float *A, const float *B, float *C, void *stream);

/*
 * gemm_f32_run_noalloc: C = A.B on `stream`, as gemm_f32_create, gemm_f32_run
 * and gemm_f32_destroy with the same arguments would compute it (the same
 * plan and kernels), for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  One
 * exception: column-major B with more than two and at most two and a half
 * 128 x 128 tiles per CU and k >= 2048, where gemm_f32_create plans stream-K
 * over 128 x 128 tiles (about 192 MiB of partial sums), runs the plan the
 * dispatch takes without that rule (equal within the tolerance, not bit for
 * bit).  It calls
 * no hipMalloc, hipFree or other allocating routine, host or device; the
 * plan lives on the call's stack.  Plans that split tiles along k (the
 * few-row path's split-k, stream-K) keep their partial sums in a scratch
 * area the library reserves once on each GPU it runs on, until the process
 * ends: 64 MiB of partial-sum words and 65536 32-bit counters.
 *   Arguments: as gemm_f32_create (sizes, layout_b, leading dimensions) and
 *   gemm_f32_run (device pointers A, B, C, 4-byte aligned, C not overlapping
 *   A or B; `stream` a hipStream_t, NULL = the null stream).
 *   Every call on one GPU shares that GPU's scratch area, which keeps the
 *   last call's contents (each call clears the counters it uses, with a
 *   small kernel on `stream` ahead of the product, and tags its words
 *   afresh: with a new tag per call, or, captured in a graph, from an epoch
 *   word in the scratch area that each replay advances): two calls that
 *   overlap in time on one GPU (other streams or host threads) race and can
 *   return wrong results; order them.
 *   The first call on each device finds the scratch area's device address;
 *   make it outside graph capture.  Give-ups of the bounded waits (see
 *   gemm_f32_plan_check) write NaN to C but are not reported here.
 * Errors: as gemm_f32_create and gemm_f32_run; GEMM_F32_ERR_SCRATCH_TOO_SMALL
 *   when the plan needs more than the scratch area holds (more than 64 MiB
 *   of words or more than 65533 split tiles).  Never synchronises.
 */
int gemm_f32_run_noalloc(int64_t m, int64_t n, int64_t k, int layout_b, int64_t lda, int64_t ldb, int64_t ldc,
                         const float *A, const float *B, float *C, void *stream);

/*
 * Linear-layer layouts and epilogue.  A linear layer (the FFN and QKV
 * projections that "GEMM 性能优化" names as GEMMs in its opening) computes
 *
 *     C[i][j] = act(alpha * sum_k A(i, k) * B(k, j) + beta * C[i][j] + bias[j])
 *
 * with A(i, k) = A[i*lda + k] (layout_a == GEMM_F32_ROW_MAJOR) or
 * A[k*lda + i] (layout_a == GEMM_F32_COL_MAJOR: column k contiguous, the
 * column-major convention of "PMPP Chapter 06", section 1, applied to A),
 * B(k, j) as for gemm_f32_create.  C is read only when beta != 0 (then it
 * must hold finite values); bias holds n floats (device memory, 4-byte
 * aligned) or is NULL.  The product is summed as by gemm_f32_run; the
 * epilogue is evaluated in float32 (alpha*acc + beta*C + bias, multiply-adds
 * may be fused), then act; GELU's erf is the Abramowitz-Stegun 7.1.26
 * approximation (|error| <= 1.5e-7).  These plans run on the direct-to-LDS tiled kernels
 * (256x256, 256x128, 128x128, 64x128 or 64x64 tiles), on the few-row kernel (up to 32 rows,
 * and shapes with few tiles; either A layout), on the few-column kernels (N <= 8, row-major
 * A), as the transposed product C^T = B^T . A^T for up to eight rows with column-major B
 * (row-major A), and, for few tiles with a long k and row-major A, on stream-K over 64x64
 * tiles, and with column-major B, row-major A and k >= 3072 where 128x128 tiles number
 * two to two and a half per CU, on stream-K over those tiles; the epilogue is applied where
 * each kernel writes C.
 */

/* gemm_f32_validate_ex: gemm_f32_validate with A's layout: lda >= k (row-major
 * A) or lda >= m (column-major A); layout_a in {0, 1}. */
int gemm_f32_validate_ex(int64_t m, int64_t n, int64_t k, int layout_a, int layout_b,
                         int64_t lda, int64_t ldb, int64_t ldc);

/*
 * gemm_f32_create_ex: a plan with A's layout and, with epilogue = 1, the
 * linear-layer epilogue (then run it with gemm_f32_run_ex).  epilogue = 0
 * gives plain C = A.B.  Errors: as gemm_f32_create (INVALID_VALUE also for
 * epilogue not in {0, 1}).
 */
int gemm_f32_create_ex(gemm_f32_plan *out, int64_t m, int64_t n, int64_t k, int layout_a, int layout_b,
                       int64_t lda, int64_t ldb, int64_t ldc, int epilogue);

/*
 * gemm_f32_run_ex: enqueue C = act(alpha * A.B + beta * C + bias) on
 * `stream`.  activation: enum gemm_f32_activation.  A plan created without
 * the epilogue accepts only alpha = 1, beta = 0, bias = NULL, activation =
 * GEMM_F32_ACT_NONE (plain C = A.B); gemm_f32_run on an epilogue plan is the
 * same as those values.  Errors: as gemm_f32_run, plus INVALID_VALUE for an
 * unknown activation, a misaligned bias, or epilogue values on a plan
 * without it.  Never synchronises.
 */
int gemm_f32_run_ex(gemm_f32_plan plan, const float *A, const float *B, float *C, float alpha, float beta,
                    const float *bias, int activation, void *stream);

/* gemm_f32_destroy: release a plan and its workspace (hipFree, which waits
 * for the device).  NULL is a no-op returning SUCCESS. */
int gemm_f32_destroy(gemm_f32_plan plan);

/* gemm_f32_describe: copy the plan's choices into *info (both non-NULL). */
int gemm_f32_describe(gemm_f32_plan plan, struct gemm_f32_info *info);

/*
 * gemm_f32_plan_check: whether a run of the plan since the last check gave
 * up waiting for another workgroup's partial sums.  Plans that split tiles
 * along k (split_k > 1 or stream_k > 0) add the splits in the last
 * workgroup of each tile to arrive; its wait for each word is bounded so
 * that a lost word can never hang the kernel, and when a wait gives up that
 * element of C is written as NaN and the plan's status word records it.
 * *lost receives 1 if that happened (and the record is cleared), else 0;
 * plans without a workspace always report 0.  Call it after synchronising
 * the streams the plan ran on (it reads device memory with a blocking copy).
 * Errors: INVALID_VALUE (NULL plan or lost), ERR_HIP.
 */
int gemm_f32_plan_check(gemm_f32_plan plan, int *lost);

/* gemm_f32_num_variants: number of entries in the compiled variant table. */
int gemm_f32_num_variants(void);

/* gemm_f32_variant_info: static description of variant `variant` (no device
 * needed; the plan-only fields are zero).  INVALID_VALUE if out of range. */
int gemm_f32_variant_info(int variant, struct gemm_f32_info *info);

/* gemm_f32_error_string: static text for a status code (never NULL). */
const char *gemm_f32_error_string(int status);

/* gemm_f32_last_hip_error: the hipError_t behind the calling thread's most
 * recent GEMM_F32_ERR_HIP (0 if none). */
int gemm_f32_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_F32_H */

// Host side of libgemm_f32.so: argument validation, the compiled variant
// table, shape dispatch, plans and launches.  The C ABI is declared in
// include/gemm_f32.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>

#include <dlfcn.h>

#include "gemm_f32.h"
#include "kernel_list.hpp"
#include "kernel_resources.hpp"

// The kernels are compiled in the k_*.hip units; this unit only takes their
// handles.
GEMMF32_ALL_UNITS(GEMMF32_EXTERN5, GEMMF32_EXTERN2, GEMMF32_EXTERN1)

// Scratch of gemm_f32_run_noalloc: the arrival counters of the split tiles,
// the status word and the count of finished split tiles first (the epoch
// word, shared by every call, is the area's last counter), then the
// epoch-tagged partial-sum words.  One copy per GPU, reserved until the
// process ends; every call on a GPU shares it.  Host code never uses this
// name as an address: it takes the device address from hipGetSymbolAddress,
// once per device (scratch_address).
namespace {
constexpr size_t kScratchCounters = 65536;             // 32-bit counters (see above)
constexpr size_t kScratchWordBytes = (size_t)64 << 20;  // 64 MiB of 8-byte words
constexpr size_t kScratchBytes = kScratchCounters * 4 + kScratchWordBytes;
}  // namespace
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

using gemmf32::GemmArgs;

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e)
{
    g_last_hip_error = static_cast<int>(e);
    return GEMM_F32_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Variant table
// ---------------------------------------------------------------------------

struct VariantDesc {
    const char *name;
    int kind;
    int bm, bn, bk;
    int waves_m, waves_n;
    int threads;
    int lds_bytes;
    int stages;
    const void *fn[2];     // [column-major B]
    const void *fn_sk[2];  // stream-K kernels (tiles' k-slabs shared across workgroups), or NULL
    const void *fn_ex[2][2][2];  // [column-major A][column-major B][epilogue], or NULL
    const void *fn_wide[2][2];  // [column-major A][epilogue]: row-major B, C stored NB columns
                                // at a time (N a multiple of NB), or NULL
    const void *fn_sliver[2];   // [column-major B]: whole tiles carrying a column sliver, or NULL
    const void *fn_sliver_wide; // the same with the wide C stores, or NULL
    const void *fn_t;           // few-column: the transposed product C^T = B^T A^T for
                                // column-major B (gemm_fewcol_t_kernel), or NULL
    const void *fn_t_epi;       // the same with the linear-layer epilogue, or NULL
    const void *fn_sk_epi[2];   // [column-major B]: stream-K with the linear-layer epilogue
                                // (row-major A), or NULL
};

template <class T>
VariantDesc mfma_variant(const char *name)
{
    return VariantDesc{
        name, GEMM_F32_KIND_MFMA, T::BM, T::BN, T::BK, T::WAVES_M, T::WAVES_N, T::THREADS, T::LDS_BYTES, 2,
        {reinterpret_cast<const void *>(&gemmf32::gemm_mfma_kernel<T, false>),
         reinterpret_cast<const void *>(&gemmf32::gemm_mfma_kernel<T, true>)}};
}

template <class T>
VariantDesc dma_variant(const char *name)
{
    VariantDesc d{
        name, GEMM_F32_KIND_MFMA, T::BM, T::BN, T::BK, T::WAVES_M, T::WAVES_N, T::THREADS, T::LDS_BYTES, T::STAGES,
        {reinterpret_cast<const void *>(&gemmf32::gemm_mfma_dma_kernel<T, false>),
         reinterpret_cast<const void *>(&gemmf32::gemm_mfma_dma_kernel<T, true>)},
        {reinterpret_cast<const void *>(&gemmf32::gemm_mfma_dma_sk_kernel<T, false>),
         reinterpret_cast<const void *>(&gemmf32::gemm_mfma_dma_sk_kernel<T, true>)}};
    if constexpr (T::NB == 2 || T::NB == 4)
        d.fn_wide[0][0] = reinterpret_cast<const void *>(&gemmf32::gemm_mfma_dma_kernel<T, false, false, false, true>);
    return d;
}

// A DMA variant that also serves column-major A and the linear-layer
// epilogue.
template <class T>
VariantDesc dma_ex_variant(const char *name)
{
    using namespace gemmf32;
    VariantDesc d = dma_variant<T>(name);
    d.fn_ex[0][0][0] = reinterpret_cast<const void *>(&gemm_mfma_dma_kernel<T, false, false, false>);
    d.fn_ex[0][1][0] = reinterpret_cast<const void *>(&gemm_mfma_dma_kernel<T, true, false, false>);
    d.fn_ex[1][0][0] = reinterpret_cast<const void *>(&gemm_mfma_dma_kernel<T, false, true, false>);
    d.fn_ex[1][1][0] = reinterpret_cast<const void *>(&gemm_mfma_dma_kernel<T, true, true, false>);
    d.fn_ex[0][0][1] = reinterpret_cast<const void *>(&gemm_mfma_dma_kernel<T, false, false, true>);
    d.fn_ex[0][1][1] = reinterpret_cast<const void *>(&gemm_mfma_dma_kernel<T, true, false, true>);
    d.fn_ex[1][0][1] = reinterpret_cast<const void *>(&gemm_mfma_dma_kernel<T, false, true, true>);
    d.fn_ex[1][1][1] = reinterpret_cast<const void *>(&gemm_mfma_dma_kernel<T, true, true, true>);
    if constexpr (T::NB == 2 || T::NB == 4) {
        d.fn_wide[1][0] = reinterpret_cast<const void *>(&gemm_mfma_dma_kernel<T, false, true, false, true>);
        d.fn_wide[0][1] = reinterpret_cast<const void *>(&gemm_mfma_dma_kernel<T, false, false, true, true>);
        d.fn_wide[1][1] = reinterpret_cast<const void *>(&gemm_mfma_dma_kernel<T, false, true, true, true>);
    }
    return d;
}

// Stream-K with the linear-layer epilogue: the two-stage 64 x 64 tile (the
// few-tile long-k plans of epilogue plans with row-major A) and the 128 x
// 128 tile (column-major B short of three tiles per CU).
template <class T>
VariantDesc with_sk_epi(VariantDesc d)
{
    d.fn_sk_epi[0] = reinterpret_cast<const void *>(&gemmf32::gemm_mfma_dma_sk_epi_kernel<T, false>);
    d.fn_sk_epi[1] = reinterpret_cast<const void *>(&gemmf32::gemm_mfma_dma_sk_epi_kernel<T, true>);
    return d;
}

// The 128 x 128 candidate: also the kernels that carry a column sliver.
template <class T>
VariantDesc with_sliver(VariantDesc d)
{
    using namespace gemmf32;
    d.fn_sliver[0] = reinterpret_cast<const void *>(&gemm_mfma_dma_sliver_kernel<T, false>);
    d.fn_sliver[1] = reinterpret_cast<const void *>(&gemm_mfma_dma_sliver_kernel<T, true>);
    if constexpr (T::NB == 2 || T::NB == 4)
        d.fn_sliver_wide = reinterpret_cast<const void *>(&gemm_mfma_dma_sliver_kernel<T, false, false, false, true>);
    return d;
}

template <class T>
VariantDesc fewcol_variant(const char *name)
{
    VariantDesc d{
        name, GEMM_F32_KIND_FEWCOL, T::ROWS, T::R, T::KC, T::WAVES, 1, T::THREADS, T::LDS_BYTES, 1,
        {reinterpret_cast<const void *>(&gemmf32::gemm_fewcol_kernel<T, false>),
         reinterpret_cast<const void *>(&gemmf32::gemm_fewcol_kernel<T, true>)}};
    // The linear-layer epilogue with row-major A.
    d.fn_ex[0][0][1] = reinterpret_cast<const void *>(&gemmf32::gemm_fewcol_epi_kernel<T, false>);
    d.fn_ex[0][1][1] = reinterpret_cast<const void *>(&gemmf32::gemm_fewcol_epi_kernel<T, true>);
    if constexpr (T::R == 1 || (T::R == 4 && T::KC == 1024) || T::ROWS_PER_WAVE == 1) {
        d.fn_t = reinterpret_cast<const void *>(&gemmf32::gemm_fewcol_t_kernel<T, true>);
        d.fn_t_epi = reinterpret_cast<const void *>(&gemmf32::gemm_fewcol_t_epi_kernel<T, true>);
    }
    return d;
}

template <class T>
VariantDesc skinny_variant(const char *name)
{
    VariantDesc d{
        name, GEMM_F32_KIND_SKINNY, T::BM, T::BN, T::KQ, 1, T::WAVES, T::THREADS, T::WAVES * T::BM * T::BN * 4, 1,
        {reinterpret_cast<const void *>(&gemmf32::gemm_skinny_kernel<T, false>),
         reinterpret_cast<const void *>(&gemmf32::gemm_skinny_kernel<T, true>)}};
    // Column-major A and the linear-layer epilogue.
    d.fn_ex[0][0][1] = reinterpret_cast<const void *>(&gemmf32::gemm_skinny_epi_kernel<T, false>);
    d.fn_ex[0][1][1] = reinterpret_cast<const void *>(&gemmf32::gemm_skinny_epi_kernel<T, true>);
    d.fn_ex[1][0][0] = reinterpret_cast<const void *>(&gemmf32::gemm_skinny_acol_kernel<T, false>);
    d.fn_ex[1][1][0] = reinterpret_cast<const void *>(&gemmf32::gemm_skinny_acol_kernel<T, true>);
    d.fn_ex[1][0][1] = reinterpret_cast<const void *>(&gemmf32::gemm_skinny_acol_epi_kernel<T, false>);
    d.fn_ex[1][1][1] = reinterpret_cast<const void *>(&gemmf32::gemm_skinny_acol_epi_kernel<T, true>);
    return d;
}

VariantDesc valu_variant(const char *name)
{
    using T = gemmf32::ValuTile;
    return VariantDesc{
        name, GEMM_F32_KIND_VALU, T::BM, T::BN, T::BK, 4, 1, T::THREADS, T::LDS_BYTES, 2,
        {reinterpret_cast<const void *>(&gemmf32::gemm_valu_kernel<false>),
         reinterpret_cast<const void *>(&gemmf32::gemm_valu_kernel<true>)}};
}

enum VariantId {
    V_MFMA_256x256x16 = 0,
    V_MFMA_128x128x16,
    V_MFMA_256x128x16,
    V_VALU_128x128x8,
    V_MFMA_256x128x32,
    V_MFMA_128x128x32,
    V_DMA_256x256x16_S2,
    V_DMA_256x256x16_S3,
    V_DMA_256x256x16_S4,
    V_DMA_256x256x32_S2,
    V_DMA_128x128x16_S3,
    V_DMA_128x128x32_S3,
    V_DMA_256x128x16_S3,
    V_SKINNY_W4_D4,
    V_SKINNY_W8_D4,
    V_DMA_64x64x16_S3,
    V_SKINNY_W16_D4,
    V_SKINNY16_W16_D4,
    V_DMA_64x64x16_S2,
    V_DMA_128x64x16_S2,
    V_DMA_128x64x16_S3,
    V_DMA_64x128x16_S2,
    V_DMA_64x128x16_S3,
    V_FEWCOL_R1,
    V_FEWCOL_R4,
    V_FEWCOL_R8,
    V_DMA_256x256x16_W24_S4,
    V_DMA_256x256x16_W42_S4,
    V_DMA_256x256x16_W42_S2,
    V_DMA_256x256x16_W44_S4,
    V_SKINNY32_W8_D4,
    V_SKINNY_16x32_W16_D4,
    V_FEWCOL_R4_K1024,
    V_SKINNY16_W4_D4,
    V_FEWCOL_R1_W8,
    V_FEWCOL_R8_W8,
    V_COUNT
};

const VariantDesc &variant(int v)
{
    using gemmf32::DmaTile;
    using gemmf32::MfmaTile;
    using gemmf32::SkinnyTile;
    static const VariantDesc table[V_COUNT] = {
        mfma_variant<MfmaTile<256, 256, 16, 2, 2>>("mfma_256x256x16_w2x2_32x32x2"),
        mfma_variant<MfmaTile<128, 128, 16, 2, 2>>("mfma_128x128x16_w2x2_32x32x2"),
        mfma_variant<MfmaTile<256, 128, 16, 2, 2>>("mfma_256x128x16_w2x2_32x32x2"),
        valu_variant("valu_128x128x8_t8x8"),
        mfma_variant<MfmaTile<256, 128, 32, 2, 2>>("mfma_256x128x32_w2x2_32x32x2"),
        mfma_variant<MfmaTile<128, 128, 32, 2, 2>>("mfma_128x128x32_w2x2_32x32x2"),
        dma_variant<DmaTile<256, 256, 16, 2, 2, 2>>("dma_256x256x16_w2x2_s2"),
        dma_variant<DmaTile<256, 256, 16, 2, 2, 3>>("dma_256x256x16_w2x2_s3"),
        dma_ex_variant<DmaTile<256, 256, 16, 2, 2, 4>>("dma_256x256x16_w2x2_s4"),
        dma_variant<DmaTile<256, 256, 32, 2, 2, 2>>("dma_256x256x32_w2x2_s2"),
        with_sk_epi<DmaTile<128, 128, 16, 2, 2, 3, false>>(with_sliver<DmaTile<128, 128, 16, 2, 2, 3, false>>(
            dma_ex_variant<DmaTile<128, 128, 16, 2, 2, 3, false>>("dma_128x128x16_w2x2_s3"))),
        dma_variant<DmaTile<128, 128, 32, 2, 2, 3, false>>("dma_128x128x32_w2x2_s3"),
        dma_ex_variant<DmaTile<256, 128, 16, 2, 2, 3>>("dma_256x128x16_w2x2_s3"),
        skinny_variant<SkinnyTile<4, 4, 64>>("skinny_16x64_w4_d4"),
        skinny_variant<SkinnyTile<8, 4, 64>>("skinny_16x64_w8_d4"),
        dma_ex_variant<DmaTile<64, 64, 16, 2, 2, 3>>("dma_64x64x16_w2x2_s3"),
        skinny_variant<SkinnyTile<16, 4, 64>>("skinny_16x64_w16_d4"),
        skinny_variant<SkinnyTile<16, 4, 16>>("skinny_16x16_w16_d4"),
        with_sk_epi<DmaTile<64, 64, 16, 2, 2, 2>>(dma_ex_variant<DmaTile<64, 64, 16, 2, 2, 2>>("dma_64x64x16_w2x2_s2")),
        dma_variant<DmaTile<128, 64, 16, 2, 2, 2>>("dma_128x64x16_w2x2_s2"),
        dma_variant<DmaTile<128, 64, 16, 2, 2, 3>>("dma_128x64x16_w2x2_s3"),
        dma_ex_variant<DmaTile<64, 128, 16, 2, 2, 2>>("dma_64x128x16_w2x2_s2"),
        dma_variant<DmaTile<64, 128, 16, 2, 2, 3>>("dma_64x128x16_w2x2_s3"),
        fewcol_variant<gemmf32::FewColR1>("fewcol_8x1_k2048"),
        fewcol_variant<gemmf32::FewColR4>("fewcol_8x4_k2048"),
        fewcol_variant<gemmf32::FewColR8>("fewcol_8x8_k1024"),
        dma_variant<DmaTile<256, 256, 16, 2, 4, 4>>("dma_256x256x16_w2x4_s4"),
        dma_ex_variant<DmaTile<256, 256, 16, 4, 2, 4>>("dma_256x256x16_w4x2_s4"),
        dma_variant<DmaTile<256, 256, 16, 4, 2, 2>>("dma_256x256x16_w4x2_s2"),
        dma_variant<DmaTile<256, 256, 16, 4, 4, 4>>("dma_256x256x16_w4x4_s4"),
        skinny_variant<SkinnyTile<8, 4, 64, 2>>("skinny_32x64_w8_d4"),
        skinny_variant<SkinnyTile<16, 4, 32>>("skinny_16x32_w16_d4"),
        fewcol_variant<gemmf32::FewColR4K1024>("fewcol_8x4_k1024"),
        skinny_variant<SkinnyTile<4, 4, 16>>("skinny_16x16_w4_d4"),
        fewcol_variant<gemmf32::FewColR1W8>("fewcol_8x1_k2048_w8"),
        fewcol_variant<gemmf32::FewColR8W8>("fewcol_8x8_k1024_w8"),
    };
    return table[v];
}

// ---------------------------------------------------------------------------
// Device facts, queried once per device
// ---------------------------------------------------------------------------

// The tiled variants the shape dispatch weighs against each other, with the
// throughput each sustains while every slot of a wave is busy (TFLOPS on one
// MI355X: 256x128 on 4096^3 (147.2-148.5) and the FFN shape (148.8-149.2),
// 128x128 on 6144^3 (three whole waves, 147.8-148.6; FFN 149.1-149.4), 64x128
// and 64x64 (two LDS stages, four and eight workgroups per CU) on 4096^3
// (two whole waves: 145.2-145.5, 136.2-138.4)), and the share of a CU's throughput
// that a lone workgroup gets (one wavefront per SIMD: 256x128 from 2048^3,
// 128 tiles; 128x128 from 2048^3, 256 tiles; the others taken as 0.92).
// 128x128 is rated a point below its measurements, 64x64 one or two below
// (on large operands 64x64 ran 120.6-127.3 where 64x128 ran 125.3-132.4:
// 7592x7093x6144, 6569x5664x6144, 3645x5638x6144) and 64x128 three below
// (rated at 145 it took shapes from 128x128 that 128x128 runs 4 % faster),
// which ranks them right on the validation shapes.
struct Candidate {
    int variant;
    double full_tflops;
    double lone_share;
    double tail_extra;  // waves added to a last wave that follows full waves
    bool packed_tail;   // a last wave after full waves comes back two workgroups per CU
    double tail_sk;     // waves a stream-K last wave costs beyond its FLOPs (0: not used for this tile)
    int tail_sk_min_k;  // ... from this k on
    bool col_b = true;  // weighed for column-major B too
    bool epi = true;    // weighed for the linear-layer epilogue too
};
// tail_extra: 64x64 tails after full waves ran 0.03 to 0.09 of a wave over
// the count (8 tiles: 0.17 against 0.14, 161: 0.23 against 0.14, 512: 0.32
// against 0.25).
// 256x256 holds one workgroup per CU, so its waves quantise coarsely, but on
// whole waves it leads.  Its eight wavefronts (4 x 2, 64 x 128 each, two per
// SIMD) run ahead of four (2 x 2, 128 x 128, one per SIMD), whose stalls at
// the slab barrier and LDS reads nothing covers (one MI355X, TFLOPS, median
// of three interleaved runs; 8 waves / 4 waves / 256x128): 4096^3 149.3 /
// 148.6 / 148.1, FFN 150.7 / 149.8 / 149.6, column-major B 149.9 / 145.6 /
// 147.3; column-major A 4096^3 148.7 / 146.8-147.3 / 145.5-146.1, FFN 149.6
// / 148.2-148.5 / 147.2-147.4; bias + GELU epilogue, FFN 147.9-148.2 /
// 145.9-146.1 / 145.7-145.8, column-major B 146.6-146.9 / 141.3 / 144.1-144.3.
// So it is weighed for every layout and for the epilogue.
constexpr int kCandidates = 5;
constexpr Candidate kCandidate[kCandidates] = {{V_DMA_256x128x16_S3, 147.5, 0.94, 0.0, true, 0.25, 4096},
                                               {V_DMA_128x128x16_S3, 147.0, 0.91, 0.0, false, 0.0, 0},
                                               {V_DMA_64x128x16_S2, 142.0, 0.92, 0.0, true, 0.1, 2048},
                                               {V_DMA_64x64x16_S2, 136.0, 0.92, 0.05, false, 0.0, 0},
                                               {V_DMA_256x256x16_W42_S4, 149.5, 1.0, 0.0, false, 0.0, 0}};

struct DeviceFacts {
    int status = -1;  // -1: not queried yet, else a gemm_f32_status
    int cu_count = 0;
    int num_xcd = 1;
    int hip_error = 0;
    int per_cu[kCandidates] = {};       // resident workgroups per CU of each candidate's kernel
    int per_cu_wide[kCandidates] = {};  // the same for its wide-store kernel (0: none)
    int per_cu_sk[kCandidates][2] = {}; // the same for its stream-K kernel, by B layout
};

constexpr int kMaxDevices = 64;
DeviceFacts g_devices[kMaxDevices];
std::mutex g_devices_mutex;

int device_facts(int *device_out, DeviceFacts *facts_out)
{
    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    if (e == hipErrorNoDevice || (e == hipSuccess && count == 0)) {
        (void)hipGetLastError();
        return GEMM_F32_ERR_NO_DEVICE;
    }
    if (e != hipSuccess) return hip_fail(e);
    int dev = 0;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= kMaxDevices) return GEMM_F32_ERR_UNSUPPORTED_DEVICE;

    std::lock_guard<std::mutex> lock(g_devices_mutex);
    DeviceFacts &f = g_devices[dev];
    if (f.status < 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return hip_fail(e);
        if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
            f.status = GEMM_F32_ERR_UNSUPPORTED_DEVICE;
        } else {
            f.cu_count = prop.multiProcessorCount;
            int xcc = 0;
            if (hipDeviceGetAttribute(&xcc, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || xcc < 1) {
                (void)hipGetLastError();
                xcc = 1;  // the rasterisation stays a bijection for any count
            }
            f.num_xcd = xcc;
            for (int i = 0; i < kCandidates; ++i) {
                const VariantDesc &d = variant(kCandidate[i].variant);
                int n = 0;
                if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, d.fn[0], d.threads, 0) != hipSuccess || n < 1) {
                    (void)hipGetLastError();
                    n = 1;
                }
                f.per_cu[i] = n;
                // The wide-store kernel may hold a few more registers and
                // fit fewer workgroups (64x128: four against five).
                int w = 0;
                if (d.fn_wide[0][0] &&
                    (hipOccupancyMaxActiveBlocksPerMultiprocessor(&w, d.fn_wide[0][0], d.threads, 0) != hipSuccess ||
                     w < 1)) {
                    (void)hipGetLastError();
                    w = n;
                }
                f.per_cu_wide[i] = w;
                for (int b = 0; b < 2; ++b) {
                    int sk = 0;
                    if (d.fn_sk[b] &&
                        (hipOccupancyMaxActiveBlocksPerMultiprocessor(&sk, d.fn_sk[b], d.threads, 0) != hipSuccess ||
                         sk < 1)) {
                        (void)hipGetLastError();
                        sk = n;
                    }
                    f.per_cu_sk[i][b] = sk;
                }
            }
            f.status = GEMM_F32_SUCCESS;
        }
    }
    *device_out = dev;
    *facts_out = f;
    return f.status;
}

// ---------------------------------------------------------------------------
// Plans
// ---------------------------------------------------------------------------

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int env_int(const char *name, int fallback)
{
    const char *s = std::getenv(name);
    if (!s || !*s) return fallback;
    char *end = nullptr;
    long v = std::strtol(s, &end, 10);
    if (end == s) return fallback;
    return static_cast<int>(v);
}

}  // namespace

struct gemm_f32_plan_impl {
    int variant;
    int device;
    int layout_a;
    int layout_b;
    int epilogue;        // 1: built with the linear-layer epilogue (gemm_f32_run_ex)
    const void *fn;      // the kernel run launches
    int64_t m, n, k, lda, ldb, ldc;
    bool strides4;       // every leading dimension is a multiple of 4 (informational)
    GemmArgs args;       // pointers filled at run time
    unsigned grid;
    unsigned block;
    void *workspace;     // split-k partial sums and arrival counters (few-row path), else NULL
    std::atomic<unsigned> runs{0};   // argument tags handed out so far
    int c_store_width = 1;           // C elements per store of the whole-tile kernel
    // Column sliver: the last sliver_cols columns of C run as a second launch
    // with a plan of their own (this plan then covers columns [0, n)), or,
    // with sliver_fused, as further workgroups of this plan's launch.
    gemm_f32_plan_impl *sliver = nullptr;
    int64_t sliver_col0 = 0;
    bool sliver_fused = false;
    // The kernel computes C^T = B^T A^T: its A is the caller's B and its B
    // the caller's A (args describe the product the kernel computes).
    bool swap_ab = false;
};

namespace {

// Estimated time of a plan ("GEMM 性能优化", Wave 模型): the tiles run in
// waves of S = (workgroups per CU) x CUs = c x CUs; a full wave takes S
// tiles' FLOPs at the variant's full-wave throughput.  The last, partial
// wave of r tiles: w = ceil(r / CUs) workgroups per CU take w/c of a wave,
// and a lone workgroup (w = 1) gets only lone_share of its CU, its four
// wavefronts having nothing to cover their waits.  After full waves, the
// tails of 256x128 (c = 2) and 64x128 (c = 4 or 5) come back packed: the
// workgroups of a CU finish together, and the CUs that free up first take
// two each, so such a tail is charged at least two per CU (measured at
// k = 4096: 64 to 256 tail tiles of 256x128 took 0.5 to 1.0 of a wave,
// mostly the whole; 104 and 256 of 64x128 half).  128x128 (c = 3), whose
// slabs run at normal wavefront priority, no longer packs since its copies
// dropped the k check: 186 and 192 tail tiles after two full waves cost
// 0.36-0.37 of a wave (5239x5308x4096 and 4578x6085x4096, 140.4 and 140.5
// TFLOPS, against two thirds of a wave before, 120.6 and 119.8); built with
// the raised priority it packs again (4096^3: 145.0 -> 117.8).  A handful of tail tiles
// (at most one per eight CUs) run alone instead (one 256x128 tile: half a
// wave; four 64x128 tiles: 0.28 of one).  With c = 8 (64x64) the workgroups
// of a CU finish staggered and tails overlap the last full wave (8 tail
// tiles cost 0.17 of a wave, 161 tiles 0.23).
// Stream-K tail: the whole plan runs in the stream-K kernel, whose
// occupancy c' may differ; when its last wave has at most one tile per CU,
// those tiles' k-slabs may be split evenly over one workgroup per CU (at
// most 8 per tile) while the others run whole.  Estimated at the plan's
// FLOPs at the full-wave rate plus tail_sk of a wave (c' x CUs tiles) for
// the partial sums and the imbalance.  256x128 from k = 4096 (0.25; measured
// 0.12 to 0.24): 4096x5120x4096 103.5 -> 132.3 TFLOPS, 4096x6144x4096
// 110.2 -> 132.6, 2304x9216x4096 101.9 -> 128.6 against data-parallel
// 256x128.  64x128 from k = 2048 (0.1; measured 0.04 at k = 4096, 0.11 at
// 2049): 4608x4608x4096 131.3 -> 139.0, 5003x4097x2049 123.6 -> 128.4.
// (128x128 lost with one tile per split: 2048x14336x4096 126.1 -> 116.8;
// 64x64 tails, which overlap the last full wave, did not gain.)  On 29
// validation shapes (one MI355X, 21 of them random in [512, 8192]^2 x {1024,
// 2048, 3000, 4096}) every data-parallel choice came within 0.8 % of the
// fastest candidate, and the stream-K tails chosen beat every
// data-parallel plan by 3-7 %.
double estimate_seconds(const Candidate &cand, int per_cu, int per_cu_sk, int64_t m, int64_t n, int64_t k, int cus,
                        bool tail_ok, int64_t *tail_tiles)
{
    const VariantDesc &d = variant(cand.variant);
    const int64_t tiles = ceil_div(m, d.bm) * ceil_div(n, d.bn);
    const int64_t slots = (int64_t)per_cu * cus;
    const int64_t full = tiles / slots, rem = tiles % slots;
    const double wave = (double)slots * 2.0 * d.bm * d.bn * (double)k / (cand.full_tflops * 1e12);
    *tail_tiles = 0;
    double last = 0.0;
    if (rem) {
        int64_t w = std::min<int64_t>(per_cu, ceil_div(rem, cus));
        if (full >= 1 && cand.packed_tail && rem > cus / 8) w = std::min<int64_t>(per_cu, std::max<int64_t>(w, 2));
        last = (double)w / per_cu;
        if (w == 1 && per_cu > 1) last /= cand.lone_share;
        if (full >= 1) last += cand.tail_extra;
    }
    const double dp = ((double)full + last) * wave;
    if (tail_ok && cand.tail_sk > 0.0 && k >= cand.tail_sk_min_k && per_cu_sk > 0) {
        const int64_t s_slots = (int64_t)per_cu_sk * cus;
        const int64_t s_full = tiles / s_slots, s_rem = tiles % s_slots;
        if (s_full >= 1 && s_rem > 0 && s_rem <= cus) {
            const double s_wave = (double)s_slots * 2.0 * d.bm * d.bn * (double)k / (cand.full_tflops * 1e12);
            const double hybrid = ((double)tiles / s_slots + cand.tail_sk) * s_wave;
            if (hybrid < dp) {
                *tail_tiles = s_rem;
                return hybrid;
            }
        }
    }
    return dp;
}

// Few tiles on the few-row kernel.  When the tiled plans leave most CUs
// idle, 16-row tiles give 4 to 16 times as many workgroups as 64 x 64 tiles,
// and the k split over a workgroup's wavefronts keeps all four SIMDs of each
// CU on one tile ("GEMM 性能优化", Wave 模型: a wave that fills the GPU).
// T16 / T64: the number of 16 x 16 / 16 x 64 tiles.  16 x 16 tiles while
// T16 <= CUs (k < 2048, or T16 <= CUs / 2 with the k split over up to 8
// workgroups that bring the grid to one workgroup per CU; at most 3072 k per
// tile otherwise); then 16 x 64 tiles with 16 wavefronts and the same k
// split; then 16 x 64 tiles with 8 wavefronts while T64 is within one
// workgroup per CU, or three for k in [512, 4096] (row-major B; column-major
// B, whose columns the few-row kernel reads less evenly, up to one, and only
// to k = 3584 unless T64 <= CUs / 2).  The row tiles of a column of tiles
// run side by side on one XCD (gemm_skinny_kernel), so B, read once per 16
// rows, comes from that XCD's L2 after the first.  Measured on one MI355X
// (us, this rule's plan / the tiled or stream-K plan it replaces):
// 256x256x256 5.5 / 7.6, 128x512x1024 5.6 / 21.2, 64x256x4096 6.8 / 25.4,
// 128x512x4096 10.2 / 26.6, 256x256x16384 23.9 / 80.7, 300x700x1500 12.0 /
// 42.3, 640x320x1024 7.7 / 21.3, 512x512x8192 39.9 / 54.0, 800x600x3000
// 33.8 / 44.7, 768x768x1024 17.7 / 28.3; row-major B, k in (2048, 4096]:
// 128x4096x4096 42.4 / 55.5, 160x4096x4096 57.2 / 70.4, 96x8192x4096 73.7 /
// 87.5, 768x768x4096 57.7 / 62.9, 192x4096x3000 45.4 / 51.0, 1000x600x4000
// 61.9 / 59.4 (the one loss); the tiled plans stay ahead from 1024x1024
// (1024 tiles of 16 x 64).  Returns the variant and *split, its k-split
// count, or -1.
// The few-tile, long-k rule of the shape dispatch (below).
bool few_tile_stream_k(int64_t m, int64_t n, int64_t k, const DeviceFacts &f, bool tail_ok)
{
    return tail_ok && 2 * ceil_div(m, 64) * ceil_div(n, 64) < 5 * (int64_t)f.cu_count && k >= 2048;
}

int few_tile_rows(int64_t m, int64_t n, int64_t k, int layout_b, const DeviceFacts &f, int *split)
{
    const int64_t cus = f.cu_count;
    const int64_t t16 = ceil_div(m, 16) * ceil_div(n, 16);
    const int64_t t64 = ceil_div(m, 16) * ceil_div(n, 64);
    auto fill = [&](int64_t tiles) { return (int)std::max<int64_t>(1, std::min<int64_t>(8, cus / tiles)); };
    // (16 x 16 tiles without a k split across workgroups run four
    // wavefronts: fewer waves to launch on these latency-bound shapes.
    // Measured on one MI355X, us, four / sixteen wavefronts, row-major then
    // column-major B: 256x256x256 3.04 / 3.57, 3.18 / 3.78; 200x300x256
    // 3.19 / 3.60; 128x256x512 3.26 / 3.76, 3.93 / 4.41; 128x128x1536 5.45 /
    // 6.15; 256x256x1024 4.38 / 4.52; 256x256x2048 6.49 / 6.77, 9.05 / 9.14;
    // 256x256x64 3.23 / 3.19.)
    if (2 * t16 <= cus) {
        if (k < 2048) {
            *split = 1;
            return V_SKINNY16_W4_D4;
        }
        *split = fill(t16);
        return V_SKINNY16_W16_D4;
    }
    if (t16 <= cus && k <= 3072) {
        *split = 1;
        return V_SKINNY16_W4_D4;
    }
    if (t16 <= cus) {
        *split = fill(t64);
        return V_SKINNY_W16_D4;
    }
    // (Column-major B with CUs / 2 < T64 <= CUs: up to k = 3584, where the
    // few-row plan with one split was measured ahead of stream-K over 64 x 64
    // tiles, us: 250x600x2500 18.9 / 28.6, 240x1000x2200 19.9 / 29.2,
    // 160x1536x3000 26.3 / 36.5, 128x2048x3000 26.6 / 32.5, 200x700x3000
    // 26.9 / 30.9, 180x900x3500 31.2 / 33.6; at k = 4096 stream-K kept its
    // lead or tied: 256x1024x4096 37.1 / 35.3, 300x500x4096 37.2 / 34.8.)
    const bool w8 = layout_b == GEMM_F32_ROW_MAJOR ? t64 <= cus || (t64 <= 3 * cus && k >= 512 && k <= 4096)
                                                   : 2 * t64 <= cus || (t64 <= cus && k <= 3584);
    if (w8) {
        *split = k < 2048 ? 1 : fill(t64);
        return V_SKINNY_W8_D4;
    }
    return -1;
}

// Up to four rows of C and column-major B (y = W x for a few vectors x, with
// W stored one output per row): the transposed product C^T = B^T A^T is a
// product with one to four columns whose N rows are B's columns, and the
// few-column kernels read each of them in whole 1 KiB runs along k, where
// the few-row kernel's operand layout reads 64 bytes of each of 16 columns
// per load instruction; no k split is summed.  The few-column kernels do not
// split k either, so the plan needs enough rows of B^T (8 per workgroup) to
// fill the CUs when k is long.  Measured on one MI355X (us, transposed /
// few-row plan, rotating B sets, best of two):
//   one row (one-column kernel, four wavefronts of two rows; the plan now
//   runs eight wavefronts of one row, 0.89-0.97 of these times: 1x2048x2048
//   4.71, 1x4096x4096 13.77, 1x14336x4096 40.14, 1x4096x8192 25.57,
//   1x2048x8192 14.76 against 16.62): 1x2048x2048 5.07 / 6.91, 1x4096x4096 14.42
//   / 16.43, 1x11008x4096 32.87 / 46.15, 1x14336x4096 41.50 / 51.08,
//   1x4096x14336 40.90 / 47.40, 1x1024x1024 3.53 / 8.29, 1x256x4096 4.50 /
//   15.78, 1x512x8192 7.36 / 13.66; long k with few columns of B lost:
//   1x2048x65536 118.9 / 109.9, 1x1024x65536 77.5 / 59.6, 1x512x32768
//   36.5 / 23.1;
//   2 to 4 rows (the staged four-column kernel, 1024-k chunks; M = 4):
//   4x6144x4096 21.75 / 27.21, 4x8192x3000 20.85 / 23.97, 4x11008x4096 36.78
//   / 48.14, 4x14336x4096 44.07 / 53.55, 4x14336x2048 23.72 / 28.50,
//   4x13824x5120 52.45 / 66.34, 4x28672x4096 80.97 / 99.97; with N up to
//   4096 or k = 8192 it lost or tied: 4x4096x4096 16.89 / 16.69,
//   4x4096x2048 9.47 / 8.39, 4x4096x8192 36.34 / 31.34, 4x8192x8192 61.45
//   / 58.33, 4x14336x8192 97.14 / 98.03; ahead again at k from 10240 (the
//   eight-wavefront four-column tile): 2x4096x11008 37.79 / 41.17,
//   4x4096x11008 38.11 / 42.42, 4x4096x14336 46.08 / 49.81 (four-wavefront
//   tile).
//   5 to 8 rows (an eight-column tile of eight wavefronts of one row): only
//   where the few-row plan's one split of 64-column tiles leaves CUs idle
//   (CUs / 2 < N / 64 < CUs): 5x11008x4096 39.79 / 48.13, 8x11008x4096
//   41.18 / 49.92, 8x14336x4096 52.90 / 54.02; with the CUs filled it lost:
//   8x4096x4096 18.53 / 17.63, 8x8192x4096 34.23 / 31.66, 5x4096x8192
//   37.77 / 31.53.
// Returns the few-column variant of the transposed plan, or -1.
// GEMM_F32_TRANSPOSE=0 turns it off; =2 (measurement) takes it for every
// shape it serves (up to eight rows, column-major B).
int transposed_few_column(int64_t m, int64_t n, int64_t k, int layout_b, int64_t cus)
{
    const int mode = env_int("GEMM_F32_TRANSPOSE", 1);
    if (mode == 0 || layout_b != GEMM_F32_COL_MAJOR || m > 8) return -1;
    const int v = m == 1 ? V_FEWCOL_R1_W8 : m <= 4 ? V_FEWCOL_R4_K1024 : V_FEWCOL_R8_W8;
    if (mode == 2) return v;
    if (m == 1) return k <= 16384 && (n >= 1024 || n * k <= (int64_t(1) << 22)) ? v : -1;
    if (m <= 4) return (n >= 6144 && k >= 2048 && k <= 5120) || (n >= 4096 && k >= 10240 && k <= 16384) ? v : -1;
    const int64_t t64 = ceil_div(n, 64);
    return 2 * t64 > cus && t64 < cus && k >= 2048 && k <= 4096 ? v : -1;
}

// Shape dispatch.  Few rows: the bandwidth-bound split-k path.  Few tiles:
// the few-row kernel on 16-row tiles (few_tile_rows).  When even
// 64 x 64 tiles leave fewer than 2.5 workgroups per CU and k >= 2048,
// 64 x 64 tiles with stream-K over all tiles (workgroups share the tiles'
// k-slabs) fill the GPU.  Measured (TFLOPS; the best data-parallel plan /
// stream-K over 64x64 tiles): 1024x1024x8192 ~64 / 118.2; 1024x1024x4096
// ~63 / 110.0; 1024x1024x2048 62.5 / 94.2; 512x512x8192 16.3 / 76.3;
// 256x256x4096 6.0 / 20.2 (these two now run faster on the few-row kernel,
// the first with row-major B only); and from two to 2.5 tiles per CU, where a
// data-parallel plan leaves the CUs unevenly loaded: 2048x1024x4096 (512
// tiles) 115.2 / 122.1, 1280x1792x4096 (560) 90.6 / 116.0, 1536x1536x4096
// (576) 99.7 / 120.9, 756x3053x6144 (576) 97.7 / 119.6, 702x3590x4096 (627)
// 99.4 / 106.8, 1536x1536x2048 97.7 / 109.6, 1536x1536x8192 100.7 / 126.4
// (918x2413x3000 (570) 88.2 / 86.5 and 1864x1288x6144 (630) 99.6 / 98.4
// lost 1-2 %).  Closer to three tiles per CU the data-parallel plans load the
// CUs evenly enough and stream-K lost: 1250x2221x6144 (700) 114.2 / 97.4,
// 2023x1453x2048 (736) 114.9 / 102.2, 2546x1202x3000 (760) 121.7 / 110.8.
// Otherwise the direct-to-LDS tile whose estimated time is least, and with
// it *tail_tiles > 0 when its partial last wave goes to stream-K.  tail_ok:
// the plan can run the stream-K kernel (row-major A, no epilogue); when it
// cannot, few-tile long-k shapes take the best data-parallel tile instead.
// epilogue: the plan fuses the linear-layer epilogue.  row_a: A is
// row-major, so the few-column kernels (which carry the epilogue) can run
// the few-column shapes; the few-row kernel serves both A layouts.
// small_scratch: the plan keeps its partial sums in the allocation-free
// entry point's 64 MiB scratch area, too small for stream-K over 128 x 128
// tiles (about 192 MiB at 768 workgroups), so that rule is skipped.
int choose_variant(int64_t m, int64_t n, int64_t k, int layout_b, const DeviceFacts &f, bool tail_ok, bool epilogue,
                   bool *stream_k, int64_t *tail_tiles, double *estimate = nullptr, int *split = nullptr,
                   bool row_a = true, bool small_scratch = false)
{
    *stream_k = false;
    *tail_tiles = 0;
    if (estimate) *estimate = 0.0;   // (not estimated for the few-row and few-tile plans)
    if (split) *split = 0;           // few-row plans: their k-split count (0: the automatic count)
    if (m <= 32) {
        // 17 to 32 rows: 32-row tiles (8 wavefronts, one workgroup per CU)
        // read B once where two 16-row tiles read it twice, with as many k
        // splits as bring the grid to one workgroup per CU.  Taken where
        // measured ahead on one MI355X (us, 32-row / 16-row, M = 32):
        // column-major B 4096x4096 25.8 / 27.3, 14336x4096 73.6 / 90.6,
        // 4096x14336 65.6 / 86.1; row-major B with B of 2^25 elements or more
        // 14336x4096 61.3 / 69.6, 4096x14336 52.5 / 60.5 (at 4096x4096 it
        // trails by 2-3 %: 21.1 / 20.7).
        if (m > 16 && n >= 1024 && (layout_b == GEMM_F32_COL_MAJOR || n * k >= (int64_t(1) << 25))) {
            if (split)
                *split = (int)std::min<int64_t>(8, std::max<int64_t>(1, ceil_div(f.cu_count, ceil_div(n, 64))));
            return V_SKINNY32_W8_D4;
        }
        // Up to 16 rows: 32-column tiles with half the k splits of 64-column
        // tiles (the same number of workgroups, each over twice the k) where
        // the 64-column plan splits k at least twice.  Each split past the
        // first adds a partial tile to write and to sum, and halving them
        // paid wherever A, which every column tile reads again, is light:
        // up to 4 rows, or k per split up to 1024, or column-major B up to 8
        // rows.  Measured on one MI355X (us, 32-column / 64-column, best of
        // two): 16x2048x2048 7.56 / 9.40 (col. B), 7.21 / 8.52 (row B);
        // 16x4096x2048 10.28 / 11.57, 8.79 / 10.05; 1x4096x4096 16.40 /
        // 18.27, 14.84 / 15.55; 8x4096x4096 col. B 17.67 / 18.95; 1x8192x4096
        // 28.49 / 31.72, 26.03 / 27.39.  Where it did not pay: 16 rows and
        // 2048 k per split (16x4096x4096 row B 17.50 / 16.50), or one split
        // (16x8192x4096 row B 31.53 / 27.98).
        const int64_t s64 = std::max<int64_t>(1, f.cu_count / ceil_div(n, 64));
        const int64_t s32 = std::max<int64_t>(1, f.cu_count / ceil_div(n, 32));
        if (m <= 16 && n >= 2048 && s64 >= 2 &&
            (m <= 4 || ceil_div(k, s32) <= 1024 || (layout_b == GEMM_F32_COL_MAJOR && m <= 8))) {
            if (split) *split = (int)s32;
            return V_SKINNY_16x32_W16_D4;
        }
        return V_SKINNY_W16_D4;
    }
    // (2 to 4 columns: the staged 1024-k chunks up to k = 4096, the 2048-k
    // chunks beyond; fewcol_gemm.hpp has the measurements.)
    if (row_a && n <= 8)
        return n == 1 ? V_FEWCOL_R1 : n <= 4 ? (k <= 4096 ? V_FEWCOL_R4_K1024 : V_FEWCOL_R4) : V_FEWCOL_R8;
    {
        // (The few-row kernel carries the epilogue and column-major A too.)
        int s = 0;
        const int v = few_tile_rows(m, n, k, layout_b, f, &s);
        if (v >= 0) {
            if (split) *split = s;
            return v;
        }
    }
    // (Epilogue plans with row-major A have the two-stage 64 x 64 tile's
    // stream-K kernel.)
    if (few_tile_stream_k(m, n, k, f, tail_ok || (epilogue && row_a))) {
        // Column-major B whose 64 x 128 tiles make one nearly full wave (7/8
        // of the CUs to all of them, one workgroup each): those tiles,
        // data-parallel.  Measured on one MI355X (us, 64x128 / stream-K over
        // 64x64): 512x4096x4096 128.0 / 144.2, 128x14336x4096 129.9 / 146.7,
        // 2048x1024x4096 127.9 / 142.5, 256x7168x4096 137.0 / 142.9,
        // 960x2048x3000 99.7 / 116.5, 1024x2048x8192 253.4 / 273.2,
        // 512x4096x2048 69.5 / 77.4; at 192 tiles stream-K stayed ahead
        // (384x4096x4096 127.6 / 109.0).  Row-major B: the three-stage
        // 64 x 128 tile where they fill 15/16 of the CUs or more and k is at
        // most 6144 (us, 64x128 s3 / stream-K): 512x4096x4096 138.2 / 142.9,
        // 1024x2048x4096 137.7 / 143.2, 128x16384x4096 138.4 / 163.2,
        // 512x4096x2048 70.8 / 78.1, 960x2048x3000 102.2 / 109.3,
        // 1000x2000x5000 167.8 / 172.1; not at 224 tiles (448x4096x4096 137.5
        // / 130.2) or k = 8192 (512x4096x8192 271.6 / 269.6).
        const int64_t t128 = ceil_div(m, 64) * ceil_div(n, 128), cus = f.cu_count;
        if (layout_b == GEMM_F32_COL_MAJOR && 8 * t128 >= 7 * cus && t128 <= cus) return V_DMA_64x128x16_S2;
        if (layout_b == GEMM_F32_ROW_MAJOR && tail_ok && 16 * t128 >= 15 * cus && t128 <= cus && k <= 6144)
            return V_DMA_64x128x16_S3;   // (no epilogue kernels)
        *stream_k = true;
        return V_DMA_64x64x16_S2;
    }
    {
        // Column-major B whose 128 x 128 tiles number more than two and at
        // most two and a half per CU, with k from 2048: stream-K over those
        // tiles with three workgroups per CU.  One data-parallel wave of
        // three per CU would leave a sixth to a third of its slots idle, and
        // the smaller tiles read B in shorter runs along its columns.
        // Measured on one MI355X (us, stream-K over 128x128 / the
        // data-parallel plan): 1536x5632x4096 545.0 / 593.7, 2048x4608x4096
        // 572.9 / 649.1, 2432x4096x4096 630.3 / 693.8, 2048x5120x5120 780.4 /
        // 867.2, 2000x5000x4000 622.1 / 678.0, 2048x5120x16384 2582.9 /
        // 2976.2, 2048x4608x2048 305.9 / 318.3; it lost at 512 tiles
        // (2048x4096x4096 498.9 / 484.3), 672 tiles (1792x6144x4096 682.0 /
        // 641.3) and k = 1024 (2048x4608x1024 171.4 / 156.8).  Row-major B
        // was level (2048x4608x4096 570.0 / 569.0).  With the linear-layer
        // epilogue (bias + GELU; us, stream-K / the data-parallel epilogue
        // plan): 2432x4096x4096 645.1 / 708.4, 2048x5120x5120 809.4 / 880.7,
        // 2000x5000x4000 642.5 / 691.3, 1536x5632x4096 565.1 / 579.8,
        // 2048x4608x4096 593.0 / 603.7; level at k = 2048 (2048x4608x2048
        // 315.3 / 312.2), so epilogue plans take it from k = 3072.
        const int64_t t128 = ceil_div(m, 128) * ceil_div(n, 128), cus = f.cu_count;
        const bool kernels = epilogue ? row_a && k >= 3072 : tail_ok;
        if (layout_b == GEMM_F32_COL_MAJOR && kernels && !small_scratch && t128 > 2 * cus && 2 * t128 <= 5 * cus &&
            k >= 2048) {
            *stream_k = true;
            return V_DMA_128x128x16_S3;
        }
    }
    int best = -1;
    double best_t = 0.0;
    const bool log = env_int("GEMM_F32_LOG", 0) >= 2;
    for (int i = 0; i < kCandidates; ++i) {
        int64_t tail = 0;
        // (tail_ok is false exactly for the plans that need linear-layer kernels)
        if (!tail_ok && !variant(kCandidate[i].variant).fn_ex[0][0][0]) continue;
        if (layout_b == GEMM_F32_COL_MAJOR && !kCandidate[i].col_b) continue;
        if (epilogue && !kCandidate[i].epi) continue;
        // The plan runs the wide-store kernel when B is row-major and N a
        // multiple of the columns a lane holds; rate it at that occupancy.
        const VariantDesc &d = variant(kCandidate[i].variant);
        const int lane_cols = d.bn / d.waves_n / 32;
        const bool wide = layout_b == GEMM_F32_ROW_MAJOR && f.per_cu_wide[i] > 0 && n % lane_cols == 0;
        const int per_cu = wide ? f.per_cu_wide[i] : f.per_cu[i];
        const double t = estimate_seconds(kCandidate[i], per_cu, f.per_cu_sk[i][layout_b], m, n, k, f.cu_count,
                                          tail_ok, &tail);
        if (log)
            std::fprintf(stderr, "[gemm_f32] candidate %s: %d per CU, estimate %.1f us%s\n", d.name, per_cu, t * 1e6,
                         tail ? " (stream-K tail)" : "");
        if (best < 0 || t < best_t) {
            best = i;
            best_t = t;
            *tail_tiles = tail;
        }
    }
    if (estimate) *estimate = best_t;
    return kCandidate[best].variant;   // 256x128, never skipped, is always weighed
}

// Column sliver.  When the chosen tile leaves a last tile-column that is at
// most an eighth full (n mod BN <= BN / 8, and at most 8 columns), every
// tile of that column runs the whole k-loop for a few columns ("GPU 算子优化中的
// 数据复用", 10.3: boundary tiles waste work): at 5003 x 4097 x 2049 the
// 4097th column costs a column of 79 tiles of 64x128, 3 % of them.  The plan
// can instead cover the first n - r columns (whose tiles may also fill the
// waves better) and run the last r columns as a second launch on the
// few-column kernel, which reads A once more: estimated at 4 m k bytes at
// 5 TB/s plus 3 us of launch.  Returns r, or 0 when one launch is estimated
// faster.  GEMM_F32_SLIVER=0 turns it off.
int64_t choose_sliver(int64_t m, int64_t n, int64_t k, int layout_b, const DeviceFacts &f, bool small_scratch = false)
{
    if (env_int("GEMM_F32_SLIVER", 1) == 0 || m <= 32 || n < 512) return 0;
    bool sk = false;
    int64_t tail = 0;
    double t_full = 0.0;
    const int v = choose_variant(m, n, k, layout_b, f, true, false, &sk, &tail, &t_full, nullptr, true, small_scratch);
    if (sk || t_full <= 0.0) return 0;
    const int bn = variant(v).bn;
    const int64_t r = n % bn;
    if (r == 0 || r * 8 > bn || r > 8) return 0;
    double t_main = 0.0;
    choose_variant(m, n - r, k, layout_b, f, true, false, &sk, &tail, &t_main, nullptr, true, small_scratch);
    if (sk || t_main <= 0.0) return 0;
    const double t_sliver = 4.0 * (double)m * (double)k / 5e12 + 3e-6;
    if (env_int("GEMM_F32_LOG", 0) >= 2)
        std::fprintf(stderr, "[gemm_f32] sliver of %lld columns: %.1f + %.1f us against %.1f us in one launch\n",
                     (long long)r, t_main * 1e6, t_sliver * 1e6, t_full * 1e6);
    return t_main + t_sliver < t_full ? r : 0;
}

// Tiles of a stream-K plan that more than one workgroup shares, the ones a
// last arriver finishes: the kernel cuts the shared tiles' shared * k_tiles
// slabs into wgs ranges, range q = [q * iters / wgs, (q + 1) * iters / wgs),
// and a tile is shared when its first and last slabs fall in different ranges.
int64_t stream_k_split_tiles(int64_t shared, int64_t k_tiles, int64_t wgs)
{
    const int64_t iters = shared * k_tiles;
    auto owner = [&](int64_t x) { return ((x + 1) * wgs - 1) / iters; };
    int64_t n = 0;
    for (int64_t t = 0; t < shared; ++t)
        if (owner(t * k_tiles) != owner(t * k_tiles + k_tiles - 1)) ++n;
    return n;
}

// Everything a plan needs except its workspace: the kernel, grid and launch
// arguments, and the workspace it asks for (*ws_words bytes of epoch-tagged
// partial-sum words and *ws_counters 32-bit arrival counters, plus one status
// word; zero for plans that split no tile along k).  No allocation.
int plan_fill(gemm_f32_plan_impl *p, int forced_variant, int64_t m, int64_t n, int64_t k, int layout_a,
              int layout_b, int64_t lda, int64_t ldb, int64_t ldc, int epilogue, size_t *ws_words,
              size_t *ws_counters, bool small_scratch = false)
{
    *ws_words = 0;
    *ws_counters = 0;
    int st = gemm_f32_validate_ex(m, n, k, layout_a, layout_b, lda, ldb, ldc);
    if (st != GEMM_F32_SUCCESS) return st;
    if (forced_variant >= V_COUNT || (epilogue != 0 && epilogue != 1)) return GEMM_F32_ERR_INVALID_VALUE;
    // Column-major A and the epilogue have kernels in the dispatch
    // candidates (and the three-stage 64x64) only.
    const bool ex = layout_a == GEMM_F32_COL_MAJOR || epilogue;

    int dev = 0;
    DeviceFacts facts;
    st = device_facts(&dev, &facts);
    if (st != GEMM_F32_SUCCESS) return st;

    int v = forced_variant;
    bool auto_stream_k = false;
    int64_t auto_tail = 0;
    int auto_split = 0;
    bool swap_ab = false;
    if (v < 0) {
        v = env_int("GEMM_F32_VARIANT", -1);
        if (v < 0 || v >= V_COUNT) {
            // (The transposed plan serves row-major A, with or without the
            // epilogue.)
            const int tv =
                layout_a == GEMM_F32_COL_MAJOR ? -1 : transposed_few_column(m, n, k, layout_b, facts.cu_count);
            swap_ab = tv >= 0;
            v = swap_ab ? tv
                        : choose_variant(m, n, k, layout_b, facts, !ex, epilogue != 0, &auto_stream_k, &auto_tail,
                                         nullptr, &auto_split, layout_a == GEMM_F32_ROW_MAJOR, small_scratch);
        }
        if (ex && !swap_ab && !variant(v).fn_ex[layout_a][layout_b][epilogue]) v = V_DMA_64x64x16_S2;
    }
    const VariantDesc &d = variant(v);
    if (ex && !swap_ab && !d.fn_ex[layout_a][layout_b][epilogue]) return GEMM_F32_ERR_INVALID_VALUE;
    // Stream-K for the linear-layer epilogue with row-major A where the
    // variant has its kernels; none for column-major A.
    const void *const *fn_sk = epilogue ? d.fn_sk_epi : d.fn_sk;
    if (layout_a == GEMM_F32_COL_MAJOR || !fn_sk[0]) {
        auto_stream_k = false;
        auto_tail = 0;
    }

    p->variant = v;
    p->device = dev;
    p->layout_a = layout_a;
    p->layout_b = layout_b;
    p->epilogue = epilogue;
    p->fn = swap_ab ? nullptr : ex ? d.fn_ex[layout_a][layout_b][epilogue] : d.fn[layout_b];
    // C's extent before the transposed plan exchanges the operands' roles.
    const uint32_t c_bytes = (uint32_t)(((m - 1) * ldc + n) * 4);
    p->swap_ab = swap_ab;
    if (swap_ab) {
        // C^T = B^T A^T: B^T is the caller's column-major B read as a
        // row-major n x k matrix (leading dimension ldb), A^T the caller's
        // row-major A read as a column-major k x m matrix (leading dimension
        // lda); the kernel stores its result (i, j) at C[j * ldc + i].
        p->fn = epilogue ? d.fn_t_epi : d.fn_t;
        std::swap(m, n);
        std::swap(lda, ldb);
    }
    // Row-major B: 8- or 16-byte C stores (and C loads of the epilogue)
    // when N is a multiple of the columns a lane holds per row
    // (bn / waves_n / 32).
    const int lane_cols = d.kind == GEMM_F32_KIND_MFMA ? d.bn / d.waves_n / 32 : 0;
    p->c_store_width = 1;
    if (layout_b == GEMM_F32_ROW_MAJOR && d.fn_wide[layout_a][epilogue] && lane_cols > 0 && n % lane_cols == 0 &&
        env_int("GEMM_F32_WIDE_C", 1) != 0) {
        p->fn = d.fn_wide[layout_a][epilogue];
        p->c_store_width = lane_cols;
    }
    p->m = m; p->n = n; p->k = k;
    p->lda = lda; p->ldb = ldb; p->ldc = ldc;
    p->strides4 = lda % 4 == 0 && ldb % 4 == 0 && ldc % 4 == 0;

    GemmArgs &a = p->args;
    std::memset(&a, 0, sizeof(a));
    a.m = (int)m; a.n = (int)n; a.k = (int)k;
    a.lda = (int)lda; a.ldb = (int)ldb; a.ldc = (int)ldc;
    a.tiles_m = (int)ceil_div(m, d.bm);
    a.tiles_n = (int)ceil_div(n, d.bn);
    a.k_tiles = (int)ceil_div(k, d.bk);
    // Tile-rows per rasterisation group.  256x256 (one tile per CU) ran
    // best with 4: 4096^3 148.7 against 148.0-148.3 with 8, FFN 148.8-148.9
    // against 148.7-148.8 (same box, two repeats; 1, 2 and 16 no better).
    a.group_m = env_int("GEMM_F32_GROUP_M", d.bm == 256 && d.bn == 256 ? 4 : 8);
    if (a.group_m < 1) a.group_m = 1;
    a.num_xcd = env_int("GEMM_F32_NUM_XCD", facts.num_xcd);   // 1: no XCD remap (measurement)
    if (a.num_xcd < 1) a.num_xcd = 1;
    a.a_bytes = (uint32_t)((layout_a == GEMM_F32_ROW_MAJOR ? (m - 1) * lda + k : (k - 1) * lda + m) * 4);
    a.alpha = 1.0f;
    a.beta = 0.0f;
    a.b_bytes = (uint32_t)((layout_b == GEMM_F32_ROW_MAJOR ? (k - 1) * ldb + n : (n - 1) * ldb + k) * 4);
    a.c_bytes = c_bytes;
    a.split_k = 1;
    a.k_per_split = (int)k;
    // The whole-chunk loads of row-major B may run up to 3 elements past the
    // last valid column of a k-row; that stays inside B when ldb >= 4.
    a.masked_loads = (layout_b == GEMM_F32_ROW_MAJOR && ldb < 4) ? 1 : 0;
    // Waits for partial sums, and two test hooks (environment, read here):
    // GEMM_F32_WAIT_BUDGET polls per thread before a wait gives up;
    // GEMM_F32_TEST_LOST_WORDS=1 makes readers wait for a tag that is never
    // written (every wait gives up, the status word records it);
    // GEMM_F32_POISON_LDS=1 fills LDS with NaN before the first copy.
    a.wait_budget = env_int("GEMM_F32_WAIT_BUDGET", gemmf32::kTaggedWaitBudget);
    if (a.wait_budget < 0) a.wait_budget = 0;
    a.epoch_xor = env_int("GEMM_F32_TEST_LOST_WORDS", 0) ? 0xc0000000u : 0u;
    a.poison_lds = env_int("GEMM_F32_POISON_LDS", 0) ? 1 : 0;
    p->grid = (unsigned)((int64_t)a.tiles_m * a.tiles_n);
    p->block = (unsigned)d.threads;
    p->workspace = nullptr;
    if (d.kind == GEMM_F32_KIND_SKINNY) {
        // Split k across workgroups up to 16 wavefronts per CU (rounded
        // down: a few workgroups past one per CU make a second wave, e.g.
        // 200x200x3000 on 16x64 tiles: 260 workgroups 15.8 us, 208 9.9 us),
        // or as the few-tile rule chose; each split is a whole number of 16-k
        // groups.
        const int64_t per_split = (int64_t)a.tiles_m * a.tiles_n;
        int64_t split = auto_split > 0 ? auto_split
                                       : std::max<int64_t>(1, 16 * (int64_t)facts.cu_count / (per_split * (d.threads / 64)));
        split = env_int("GEMM_F32_SPLIT_K", (int)split);   // tuning override
        split = split < 1 ? 1 : split;
        const int64_t max_split = ceil_div(k, 64);
        split = split > max_split ? max_split : split;
        int64_t kps = ceil_div(ceil_div(k, split), 16) * 16;
        split = ceil_div(k, kps);
        a.split_k = (int)split;
        a.k_per_split = (int)kps;
        p->grid = (unsigned)(per_split * split);
        if (split > 1) {
            // split * m * n tagged words and one arrival counter per tile;
            // every tile is shared by its splits.
            *ws_words = (size_t)split * (size_t)m * (size_t)n * sizeof(unsigned long long);
            *ws_counters = (size_t)per_split;
            a.split_tiles = (int)per_split;
        }
    }

    if (fn_sk[0]) {
        // Stream-K, chosen by the shape dispatch: either up to three
        // workgroups per CU share the k-slabs of all tiles evenly, or one
        // workgroup per CU shares those of the partial last wave's tiles
        // (the rest run whole).  GEMM_F32_SK_WGS forces it with that many
        // workgroups, over the first GEMM_F32_SK_TILES tiles (default all;
        // the other tiles get a workgroup each); GEMM_F32_STREAMK=0 disables
        // the automatic choice.
        const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n;
        int64_t wgs = layout_a == GEMM_F32_COL_MAJOR ? 0 : env_int("GEMM_F32_SK_WGS", 0);
        int64_t shared = wgs > 0 ? env_int("GEMM_F32_SK_TILES", (int)tiles) : tiles;
        if (wgs <= 0 && auto_tail > 0 && env_int("GEMM_F32_STREAMK", 1) != 0) {
            // The partial last wave's tiles (the first ones in raster order)
            // split over one workgroup per CU, at most 8 per tile (the last
            // segment reads all the others); the other tiles whole.
            wgs = std::min<int64_t>(facts.cu_count, 8 * auto_tail);
            shared = auto_tail;
        } else if (wgs <= 0 && auto_stream_k && env_int("GEMM_F32_STREAMK", 1) != 0) {
            int per_cu = 0;
            hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn_sk[layout_b], d.threads, 0);
            if (e != hipSuccess) return hip_fail(e);
            // Three workgroups per CU (fewer if fewer fit), at most 8
            // segments per tile (the last one to arrive reads all the
            // others) and at least 8 slabs per workgroup.  Measured with
            // 64x64 tiles, TFLOPS at P = 512 / 768 / 1024 / 1280:
            // 1024x1024x8192 104.1 / 118.2 / 117.1 / 109.6, 1024x1024x2048
            // 88.8 / 94.2 / 88.6 / 83.1, 768x768x8192 91.5 / 101.5 / 100.5 /
            // 89.3; 512x512x8192 at P = 256 / 384 / 512 (8 per tile) 52.7 /
            // 68.3 / 76.3; 256x256x4096 at 64 / 128 (8 per tile) / 256 17.8
            // / 20.2 / 15.7.
            wgs = std::min<int64_t>(std::min<int64_t>((int64_t)std::min(3, per_cu) * facts.cu_count, 8 * tiles),
                                    tiles * a.k_tiles / 8);
            if (wgs < 2) wgs = 0;
        }
        if (shared < 1 || shared > tiles) shared = tiles;
        const int64_t iters = shared * a.k_tiles;
        if (wgs > iters) wgs = iters;
        if (wgs > 0) {
            a.sk_wgs = (int)wgs;
            a.sk_tiles = (int)shared;
            p->fn = fn_sk[layout_b];
            p->c_store_width = 1;   // the stream-K kernel stores one element at a time
            p->grid = (unsigned)(wgs + tiles - shared);
            const size_t words = (size_t)2 * wgs * d.bm * d.bn * sizeof(unsigned long long);
            // The words are addressed through a buffer descriptor (32-bit
            // extent); the automatic plans stay far below this.
            if (words >= ((size_t)1 << 31)) return GEMM_F32_ERR_INVALID_VALUE;
            a.partial_bytes = (uint32_t)words;
            *ws_words = words;
            *ws_counters = (size_t)shared;
            a.split_tiles = (int)stream_k_split_tiles(shared, a.k_tiles, wgs);
        }
    }

    if (env_int("GEMM_F32_LOG", 0))
        std::fprintf(stderr, "[gemm_f32] m=%lld n=%lld k=%lld layoutB=%d -> %s grid=%u group_m=%d split_k=%d stream_k=%d over %d tiles\n",
                     (long long)m, (long long)n, (long long)k, layout_b, d.name, p->grid, a.group_m, a.split_k,
                     a.sk_wgs, a.sk_tiles);
    return GEMM_F32_SUCCESS;
}

// Counters of a plan's workspace beyond the per-tile arrival counters: the
// status word, the count of finished split tiles and the epoch word.
constexpr size_t kExtraCounters = 3;

// Point a plan's launch arguments at its workspace: the words, then the
// arrival counters, the status word, the finished-tile count and the epoch
// word.
void plan_attach(gemm_f32_plan_impl *p, void *words, unsigned *counters, size_t n_counters)
{
    p->args.partial = static_cast<unsigned long long *>(words);
    p->args.arrivals = counters;
    p->args.status = counters + n_counters;
    p->args.done_tiles = counters + n_counters + 1;
    p->args.epoch_word = counters + n_counters + 2;
}

// Columns of a column sliver for a plan (0: none): plain products with the
// shape dispatch's own choices only (no forced variant, stream-K or split).
int64_t plan_sliver(int forced_variant, int64_t m, int64_t n, int64_t k, int layout_a, int layout_b, int64_t lda,
                    int64_t ldb, int64_t ldc, int epilogue, bool small_scratch = false)
{
    if (forced_variant >= 0 || layout_a != GEMM_F32_ROW_MAJOR || epilogue) return 0;
    if (env_int("GEMM_F32_VARIANT", -1) >= 0 || env_int("GEMM_F32_SK_WGS", 0) > 0 ||
        env_int("GEMM_F32_SPLIT_K", 0) > 0)
        return 0;
    if (gemm_f32_validate_ex(m, n, k, layout_a, layout_b, lda, ldb, ldc) != GEMM_F32_SUCCESS) return 0;
    int dev = 0;
    DeviceFacts facts;
    if (device_facts(&dev, &facts) != GEMM_F32_SUCCESS) return 0;
    return choose_sliver(m, n, k, layout_b, facts, small_scratch);
}

// B and C of a plan's sliver: column sliver_col0 of B (row-major: the next
// element of each k-row; column-major: the next column) and of C.
const float *sliver_b(const gemm_f32_plan_impl *p, const float *B)
{
    return p->layout_b == GEMM_F32_ROW_MAJOR ? B + p->sliver_col0 : B + p->sliver_col0 * p->ldb;
}

// Fused column sliver.  A whole-tile plan whose last wave of tiles leaves
// workgroup slots idle can carry its sliver in the same launch
// (gemm_mfma_dma_sliver_kernel): the few-column workgroups come after every
// tile in the grid, so they are dispatched into those idle slots instead of
// running as a second launch after the last tile.  Taken when the kernel
// exists for the plan's tile and B layout, holds as many workgroups per CU
// as the plan's own kernel, and the idle slot time of the last wave (idle
// slots x one tile's time at that occupancy) is at least twice the sliver's
// estimated work (per workgroup: 3 us plus its rows of A at 40 GB/s).
// Slivers of one or two columns only: the fused workgroups take one column
// each and read A once per column, where the second launch reads it once for
// up to 8 columns.  At 5003 x (4096 + r) x 2049 (1280 tiles of 128 x 128 in
// 768 slots; the sliver's workgroups run in the 256 slots the second wave
// leaves idle), fused against two launches, in alternation on one GPU:
// r = 1 594.3-594.5 against 606.7-608.4 us, r = 2 604.1-604.9 against
// 611.1, r = 4 630.1-630.8 against 604.9-609.8, r = 8 683.9 against
// 613.3-613.9.  GEMM_F32_SLIVER_FUSE=0 keeps the second launch.
void fuse_sliver(gemm_f32_plan p, const DeviceFacts &f)
{
    if (!p->sliver || p->sliver->n > 2 || p->workspace || p->args.sk_wgs || p->args.split_k != 1 ||
        p->epilogue || p->layout_a != GEMM_F32_ROW_MAJOR || env_int("GEMM_F32_SLIVER_FUSE", 1) == 0)
        return;
    const VariantDesc &d = variant(p->variant);
    const int col = p->layout_b == GEMM_F32_COL_MAJOR ? 1 : 0;
    const void *fn = p->c_store_width > 1 ? d.fn_sliver_wide : d.fn_sliver[col];
    if (!fn) return;
    int plain = 0, fused = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&plain, p->fn, (int)p->block, 0) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&fused, fn, (int)p->block, 0) != hipSuccess) {
        (void)hipGetLastError();
        return;
    }
    if (fused < 1 || fused != plain) return;
    const int64_t slots = (int64_t)plain * f.cu_count;
    const int64_t last = (int64_t)p->grid % slots;
    if (last == 0) return;
    const int rows = (int)p->block / 64;   // rows per few-column workgroup (one per wavefront)
    const int64_t wgs = ceil_div(p->m, rows) * p->sliver->n;
    const double t_tile = 2.0 * d.bm * d.bn * (double)p->k * plain / (157.3e12 / f.cu_count);
    const double t_wg = 3e-6 + 4.0 * rows * (double)p->k / 40e9;
    if ((double)(slots - last) * t_tile < 2.0 * (double)wgs * t_wg) return;
    if ((int64_t)p->grid + wgs > INT32_MAX) return;
    p->fn = fn;
    p->args.sliver_wg0 = (int)p->grid;
    p->args.sliver_cols = (int)p->sliver->n;
    p->args.sliver_b_bytes = p->sliver->args.b_bytes;
    p->grid += (unsigned)wgs;
    p->sliver_fused = true;
    if (env_int("GEMM_F32_LOG", 0))
        std::fprintf(stderr, "[gemm_f32] column sliver of %lld columns in the same launch: %lld workgroups after %d tiles\n",
                     (long long)p->sliver->n, (long long)wgs, p->args.sliver_wg0);
}

int make_plan(gemm_f32_plan *out, int forced_variant, int64_t m, int64_t n, int64_t k, int layout_a,
              int layout_b, int64_t lda, int64_t ldb, int64_t ldc, int epilogue, bool allow_sliver = true)
{
    if (!out) return GEMM_F32_ERR_INVALID_VALUE;
    *out = nullptr;
    gemm_f32_plan p = new (std::nothrow) gemm_f32_plan_impl();
    if (!p) return GEMM_F32_ERR_ALLOC;
    const int64_t r =
        allow_sliver ? plan_sliver(forced_variant, m, n, k, layout_a, layout_b, lda, ldb, ldc, epilogue) : 0;
    size_t words = 0, counters = 0;
    int st = plan_fill(p, forced_variant, m, n - r, k, layout_a, layout_b, lda, ldb, ldc, epilogue, &words,
                       &counters);
    if (st != GEMM_F32_SUCCESS) {
        delete p;
        return st;
    }
    if (words) {
        // The plan's own workspace, all zero: every counter starts at zero,
        // the epoch word too, so the first run tags its words 1 and no word
        // carries a valid tag before it is written.
        const size_t bytes = words + (counters + kExtraCounters) * sizeof(unsigned);
        hipError_t e = hipMalloc(&p->workspace, bytes);
        if (e == hipSuccess) e = hipMemsetAsync(p->workspace, 0, bytes, nullptr);
        if (e == hipSuccess) e = hipStreamSynchronize(nullptr);
        if (e != hipSuccess) {
            if (p->workspace) (void)hipFree(p->workspace);
            delete p;
            return hip_fail(e);
        }
        plan_attach(p, p->workspace, reinterpret_cast<unsigned *>(static_cast<char *>(p->workspace) + words),
                    counters);
    }
    if (r) {
        st = make_plan(&p->sliver, -1, m, r, k, layout_a, layout_b, lda, ldb, ldc, epilogue, false);
        if (st != GEMM_F32_SUCCESS) {
            if (p->workspace) (void)hipFree(p->workspace);
            delete p;
            return st;
        }
        p->sliver_col0 = n - r;
        int dev = 0;
        DeviceFacts facts;
        if (device_facts(&dev, &facts) == GEMM_F32_SUCCESS) fuse_sliver(p, facts);
    }
    *out = p;
    return GEMM_F32_SUCCESS;
}

// The build's resource entry of a kernel, found by the mangled name of its
// handle (the handles are exported symbols of this library), or NULL.
const gemmf32::KernelResources *kernel_resources(const void *fn)
{
    Dl_info d;
    if (!fn || !dladdr(fn, &d) || !d.dli_sname) return nullptr;
    for (int i = 0; i < gemmf32::kKernelResourcesCount; ++i)
        if (std::strcmp(gemmf32::kKernelResources[i].name, d.dli_sname) == 0) return &gemmf32::kKernelResources[i];
    return nullptr;
}

void fill_resources(const void *fn, gemm_f32_info *info)
{
    const gemmf32::KernelResources *r = kernel_resources(fn);
    if (!r) return;
    info->vgprs = r->vgprs;
    info->agprs = r->agprs;
    info->sgprs = r->sgprs;
    info->scratch_bytes = r->scratch_bytes;
    info->compiler_waves_per_simd = r->waves_per_simd;
}

// Every kernel handle of a variant.
template <class F>
void for_each_kernel(const VariantDesc &d, F f)
{
    for (const void *fn : d.fn) f(fn);
    for (const void *fn : d.fn_sk) f(fn);
    for (const void *fn : d.fn_sk_epi) f(fn);
    for (int a = 0; a < 2; ++a)
        for (int b = 0; b < 2; ++b)
            for (int e = 0; e < 2; ++e) f(d.fn_ex[a][b][e]);
    for (int a = 0; a < 2; ++a)
        for (int e = 0; e < 2; ++e) f(d.fn_wide[a][e]);
    f(d.fn_t);
    f(d.fn_t_epi);
}

void fill_static_info(int v, gemm_f32_info *info)
{
    std::memset(info, 0, sizeof(*info));
    const VariantDesc &d = variant(v);
    info->variant = v;
    info->kind = d.kind;
    info->bm = d.bm; info->bn = d.bn; info->bk = d.bk;
    info->waves_m = d.waves_m; info->waves_n = d.waves_n;
    info->wave_m = d.bm / d.waves_m;
    info->wave_n = d.bn / d.waves_n;
    info->threads = d.threads;
    info->lds_bytes = d.lds_bytes;
    info->stages = d.stages;
    info->split_k = 1;
    std::snprintf(info->name, sizeof(info->name), "%s", d.name);
    fill_resources(d.fn[0], info);
    // Spills anywhere in the variant: the largest scratch of its kernels.
    for_each_kernel(d, [&](const void *fn) {
        const gemmf32::KernelResources *r = fn ? kernel_resources(fn) : nullptr;
        if (r && r->scratch_bytes > info->scratch_bytes) info->scratch_bytes = r->scratch_bytes;
    });
}

}  // namespace

extern "C" {

int gemm_f32_validate_ex(int64_t m, int64_t n, int64_t k, int layout_a, int layout_b, int64_t lda, int64_t ldb,
                         int64_t ldc)
{
    if (m < 1 || n < 1 || k < 1) return GEMM_F32_ERR_INVALID_VALUE;
    if (layout_a != GEMM_F32_ROW_MAJOR && layout_a != GEMM_F32_COL_MAJOR) return GEMM_F32_ERR_INVALID_VALUE;
    if (layout_b != GEMM_F32_ROW_MAJOR && layout_b != GEMM_F32_COL_MAJOR) return GEMM_F32_ERR_INVALID_VALUE;
    if (ldc < n) return GEMM_F32_ERR_INVALID_VALUE;
    if (layout_a == GEMM_F32_ROW_MAJOR ? lda < k : lda < m) return GEMM_F32_ERR_INVALID_VALUE;
    if (layout_b == GEMM_F32_ROW_MAJOR ? ldb < n : ldb < k) return GEMM_F32_ERR_INVALID_VALUE;
    // Byte extents below 2^31: 32-bit buffer offsets address every element
    // and the out-of-range offset 2^31 is never a valid element.
    const int64_t limit = (int64_t)1 << 31;
    const int64_t cap = limit / 4;  // elements; also bounds each factor against overflow
    if (m >= cap || n >= cap || k >= cap || lda >= cap || ldb >= cap || ldc >= cap)
        return GEMM_F32_ERR_INVALID_VALUE;
    const int64_t a_ext = layout_a == GEMM_F32_ROW_MAJOR ? (m - 1) * lda + k : (k - 1) * lda + m;
    const int64_t b_ext = layout_b == GEMM_F32_ROW_MAJOR ? (k - 1) * ldb + n : (n - 1) * ldb + k;
    const int64_t c_ext = (m - 1) * ldc + n;
    if (a_ext >= cap || b_ext >= cap || c_ext >= cap) return GEMM_F32_ERR_INVALID_VALUE;
    return GEMM_F32_SUCCESS;
}

int gemm_f32_validate(int64_t m, int64_t n, int64_t k, int layout_b, int64_t lda, int64_t ldb, int64_t ldc)
{
    return gemm_f32_validate_ex(m, n, k, GEMM_F32_ROW_MAJOR, layout_b, lda, ldb, ldc);
}

int gemm_f32_create(gemm_f32_plan *out, int64_t m, int64_t n, int64_t k, int layout_b, int64_t lda,
                    int64_t ldb, int64_t ldc)
{
    return make_plan(out, -1, m, n, k, GEMM_F32_ROW_MAJOR, layout_b, lda, ldb, ldc, 0);
}

int gemm_f32_create_ex(gemm_f32_plan *out, int64_t m, int64_t n, int64_t k, int layout_a, int layout_b,
                       int64_t lda, int64_t ldb, int64_t ldc, int epilogue)
{
    return make_plan(out, -1, m, n, k, layout_a, layout_b, lda, ldb, ldc, epilogue);
}

int gemm_f32_create_variant(gemm_f32_plan *out, int v, int64_t m, int64_t n, int64_t k, int layout_b,
                            int64_t lda, int64_t ldb, int64_t ldc)
{
    if (v < 0 || v >= V_COUNT) {
        if (out) *out = nullptr;
        return GEMM_F32_ERR_INVALID_VALUE;
    }
    return make_plan(out, v, m, n, k, GEMM_F32_ROW_MAJOR, layout_b, lda, ldb, ldc, 0);
}

}  // extern "C"

namespace {

// Launch the plan's kernel with arguments `a` (pointers filled).
int launch_kernel(const gemm_f32_plan_impl *p, GemmArgs &a, void *stream)
{
    void *kargs[] = {&a};
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = hipLaunchKernel(p->fn, dim3(p->grid), dim3(p->block), kargs, 0, s);
    if (e != hipSuccess) return hip_fail(e);
    return GEMM_F32_SUCCESS;
}

// Whether `stream` is capturing into a graph (or the query fails: then the
// launch takes the tag kind that is right either way).
bool capturing(void *stream)
{
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(reinterpret_cast<hipStream_t>(stream), &st) != hipSuccess) {
        (void)hipGetLastError();
        return true;
    }
    return st != hipStreamCaptureStatusNone;
}

// The tag of a split plan's run: a fresh argument tag (bit 31 clear, never
// 0) from `counter`, or, for a launch captured in a graph, the workspace
// word (a.epoch_word stays set; see load_run_epoch).
void tag_run(GemmArgs &a, std::atomic<unsigned> &counter, void *stream)
{
    if (capturing(stream)) return;
    a.epoch_word = nullptr;
    unsigned ep = ++counter & 0x7fffffffu;
    if (ep == 0) ep = ++counter & 0x7fffffffu;
    a.epoch = ep;
}

int launch(gemm_f32_plan p, GemmArgs &a, void *stream)
{
    if (p->workspace) tag_run(a, p->runs, stream);
    return launch_kernel(p, a, stream);
}

// The device address of `scratch` on the current device, found once per
// device with that device current.
struct ScratchSlot {
    void *ptr = nullptr;
    std::atomic<unsigned> runs{0};   // argument tags handed out to calls on this device
};
ScratchSlot g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

int scratch_address(int dev, void **out)
{
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    ScratchSlot &s = g_scratch[dev];
    if (!s.ptr) {
        void *ptr = nullptr;
        hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol);
        s.ptr = ptr;
    }
    *out = s.ptr;
    return GEMM_F32_SUCCESS;
}

bool pointers_ok(const float *A, const float *B, const float *C)
{
    if (!A || !B || !C) return false;
    const uintptr_t ua = reinterpret_cast<uintptr_t>(A), ub = reinterpret_cast<uintptr_t>(B),
                    uc = reinterpret_cast<uintptr_t>(C);
    return ((ua | ub | uc) & 3u) == 0;
}

}  // namespace

extern "C" {

int gemm_f32_run(gemm_f32_plan p, const float *A, const float *B, float *C, void *stream)
{
    if (!p || !pointers_ok(A, B, C)) return GEMM_F32_ERR_INVALID_VALUE;
    GemmArgs a = p->args;
    a.A = p->swap_ab ? B : A;
    a.B = p->swap_ab ? A : B;
    a.C = C;
    if (p->sliver_fused) {
        a.sliver_B = sliver_b(p, B);
        a.sliver_C = C + p->sliver_col0;
    }
    const int st = launch(p, a, stream);
    if (st != GEMM_F32_SUCCESS || !p->sliver || p->sliver_fused) return st;
    return gemm_f32_run(p->sliver, A, sliver_b(p, B), C + p->sliver_col0, stream);
}

int gemm_f32_run_noalloc(int64_t m, int64_t n, int64_t k, int layout_b, int64_t lda, int64_t ldb, int64_t ldc,
                         const float *A, const float *B, float *C, void *stream)
{
    if (!pointers_ok(A, B, C)) return GEMM_F32_ERR_INVALID_VALUE;
    // Host state on the stack, nothing allocated: the plan and, when the
    // dispatch splits off a column sliver, the sliver's plan; both without
    // the stream-K plans whose partial sums outgrow the scratch area.
    const int64_t r = plan_sliver(-1, m, n, k, GEMM_F32_ROW_MAJOR, layout_b, lda, ldb, ldc, 0, true);
    gemm_f32_plan_impl parts[2];
    size_t words[2] = {0, 0}, counters[2] = {0, 0};
    int st = plan_fill(&parts[0], -1, m, n - r, k, GEMM_F32_ROW_MAJOR, layout_b, lda, ldb, ldc, 0, &words[0],
                       &counters[0], true);
    if (st == GEMM_F32_SUCCESS && r)
        st = plan_fill(&parts[1], -1, m, r, k, GEMM_F32_ROW_MAJOR, layout_b, lda, ldb, ldc, 0, &words[1],
                       &counters[1], true);
    if (st != GEMM_F32_SUCCESS) return st;
    for (int i = 0; i < (r ? 2 : 1); ++i)
        if (words[i] > kScratchWordBytes || counters[i] + kExtraCounters > kScratchCounters)
            return GEMM_F32_ERR_SCRATCH_TOO_SMALL;
    parts[0].sliver_col0 = n - r;
    for (int i = 0; i < (r ? 2 : 1); ++i) {
        // The two launches run one after the other on `stream`, so they can
        // share the scratch area.
        gemm_f32_plan_impl &p = parts[i];
        GemmArgs a = p.args;
        a.A = p.swap_ab ? B : A;
        a.B = p.swap_ab ? A : i ? sliver_b(&parts[0], B) : B;
        a.C = i ? C + parts[0].sliver_col0 : C;
        if (words[i]) {
            void *base = nullptr;
            st = scratch_address(p.device, &base);
            if (st != GEMM_F32_SUCCESS) return st;
            unsigned *ctr = static_cast<unsigned *>(base);
            a.partial = reinterpret_cast<unsigned long long *>(static_cast<char *>(base) + kScratchCounters * 4);
            a.arrivals = ctr;
            a.status = ctr + counters[i];
            a.done_tiles = ctr + counters[i] + 1;
            a.epoch_word = ctr + (kScratchCounters - 1);
            // The arrival counters, the status word and the finished-tile
            // count start at zero: a fill kernel on the caller's stream ahead
            // of the product (a kernel, not a memset, so that the call can be
            // captured in a graph).  The words need no clearing: each launch
            // on this device tags its words afresh, with an argument tag or,
            // captured in a graph, from the epoch word, which is never
            // cleared.
            const int n_zero = (int)(counters[i] + 2);
            unsigned *zp = ctr;
            int zn = n_zero;
            void *zargs[] = {&zp, &zn};
            hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&gemmf32::zero_words_kernel),
                                           dim3((unsigned)((n_zero + 255) / 256)), dim3(256), zargs, 0,
                                           reinterpret_cast<hipStream_t>(stream));
            if (e != hipSuccess) return hip_fail(e);
            tag_run(a, g_scratch[p.device].runs, stream);
        }
        st = launch_kernel(&p, a, stream);
        if (st != GEMM_F32_SUCCESS) return st;
    }
    return GEMM_F32_SUCCESS;
}

int gemm_f32_run_ex(gemm_f32_plan p, const float *A, const float *B, float *C, float alpha, float beta,
                    const float *bias, int activation, void *stream)
{
    if (!p || !pointers_ok(A, B, C)) return GEMM_F32_ERR_INVALID_VALUE;
    if (activation < GEMM_F32_ACT_NONE || activation > GEMM_F32_ACT_GELU) return GEMM_F32_ERR_INVALID_VALUE;
    if (bias && (reinterpret_cast<uintptr_t>(bias) & 3u)) return GEMM_F32_ERR_INVALID_VALUE;
    const bool plain = alpha == 1.0f && beta == 0.0f && !bias && activation == GEMM_F32_ACT_NONE;
    if (!plain && !p->epilogue) return GEMM_F32_ERR_INVALID_VALUE;
    GemmArgs a = p->args;
    a.A = p->swap_ab ? B : A;
    a.B = p->swap_ab ? A : B;
    a.C = C;
    a.alpha = alpha;
    a.beta = beta;
    a.use_beta = beta != 0.0f ? 1 : 0;
    a.bias = bias;
    a.act = activation;
    if (p->sliver_fused) {
        a.sliver_B = sliver_b(p, B);
        a.sliver_C = C + p->sliver_col0;
    }
    const int st = launch(p, a, stream);
    // (Only plain plans have a sliver, so these are the plain values.)
    if (st != GEMM_F32_SUCCESS || !p->sliver || p->sliver_fused) return st;
    return gemm_f32_run(p->sliver, A, sliver_b(p, B), C + p->sliver_col0, stream);
}

int gemm_f32_destroy(gemm_f32_plan p)
{
    if (!p) return GEMM_F32_SUCCESS;
    int st = GEMM_F32_SUCCESS;
    if (p->workspace) {
        hipError_t e = hipFree(p->workspace);
        if (e != hipSuccess) st = hip_fail(e);
    }
    if (p->sliver) {
        const int s2 = gemm_f32_destroy(p->sliver);
        if (st == GEMM_F32_SUCCESS) st = s2;
    }
    delete p;
    return st;
}

int gemm_f32_describe(gemm_f32_plan p, gemm_f32_info *info)
{
    if (!p || !info) return GEMM_F32_ERR_INVALID_VALUE;
    fill_static_info(p->variant, info);
    info->aligned = p->strides4 ? 1 : 0;
    info->tiles_m = p->args.tiles_m;
    info->tiles_n = p->args.tiles_n;
    info->k_tiles = p->args.k_tiles;
    info->grid = p->grid;
    info->group_m = p->args.group_m;
    info->c_store_width = p->c_store_width;
    info->split_k = p->args.split_k;
    info->stream_k = p->args.sk_wgs;
    info->stream_k_tiles = p->args.sk_tiles;
    info->layout_a = p->layout_a;
    info->epilogue = p->epilogue;
    // The kernel this plan launches, its resources and its occupancy.
    const void *fn = p->fn;
    info->vgprs = info->agprs = info->sgprs = info->scratch_bytes = info->compiler_waves_per_simd = 0;
    fill_resources(fn, info);
    int wgs = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&wgs, fn, (int)p->block, 0) != hipSuccess) {
        (void)hipGetLastError();
        wgs = 0;
    }
    info->workgroups_per_cu = wgs;
    info->waves_per_simd = wgs * ((int)p->block / 64) / 4;
    if (p->sliver) {
        info->sliver_cols = p->sliver->n;
        info->sliver_variant = p->sliver->variant;
        info->sliver_stream_k = p->sliver->args.sk_wgs;
        info->sliver_fused = p->sliver_fused ? 1 : 0;
    }
    info->transposed = p->swap_ab ? 1 : 0;
    return GEMM_F32_SUCCESS;
}

int gemm_f32_plan_check(gemm_f32_plan p, int *lost)
{
    if (!p || !lost) return GEMM_F32_ERR_INVALID_VALUE;
    *lost = 0;
    if (p->sliver) {
        const int st = gemm_f32_plan_check(p->sliver, lost);
        if (st != GEMM_F32_SUCCESS) return st;
    }
    if (!p->args.status) return GEMM_F32_SUCCESS;
    unsigned v = 0;
    hipError_t e = hipMemcpy(&v, p->args.status, sizeof(v), hipMemcpyDeviceToHost);
    if (e == hipSuccess && v) e = hipMemset(p->args.status, 0, sizeof(v));
    if (e != hipSuccess) return hip_fail(e);
    if (v) *lost = 1;
    return GEMM_F32_SUCCESS;
}

int gemm_f32_num_variants(void) { return V_COUNT; }

int gemm_f32_variant_info(int v, gemm_f32_info *info)
{
    if (!info || v < 0 || v >= V_COUNT) return GEMM_F32_ERR_INVALID_VALUE;
    fill_static_info(v, info);
    return GEMM_F32_SUCCESS;
}

const char *gemm_f32_error_string(int status)
{
    switch (status) {
    case GEMM_F32_SUCCESS: return "success";
    case GEMM_F32_ERR_INVALID_VALUE: return "invalid value (size, stride, layout, NULL or misaligned pointer)";
    case GEMM_F32_ERR_NO_DEVICE: return "no HIP device visible";
    case GEMM_F32_ERR_UNSUPPORTED_DEVICE: return "current device is not gfx950";
    case GEMM_F32_ERR_HIP: return "HIP runtime call failed (see gemm_f32_last_hip_error)";
    case GEMM_F32_ERR_ALLOC: return "host allocation failed";
    case GEMM_F32_ERR_SCRATCH_TOO_SMALL:
        return "the plan's partial sums exceed the static scratch area of gemm_f32_run_noalloc "
               "(64 MiB of partial-sum words, 65535 split tiles)";
    default: return "unknown status";
    }
}

int gemm_f32_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"

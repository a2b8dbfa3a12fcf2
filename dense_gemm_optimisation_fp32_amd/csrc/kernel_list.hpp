// Every kernel instantiation of the library, as X-macro lists over named
// tile types.  The host translation unit (gemm_f32.hip) declares each one
// `extern template`, and the kernel translation units (k_*.hip) define them
// by explicit instantiation, so the device code is compiled once, in
// several units that build in parallel.  A kernel the host unit uses that is
// missing here would be instantiated implicitly in the host unit; the build
// rejects that (it checks that the host unit compiles no kernel).
#pragma once

#include "mfma_dma_gemm.hpp"
#include "mfma_gemm.hpp"
#include "skinny_gemm.hpp"
#include "valu_gemm.hpp"
#include "fewcol_gemm.hpp"
#include "sliver_gemm.hpp"

namespace gemmf32 {

// Register-staged MFMA tiles (BM, BN, BK, wavefront grid).
using Reg256x256x16 = MfmaTile<256, 256, 16, 2, 2>;
using Reg128x128x16 = MfmaTile<128, 128, 16, 2, 2>;
using Reg256x128x16 = MfmaTile<256, 128, 16, 2, 2>;
using Reg256x128x32 = MfmaTile<256, 128, 32, 2, 2>;
using Reg128x128x32 = MfmaTile<128, 128, 32, 2, 2>;

// Direct-to-LDS tiles (BM, BN, BK, wavefront grid, LDS stages, priority).
using Dma256x256x16S2 = DmaTile<256, 256, 16, 2, 2, 2>;
using Dma256x256x16S3 = DmaTile<256, 256, 16, 2, 2, 3>;
using Dma256x256x16S4 = DmaTile<256, 256, 16, 2, 2, 4>;
using Dma256x256x32S2 = DmaTile<256, 256, 32, 2, 2, 2>;
using Dma128x128x16S3 = DmaTile<128, 128, 16, 2, 2, 3, false>;
using Dma128x128x32S3 = DmaTile<128, 128, 32, 2, 2, 3, false>;
using Dma256x128x16S3 = DmaTile<256, 128, 16, 2, 2, 3>;
using Dma64x64x16S3 = DmaTile<64, 64, 16, 2, 2, 3>;
using Dma64x64x16S2 = DmaTile<64, 64, 16, 2, 2, 2>;
using Dma128x64x16S2 = DmaTile<128, 64, 16, 2, 2, 2>;
using Dma128x64x16S3 = DmaTile<128, 64, 16, 2, 2, 3>;
using Dma64x128x16S2 = DmaTile<64, 128, 16, 2, 2, 2>;
using Dma64x128x16S3 = DmaTile<64, 128, 16, 2, 2, 3>;
using Dma256x256x16W24S4 = DmaTile<256, 256, 16, 2, 4, 4>;
using Dma256x256x16W42S4 = DmaTile<256, 256, 16, 4, 2, 4>;
using Dma256x256x16W42S2 = DmaTile<256, 256, 16, 4, 2, 2>;
using Dma256x256x16W44S4 = DmaTile<256, 256, 16, 4, 4, 4>;

// Zero n 32-bit words (the arrival counters of gemm_f32_run_noalloc's
// scratch area), with vector stores; defined in k_other.hip.
__global__ void zero_words_kernel(unsigned *p, int n);

// Few-column tiles (columns per workgroup).
using FewColR1 = FewColTile<1>;
using FewColR4 = FewColTile<4>;
using FewColR4K1024 = FewColTile<4, 8, 1, 1024>;   // eight wavefronts of one row
using FewColR1W8 = FewColTile<1, 8, 1, 2048>;      // the transposed one-row product's tile
using FewColR8W8 = FewColTile<8, 8, 1, 1024>;      // the transposed 5- to 8-row product's tile
using FewColR8 = FewColTile<8>;

// Few-row tiles (wavefronts, k groups in flight, columns).
using SkinnyW4D4 = SkinnyTile<4, 4, 64>;
using SkinnyW8D4 = SkinnyTile<8, 4, 64>;
using SkinnyW16D4 = SkinnyTile<16, 4, 64>;
using Skinny16W16D4 = SkinnyTile<16, 4, 16>;
using Skinny16W4D4 = SkinnyTile<4, 4, 16>;       // 16x16 tiles, 4 wavefronts
using Skinny32W8D4 = SkinnyTile<8, 4, 64, 2>;     // 32-row tiles
using Skinny16x32W16D4 = SkinnyTile<16, 4, 32>;   // 32-column tiles

}  // namespace gemmf32

// X5(kernel, Tile, B_COL, A_COL, EPI, WIDE_C) for gemm_mfma_dma_kernel;
// X2(kernel, Tile, B_COL) for the two-parameter kernels; X1(kernel, B_COL).

// Whole-tile and stream-K kernels of a direct-to-LDS tile (row-major A, no
// epilogue, one C element per store).
#define GEMMF32_DMA_BASE(X5, X2, T)                               \
    X5(gemm_mfma_dma_kernel, T, false, false, false, false)       \
    X5(gemm_mfma_dma_kernel, T, true, false, false, false)        \
    X2(gemm_mfma_dma_sk_kernel, T, false)                         \
    X2(gemm_mfma_dma_sk_kernel, T, true)
// Row-major B with NB (2 or 4) adjacent C columns per store.
#define GEMMF32_DMA_WIDE(X5, T) X5(gemm_mfma_dma_kernel, T, false, false, false, true)
// Column-major A and the linear-layer epilogue.
#define GEMMF32_DMA_EX(X5, T)                                     \
    X5(gemm_mfma_dma_kernel, T, false, true, false, false)        \
    X5(gemm_mfma_dma_kernel, T, true, true, false, false)         \
    X5(gemm_mfma_dma_kernel, T, false, false, true, false)        \
    X5(gemm_mfma_dma_kernel, T, true, false, true, false)         \
    X5(gemm_mfma_dma_kernel, T, false, true, true, false)         \
    X5(gemm_mfma_dma_kernel, T, true, true, true, false)
// Whole-tile kernels that carry a column sliver (the 128 x 128 tile: the
// dispatch's larger candidates pick shapes whose tiles fill whole waves, and
// the few-column path does not fit the 64-row tiles' register budget);
// _WIDE: with the 8/16-byte C stores.
#define GEMMF32_DMA_SLIVER(X5, T)                                 \
    X5(gemm_mfma_dma_sliver_kernel, T, false, false, false, false) \
    X5(gemm_mfma_dma_sliver_kernel, T, true, false, false, false)
#define GEMMF32_DMA_SLIVER_WIDE(X5, T) X5(gemm_mfma_dma_sliver_kernel, T, false, false, false, true)
#define GEMMF32_DMA_EX_WIDE(X5, T)                                \
    X5(gemm_mfma_dma_kernel, T, false, true, false, true)         \
    X5(gemm_mfma_dma_kernel, T, false, false, true, true)         \
    X5(gemm_mfma_dma_kernel, T, false, true, true, true)

// Kernel translation units.
#define GEMMF32_UNIT_DMA256(X5, X2, X1)                           \
    GEMMF32_DMA_BASE(X5, X2, Dma256x256x16S2) GEMMF32_DMA_WIDE(X5, Dma256x256x16S2) \
    GEMMF32_DMA_BASE(X5, X2, Dma256x256x16S3) GEMMF32_DMA_WIDE(X5, Dma256x256x16S3) \
    GEMMF32_DMA_BASE(X5, X2, Dma256x256x32S2) GEMMF32_DMA_WIDE(X5, Dma256x256x32S2)
#define GEMMF32_UNIT_DMA256S4(X5, X2, X1)                         \
    GEMMF32_DMA_BASE(X5, X2, Dma256x256x16S4) GEMMF32_DMA_WIDE(X5, Dma256x256x16S4) \
    GEMMF32_DMA_EX(X5, Dma256x256x16S4) GEMMF32_DMA_EX_WIDE(X5, Dma256x256x16S4)
#define GEMMF32_UNIT_DMA256x128(X5, X2, X1)                       \
    GEMMF32_DMA_BASE(X5, X2, Dma256x128x16S3) GEMMF32_DMA_WIDE(X5, Dma256x128x16S3) \
    GEMMF32_DMA_EX(X5, Dma256x128x16S3) GEMMF32_DMA_EX_WIDE(X5, Dma256x128x16S3)
#define GEMMF32_UNIT_DMA128(X5, X2, X1)                           \
    GEMMF32_DMA_BASE(X5, X2, Dma128x128x16S3) GEMMF32_DMA_WIDE(X5, Dma128x128x16S3) \
    GEMMF32_DMA_EX(X5, Dma128x128x16S3) GEMMF32_DMA_EX_WIDE(X5, Dma128x128x16S3) \
    GEMMF32_DMA_SLIVER(X5, Dma128x128x16S3) GEMMF32_DMA_SLIVER_WIDE(X5, Dma128x128x16S3) \
    X2(gemm_mfma_dma_sk_epi_kernel, Dma128x128x16S3, false) X2(gemm_mfma_dma_sk_epi_kernel, Dma128x128x16S3, true) \
    GEMMF32_DMA_BASE(X5, X2, Dma128x128x32S3) GEMMF32_DMA_WIDE(X5, Dma128x128x32S3)
#define GEMMF32_UNIT_DMA64(X5, X2, X1)                            \
    GEMMF32_DMA_BASE(X5, X2, Dma64x64x16S3) GEMMF32_DMA_EX(X5, Dma64x64x16S3) \
    GEMMF32_DMA_BASE(X5, X2, Dma64x64x16S2) GEMMF32_DMA_EX(X5, Dma64x64x16S2) \
    X2(gemm_mfma_dma_sk_epi_kernel, Dma64x64x16S2, false) X2(gemm_mfma_dma_sk_epi_kernel, Dma64x64x16S2, true) \
    GEMMF32_DMA_BASE(X5, X2, Dma128x64x16S2) GEMMF32_DMA_BASE(X5, X2, Dma128x64x16S3)
#define GEMMF32_UNIT_DMA64x128(X5, X2, X1)                        \
    GEMMF32_DMA_BASE(X5, X2, Dma64x128x16S2) GEMMF32_DMA_WIDE(X5, Dma64x128x16S2) \
    GEMMF32_DMA_EX(X5, Dma64x128x16S2) GEMMF32_DMA_EX_WIDE(X5, Dma64x128x16S2) \
    GEMMF32_DMA_BASE(X5, X2, Dma64x128x16S3) GEMMF32_DMA_WIDE(X5, Dma64x128x16S3)
#define GEMMF32_UNIT_DMA256W8(X5, X2, X1)                         \
    GEMMF32_DMA_BASE(X5, X2, Dma256x256x16W24S4) GEMMF32_DMA_WIDE(X5, Dma256x256x16W24S4) \
    GEMMF32_DMA_BASE(X5, X2, Dma256x256x16W42S4) GEMMF32_DMA_WIDE(X5, Dma256x256x16W42S4) \
    GEMMF32_DMA_EX(X5, Dma256x256x16W42S4) GEMMF32_DMA_EX_WIDE(X5, Dma256x256x16W42S4) \
    GEMMF32_DMA_BASE(X5, X2, Dma256x256x16W42S2) GEMMF32_DMA_WIDE(X5, Dma256x256x16W42S2) \
    GEMMF32_DMA_BASE(X5, X2, Dma256x256x16W44S4) GEMMF32_DMA_WIDE(X5, Dma256x256x16W44S4)
#define GEMMF32_UNIT_OTHER(X5, X2, X1)                            \
    X2(gemm_mfma_kernel, Reg256x256x16, false) X2(gemm_mfma_kernel, Reg256x256x16, true) \
    X2(gemm_mfma_kernel, Reg128x128x16, false) X2(gemm_mfma_kernel, Reg128x128x16, true) \
    X2(gemm_mfma_kernel, Reg256x128x16, false) X2(gemm_mfma_kernel, Reg256x128x16, true) \
    X2(gemm_mfma_kernel, Reg256x128x32, false) X2(gemm_mfma_kernel, Reg256x128x32, true) \
    X2(gemm_mfma_kernel, Reg128x128x32, false) X2(gemm_mfma_kernel, Reg128x128x32, true) \
    X1(gemm_valu_kernel, false) X1(gemm_valu_kernel, true)                                   \
    X2(gemm_skinny_kernel, SkinnyW4D4, false) X2(gemm_skinny_kernel, SkinnyW4D4, true) X2(gemm_skinny_epi_kernel, SkinnyW4D4, false) X2(gemm_skinny_epi_kernel, SkinnyW4D4, true) \
    X2(gemm_skinny_acol_kernel, SkinnyW4D4, false) X2(gemm_skinny_acol_kernel, SkinnyW4D4, true) X2(gemm_skinny_acol_epi_kernel, SkinnyW4D4, false) X2(gemm_skinny_acol_epi_kernel, SkinnyW4D4, true)       \
    X2(gemm_skinny_kernel, SkinnyW8D4, false) X2(gemm_skinny_kernel, SkinnyW8D4, true) X2(gemm_skinny_epi_kernel, SkinnyW8D4, false) X2(gemm_skinny_epi_kernel, SkinnyW8D4, true) \
    X2(gemm_skinny_acol_kernel, SkinnyW8D4, false) X2(gemm_skinny_acol_kernel, SkinnyW8D4, true) X2(gemm_skinny_acol_epi_kernel, SkinnyW8D4, false) X2(gemm_skinny_acol_epi_kernel, SkinnyW8D4, true)       \
    X2(gemm_skinny_kernel, SkinnyW16D4, false) X2(gemm_skinny_kernel, SkinnyW16D4, true) X2(gemm_skinny_epi_kernel, SkinnyW16D4, false) X2(gemm_skinny_epi_kernel, SkinnyW16D4, true) \
    X2(gemm_skinny_acol_kernel, SkinnyW16D4, false) X2(gemm_skinny_acol_kernel, SkinnyW16D4, true) X2(gemm_skinny_acol_epi_kernel, SkinnyW16D4, false) X2(gemm_skinny_acol_epi_kernel, SkinnyW16D4, true)     \
    X2(gemm_skinny_kernel, Skinny16W16D4, false) X2(gemm_skinny_kernel, Skinny16W16D4, true) X2(gemm_skinny_epi_kernel, Skinny16W16D4, false) X2(gemm_skinny_epi_kernel, Skinny16W16D4, true) \
    X2(gemm_skinny_acol_kernel, Skinny16W16D4, false) X2(gemm_skinny_acol_kernel, Skinny16W16D4, true) X2(gemm_skinny_acol_epi_kernel, Skinny16W16D4, false) X2(gemm_skinny_acol_epi_kernel, Skinny16W16D4, true)     \
    X2(gemm_skinny_kernel, Skinny16W4D4, false) X2(gemm_skinny_kernel, Skinny16W4D4, true) X2(gemm_skinny_epi_kernel, Skinny16W4D4, false) X2(gemm_skinny_epi_kernel, Skinny16W4D4, true) \
    X2(gemm_skinny_acol_kernel, Skinny16W4D4, false) X2(gemm_skinny_acol_kernel, Skinny16W4D4, true) X2(gemm_skinny_acol_epi_kernel, Skinny16W4D4, false) X2(gemm_skinny_acol_epi_kernel, Skinny16W4D4, true)     \
    X2(gemm_skinny_kernel, Skinny32W8D4, false) X2(gemm_skinny_kernel, Skinny32W8D4, true) X2(gemm_skinny_epi_kernel, Skinny32W8D4, false) X2(gemm_skinny_epi_kernel, Skinny32W8D4, true) \
    X2(gemm_skinny_acol_kernel, Skinny32W8D4, false) X2(gemm_skinny_acol_kernel, Skinny32W8D4, true) X2(gemm_skinny_acol_epi_kernel, Skinny32W8D4, false) X2(gemm_skinny_acol_epi_kernel, Skinny32W8D4, true)       \
    X2(gemm_skinny_kernel, Skinny16x32W16D4, false) X2(gemm_skinny_kernel, Skinny16x32W16D4, true) X2(gemm_skinny_epi_kernel, Skinny16x32W16D4, false) X2(gemm_skinny_epi_kernel, Skinny16x32W16D4, true) \
    X2(gemm_skinny_acol_kernel, Skinny16x32W16D4, false) X2(gemm_skinny_acol_kernel, Skinny16x32W16D4, true) X2(gemm_skinny_acol_epi_kernel, Skinny16x32W16D4, false) X2(gemm_skinny_acol_epi_kernel, Skinny16x32W16D4, true) \
    X2(gemm_fewcol_kernel, FewColR1, false) X2(gemm_fewcol_kernel, FewColR1, true) X2(gemm_fewcol_epi_kernel, FewColR1, false) X2(gemm_fewcol_epi_kernel, FewColR1, true)             \
    X2(gemm_fewcol_t_kernel, FewColR1, true) X2(gemm_fewcol_t_epi_kernel, FewColR1, true)          \
    X2(gemm_fewcol_kernel, FewColR4, false) X2(gemm_fewcol_kernel, FewColR4, true) X2(gemm_fewcol_epi_kernel, FewColR4, false) X2(gemm_fewcol_epi_kernel, FewColR4, true)             \
    X2(gemm_fewcol_kernel, FewColR1W8, false) X2(gemm_fewcol_kernel, FewColR1W8, true) X2(gemm_fewcol_epi_kernel, FewColR1W8, false) X2(gemm_fewcol_epi_kernel, FewColR1W8, true) \
    X2(gemm_fewcol_t_kernel, FewColR1W8, true) X2(gemm_fewcol_t_epi_kernel, FewColR1W8, true) \
    X2(gemm_fewcol_kernel, FewColR8W8, false) X2(gemm_fewcol_kernel, FewColR8W8, true) X2(gemm_fewcol_epi_kernel, FewColR8W8, false) X2(gemm_fewcol_epi_kernel, FewColR8W8, true) \
    X2(gemm_fewcol_t_kernel, FewColR8W8, true) X2(gemm_fewcol_t_epi_kernel, FewColR8W8, true) \
    X2(gemm_fewcol_kernel, FewColR8, false) X2(gemm_fewcol_kernel, FewColR8, true) X2(gemm_fewcol_epi_kernel, FewColR8, false) X2(gemm_fewcol_epi_kernel, FewColR8, true)             \
    X2(gemm_fewcol_kernel, FewColR4K1024, false) X2(gemm_fewcol_kernel, FewColR4K1024, true) X2(gemm_fewcol_epi_kernel, FewColR4K1024, false) X2(gemm_fewcol_epi_kernel, FewColR4K1024, true)   \
    X2(gemm_fewcol_t_kernel, FewColR4K1024, true) X2(gemm_fewcol_t_epi_kernel, FewColR4K1024, true)

#define GEMMF32_ALL_UNITS(X5, X2, X1)                                                     \
    GEMMF32_UNIT_DMA256(X5, X2, X1) GEMMF32_UNIT_DMA256S4(X5, X2, X1)                     \
    GEMMF32_UNIT_DMA256x128(X5, X2, X1) GEMMF32_UNIT_DMA128(X5, X2, X1)                   \
    GEMMF32_UNIT_DMA64(X5, X2, X1) GEMMF32_UNIT_DMA64x128(X5, X2, X1)                     \
    GEMMF32_UNIT_DMA256W8(X5, X2, X1) GEMMF32_UNIT_OTHER(X5, X2, X1)

// Explicit instantiation definitions (kernel units) and declarations (host unit).
#define GEMMF32_DEFINE5(K, T, a, b, c, d) template __global__ void gemmf32::K<gemmf32::T, a, b, c, d>(gemmf32::GemmArgs);
#define GEMMF32_DEFINE2(K, T, a) template __global__ void gemmf32::K<gemmf32::T, a>(gemmf32::GemmArgs);
#define GEMMF32_DEFINE1(K, a) template __global__ void gemmf32::K<a>(gemmf32::GemmArgs);
#define GEMMF32_EXTERN5(K, T, a, b, c, d) extern template __global__ void gemmf32::K<gemmf32::T, a, b, c, d>(gemmf32::GemmArgs);
#define GEMMF32_EXTERN2(K, T, a) extern template __global__ void gemmf32::K<gemmf32::T, a>(gemmf32::GemmArgs);
#define GEMMF32_EXTERN1(K, a) extern template __global__ void gemmf32::K<a>(gemmf32::GemmArgs);

// Kernel translation unit: explicit instantiations of the GEMMF32_UNIT_DMA256W8
// list of kernel_list.hpp (compiled in parallel with the other units).
#include "kernel_list.hpp"

GEMMF32_UNIT_DMA256W8(GEMMF32_DEFINE5, GEMMF32_DEFINE2, GEMMF32_DEFINE1)

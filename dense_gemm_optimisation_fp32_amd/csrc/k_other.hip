// Kernel translation unit: explicit instantiations of the GEMMF32_UNIT_OTHER
// list of kernel_list.hpp (compiled in parallel with the other units).
#include "kernel_list.hpp"

GEMMF32_UNIT_OTHER(GEMMF32_DEFINE5, GEMMF32_DEFINE2, GEMMF32_DEFINE1)

__global__ void gemmf32::zero_words_kernel(unsigned *p, int n)
{
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// The linear-layer epilogue on one element of C, for the kernels that write
// C one element at a time (the few-row and few-column kernels): the
// arithmetic of the whole-tile kernels' epilogue, act(alpha * x + beta *
// C[r][c] + bias[c]), with C read only when beta != 0 and the bias only when
// there is one.
#pragma once

#include "device_common.hpp"

namespace gemmf32 {

__device__ __forceinline__ float linear_epilogue(const GemmArgs &g, float x, int r, int c)
{
    const float cold = g.use_beta ? g.C[(size_t)r * g.ldc + c] : 0.0f;
    const float bias = g.bias ? g.bias[c] : 0.0f;
    const float y = fmaxf(g.alpha * x + g.beta * cold + bias, g.act == 1 ? 0.0f : -__builtin_inff());
    return g.act == 2 ? gelu_erf(y) : y;
}

}  // namespace gemmf32

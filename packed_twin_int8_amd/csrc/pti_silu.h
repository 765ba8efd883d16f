// SiLU(g) * u, the gated activation of the stand-in decoder stack (a
// random-weight MLP-residual stack with the step structure of [Digest =
// "Packed Twin Inference：无需草稿模型的推测解码新方案，实现2倍吞吐量提升",
// section "技术实现架构" (implementation architecture)]), shared by the
// elementwise kernels and the gate|up GEMV that applies it to its own two
// outputs, so that every path gives the same bits.  Computed in fp64 and
// rounded once to fp32 (within one fp32 ulp of the exact value); no
// contraction, so the operation sequence is the same at every call site.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>

namespace pti_silu {

__device__ __forceinline__ float silu_mul(float g, float u)
{
#pragma clang fp contract(off)
    const double gv = g;
    return float(gv / (1.0 + exp(-gv)) * double(u));
}

}  // namespace pti_silu

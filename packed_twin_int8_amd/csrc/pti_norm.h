// RMSNorm arithmetic shared by pti_rmsnorm and the GEMV that normalises x
// while staging it, so that both give the same bits.
//
// The norm of the stand-in decoder stack (a random-weight MLP-residual stack
// with the step structure of [Digest = "Packed Twin Inference：无需草稿模型的
// 推测解码新方案，实现2倍吞吐量提升", section "技术实现架构" (implementation
// architecture)]): y = x / sqrt(mean(x^2) + eps), no gain.  Computed in fp64
// and rounded once to fp32: a group of 256
// threads, thread t summing x[t], x[t + 256], ... with one fp64 FMA each, each
// wave of 64 reducing with a fixed butterfly, the four wave sums added in
// order; every element is then multiplied by the fp64 reciprocal of the root
// (one division per vector, not per element).
#pragma once

#include <hip/hip_runtime.h>

namespace pti_norm {

constexpr int kGroup = 256;  // threads that form the sum of squares

__device__ __forceinline__ double sq_acc(double acc, float v)
{
    const double d = v;
    return __builtin_fma(d, d, acc);
}

__device__ __forceinline__ double wave_sum_f64(double v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

// 1 / root from the four wave sums part[0..3].
__device__ __forceinline__ double inv_root(const double *part, int64_t dim, double eps)
{
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < kGroup / 64; i++)
        ss += part[i];
    return 1.0 / sqrt(ss / double(dim) + eps);
}

// x * (1 / root) in fp64, rounded once to fp32: two fp64 roundings before the
// last, so the result is within one fp32 ulp of x / root.
__device__ __forceinline__ float apply(float v, double inv) { return float(double(v) * inv); }

}  // namespace pti_norm

// Greedy verify for staggered self-speculation on gfx950.
//
// [README = "打包双子推理（PTI）", section "接受机制如何工作" (how acceptance
// works); Digest = "Packed Twin Inference：无需草稿模型的推测解码新方案，实现2倍
// 吞吐量提升", section "技术实现架构" (implementation architecture), step 3]:
// stream 0 decodes from the confirmed token, stream i >= 1 from a guess of the
// token stream i-1 produces.  Under greedy decoding each stream's token is the
// argmax of its logits; the guess of stream i is confirmed when it equals
// stream i-1's token, and the first failed check voids every later stream.
//
// One workgroup of 1024 threads (16 wave64s) handles all streams: the logits
// of a step are at most 4 x vocab floats, so one CU streams them in a few
// microseconds and no cross-workgroup combine (and no scratch memory) is
// needed.  Each thread scans a strided slice with 16-byte loads keeping the
// first maximum it meets; slices combine with (value larger, or equal and index
// lower), first across a wavefront with shuffles, then across waves in LDS.
#include <hip/hip_runtime.h>

#include <climits>

#include "pti_internal.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

struct Best {
    float v;
    int i;
};

__device__ __forceinline__ Best better(Best a, Best b)
{
    return (b.v > a.v || (b.v == a.v && b.i < a.i)) ? b : a;
}

__device__ __forceinline__ Best wave_best(Best b)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        Best o;
        o.v = __shfl_xor(b.v, off, 64);
        o.i = __shfl_xor(b.i, off, 64);
        b = better(b, o);
    }
    return b;
}

template <bool VEC4>
__global__ __launch_bounds__(kThreads) void verify_kernel(const float *__restrict__ logits,
                                                          const int32_t *__restrict__ tokens_in,
                                                          int32_t *__restrict__ argmax_out,
                                                          int32_t *__restrict__ accept_out, int64_t vocab,
                                                          int n)
{
    __shared__ Best part[kWaves];
    __shared__ int amax[4];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    for (int s = 0; s < n; s++) {
        const float *v = logits + (int64_t)s * vocab;
        Best b{-__builtin_inff(), INT_MAX};
        if constexpr (VEC4) {
            const float4 *v4 = reinterpret_cast<const float4 *>(v);
            const int64_t n4 = vocab / 4;
            for (int64_t k = tid; k < n4; k += kThreads) {
                const float4 t = v4[k];
                const int i0 = (int)(4 * k);
                // indices rise within and across iterations: strict > keeps the first maximum,
                // the index test admits a first element equal to the initial -inf
                if (t.x > b.v || b.i == INT_MAX) b = Best{t.x, i0};
                if (t.y > b.v) b = Best{t.y, i0 + 1};
                if (t.z > b.v) b = Best{t.z, i0 + 2};
                if (t.w > b.v) b = Best{t.w, i0 + 3};
            }
        } else {
            for (int64_t k = tid; k < vocab; k += kThreads) {
                const float t = v[k];
                if (t > b.v || b.i == INT_MAX)
                    b = Best{t, (int)k};
            }
        }
        b = wave_best(b);
        if (lane == 0)
            part[wv] = b;
        __syncthreads();
        if (wv == 0) {
            Best c = lane < kWaves ? part[lane] : Best{-__builtin_inff(), INT_MAX};
            c = wave_best(c);
            if (lane == 0) {
                amax[s] = c.i;
                argmax_out[s] = c.i;
            }
        }
        __syncthreads();
    }
    if (tid == 0) {
        int a = 1;
        for (int i = 1; i < n; i++) {
            if (tokens_in[i] != amax[i - 1])
                break;
            a++;
        }
        accept_out[0] = a;
    }
}

}  // namespace

extern "C" int pti_verify_argmax(const float *logits, const int32_t *tokens_in, int32_t *argmax_out,
                                 int32_t *accept_out, int64_t vocab, int n_streams, void *stream)
{
    if (!logits || !tokens_in || !argmax_out || !accept_out)
        return PTI_ERR_NULL;
    if (vocab < 1 || vocab > PTI_MAX_VOCAB)
        return PTI_ERR_SHAPE;
    if (n_streams < 1 || n_streams > PTI_MAX_STREAMS)
        return PTI_ERR_NSTREAMS;
    if (!pti::aligned(logits, 4) || !pti::aligned(tokens_in, 4) || !pti::aligned(argmax_out, 4) ||
        !pti::aligned(accept_out, 4))
        return PTI_ERR_ALIGN;
    const pti::Range L{logits, size_t(n_streams) * size_t(vocab) * 4}, T{tokens_in, size_t(n_streams) * 4},
        A{argmax_out, size_t(n_streams) * 4}, C{accept_out, 4};
    if (pti::overlap(A, L) || pti::overlap(A, T) || pti::overlap(C, L) || pti::overlap(C, T) || pti::overlap(A, C))
        return PTI_ERR_OVERLAP;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool vec4 = vocab % 4 == 0 && pti::aligned(logits, 16);
    if (vec4)
        hipLaunchKernelGGL(verify_kernel<true>, dim3(1), dim3(kThreads), 0, st, logits, tokens_in, argmax_out,
                           accept_out, vocab, n_streams);
    else
        hipLaunchKernelGGL(verify_kernel<false>, dim3(1), dim3(kThreads), 0, st, logits, tokens_in, argmax_out,
                           accept_out, vocab, n_streams);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        pti::set_hip_error(e);
        return PTI_ERR_HIP;
    }
    return PTI_OK;
}

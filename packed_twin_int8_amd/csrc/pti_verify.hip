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
// needed.  Each thread scans a strided slice of every stream in one pass with
// 16-byte loads, keeping the first maximum it meets; slices combine with
// (value larger, or equal and index lower), first across a wavefront with
// shuffles, then across waves in LDS.
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

// All streams in one pass: a thread keeps the first maximum of its strided
// slice of every stream, with UNROLL independent 16-byte loads per stream in
// flight; slices combine with better() across the wave, then across waves.
template <bool VEC4, int NS>
__global__ __launch_bounds__(kThreads) void verify_kernel(const pti::StreamRows logits,
                                                          const int32_t *__restrict__ tokens_in,
                                                          int32_t *__restrict__ argmax_out,
                                                          int32_t *__restrict__ accept_out, int64_t vocab)
{
    constexpr int UNROLL = 4;
    __shared__ Best part[NS][kWaves];
    __shared__ int amax[NS];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    Best b[NS];
#pragma unroll
    for (int s = 0; s < NS; s++)
        b[s] = Best{-__builtin_inff(), INT_MAX};
    // indices rise within and across iterations: strict > keeps the first
    // maximum, the index test admits a first element equal to the initial -inf
    auto take = [&](Best &bb, float v, int i) {
        if (v > bb.v || bb.i == INT_MAX)
            bb = Best{v, i};
    };
    if constexpr (VEC4) {
        const int64_t n4 = vocab / 4;
        int64_t k = tid;
        for (; k + (UNROLL - 1) * kThreads < n4; k += UNROLL * kThreads) {
            float4 t[NS][UNROLL];
#pragma unroll
            for (int s = 0; s < NS; s++)
#pragma unroll
                for (int u = 0; u < UNROLL; u++)
                    t[s][u] = reinterpret_cast<const float4 *>(logits.p[s])[k + u * kThreads];
#pragma unroll
            for (int u = 0; u < UNROLL; u++) {
                const int i0 = (int)(4 * (k + u * kThreads));
#pragma unroll
                for (int s = 0; s < NS; s++) {
                    take(b[s], t[s][u].x, i0);
                    take(b[s], t[s][u].y, i0 + 1);
                    take(b[s], t[s][u].z, i0 + 2);
                    take(b[s], t[s][u].w, i0 + 3);
                }
            }
        }
        for (; k < n4; k += kThreads) {
            const int i0 = (int)(4 * k);
#pragma unroll
            for (int s = 0; s < NS; s++) {
                const float4 t = reinterpret_cast<const float4 *>(logits.p[s])[k];
                take(b[s], t.x, i0);
                take(b[s], t.y, i0 + 1);
                take(b[s], t.z, i0 + 2);
                take(b[s], t.w, i0 + 3);
            }
        }
    } else {
        for (int64_t k = tid; k < vocab; k += kThreads)
#pragma unroll
            for (int s = 0; s < NS; s++)
                take(b[s], logits.p[s][k], (int)k);
    }
#pragma unroll
    for (int s = 0; s < NS; s++) {
        b[s] = wave_best(b[s]);
        if (lane == 0)
            part[s][wv] = b[s];
    }
    __syncthreads();
    if (wv == 0) {
#pragma unroll
        for (int s = 0; s < NS; s++) {
            Best c = lane < kWaves ? part[s][lane] : Best{-__builtin_inff(), INT_MAX};
            c = wave_best(c);
            if (lane == 0) {
                amax[s] = c.i;
                argmax_out[s] = c.i;
            }
        }
    }
    __syncthreads();
    if (tid == 0) {
        int a = 1;
        for (int i = 1; i < NS; i++) {
            if (tokens_in[i] != amax[i - 1])
                break;
            a++;
        }
        accept_out[0] = a;
    }
}

template <bool VEC4>
void launch_verify(const pti::StreamRows &lg, const int32_t *tokens_in, int32_t *argmax_out, int32_t *accept_out,
                   int64_t vocab, int n, hipStream_t st)
{
    switch (n) {
    case 1:
        hipLaunchKernelGGL((verify_kernel<VEC4, 1>), dim3(1), dim3(kThreads), 0, st, lg, tokens_in, argmax_out,
                           accept_out, vocab);
        break;
    case 2:
        hipLaunchKernelGGL((verify_kernel<VEC4, 2>), dim3(1), dim3(kThreads), 0, st, lg, tokens_in, argmax_out,
                           accept_out, vocab);
        break;
    case 3:
        hipLaunchKernelGGL((verify_kernel<VEC4, 3>), dim3(1), dim3(kThreads), 0, st, lg, tokens_in, argmax_out,
                           accept_out, vocab);
        break;
    default:
        hipLaunchKernelGGL((verify_kernel<VEC4, 4>), dim3(1), dim3(kThreads), 0, st, lg, tokens_in, argmax_out,
                           accept_out, vocab);
        break;
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
    pti::StreamRows lg{};
    for (int s = 0; s < n_streams; s++)
        lg.p[s] = logits + (int64_t)s * vocab;
    return pti::launch_verify_rows(lg, tokens_in, argmax_out, accept_out, vocab, n_streams, stream);
}

namespace pti {
int launch_verify_rows(const StreamRows &lg, const int32_t *tokens_in, int32_t *argmax_out, int32_t *accept_out,
                       int64_t vocab, int n_streams, void *stream)
{
    hipStream_t st = static_cast<hipStream_t>(stream);
    bool vec4 = vocab % 4 == 0;
    for (int s = 0; s < n_streams; s++)
        vec4 = vec4 && aligned(lg.p[s], 16);
    if (vec4)
        launch_verify<true>(lg, tokens_in, argmax_out, accept_out, vocab, n_streams, st);
    else
        launch_verify<false>(lg, tokens_in, argmax_out, accept_out, vocab, n_streams, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        set_hip_error(e);
        return PTI_ERR_HIP;
    }
    return PTI_OK;
}
}  // namespace pti

// Glue kernels of the decoder stack around the packed GEMVs, and the sampled
// verify, for gfx950.
//
// [Digest = "Packed Twin Inference：无需草稿模型的推测解码新方案，实现2倍吞吐量提升",
// section "技术实现架构" (implementation architecture): the kernel set holds the
// matrix products, the verify and a softmax; README = "打包双子推理（PTI）",
// section "接受机制如何工作" (how acceptance works): at temperature > 0 each
// stream samples its token and a guess is confirmed when it equals the sample
// of the stream before it.]
//
// These kernels move a few hundred KB per call, so they are bound by launch
// latency, not by HBM.  They compute in fp64 internally and round once to fp32
// at the end: the cost is invisible at these sizes and each output is then the
// correctly rounded value of its formula up to the last fp64 ulp.
//   * embed: dequantise one matrix row per stream (scale * q is exact in fp32).
//   * rmsnorm: y = x / sqrt(mean(x^2) + eps), one workgroup per stream.
//   * silu_mul: y = g / (1 + exp(-g)) * u, elementwise.
//   * add: y = a + b in fp32, elementwise.
//   * sample_verify: per stream, weights w_j = exp((l_j - max) / t) in fp64 and
//     the smallest index whose running sum of weights exceeds u * sum(w); then
//     the accept count of the drawn tokens.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>

#include "pti_internal.h"

namespace {

__device__ __forceinline__ float f16_to_f32(uint32_t bits)
{
    union {
        uint16_t u;
        _Float16 f;
    } c;
    c.u = static_cast<uint16_t>(bits);
    return static_cast<float>(c.f);
}

// ------------------------------------------------------------------ embed

__global__ void embed_q8_kernel(const uint8_t *__restrict__ w, const int32_t *__restrict__ tokens,
                                float *__restrict__ x, int64_t vocab, int64_t hidden)
{
    const int s = blockIdx.y;
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= hidden)
        return;
    const int64_t t = tokens[s];
    float v = __builtin_nanf("");
    if (t >= 0 && t < vocab) {
        const uint8_t *blk = w + (t * (hidden / 32) + c / 32) * PTI_Q8_BLOCK_BYTES;
        v = f16_to_f32(blk[0] | (uint32_t(blk[1]) << 8)) * float(int8_t(blk[2 + (c & 31)]));
    }
    x[s * hidden + c] = v;
}

// Stream 0 reads twin A's row tokens[0], stream 1 twin B's row tokens[1].
__global__ void embed_ssq_kernel(const uint8_t *__restrict__ w, const int32_t *__restrict__ tokens,
                                 float *__restrict__ x, int64_t vocab, int64_t hidden)
{
    const int s = blockIdx.y;
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= hidden)
        return;
    const int64_t t = tokens[s];
    float v = __builtin_nanf("");
    if (t >= 0 && t < vocab) {
        const uint8_t *blk = w + (t * (hidden / 32) + c / 32) * PTI_SSQ_BLOCK_BYTES;
        const uint8_t *sc = blk + 2 * s;                    // scale_A, then scale_B
        const uint8_t q = blk[4 + 2 * (c & 31) + (1 - s)];  // slot byte 1 = A, byte 0 = B
        v = f16_to_f32(sc[0] | (uint32_t(sc[1]) << 8)) * float(int8_t(q));
    }
    x[s * hidden + c] = v;
}

// ------------------------------------------------------------------ reductions

__device__ __forceinline__ double wave_sum_f64(double v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

__device__ __forceinline__ float wave_max_f32(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

// ------------------------------------------------------------------ rmsnorm

constexpr int kNormThreads = 256;

__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(const float *__restrict__ x, float *__restrict__ y,
                                                               int64_t dim, double eps)
{
    __shared__ double part[kNormThreads / 64];
    __shared__ double root;
    const int tid = threadIdx.x;
    const float *xs = x + blockIdx.x * dim;
    float *ys = y + blockIdx.x * dim;
    double acc = 0.0;
    for (int64_t c = tid; c < dim; c += kNormThreads) {
        const double v = xs[c];
        acc += v * v;
    }
    acc = wave_sum_f64(acc);
    if ((tid & 63) == 0)
        part[tid >> 6] = acc;
    __syncthreads();
    if (tid == 0) {
        double ss = 0.0;
        for (int i = 0; i < kNormThreads / 64; i++)
            ss += part[i];
        root = sqrt(ss / double(dim) + eps);
    }
    __syncthreads();
    const double r = root;
    for (int64_t c = tid; c < dim; c += kNormThreads)
        ys[c] = float(double(xs[c]) / r);
}

// ------------------------------------------------------------------ elementwise

__global__ void silu_mul_kernel(const float *g, const float *u, float *y, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const double gv = g[i];
        y[i] = float(gv / (1.0 + exp(-gv)) * double(u[i]));
    }
}

// The same arithmetic on the rows of a stacked gate|up output: g = gu[s][j],
// u = gu[s][cols + j].
__global__ void silu_mul_rows_kernel(const float *gu, float *y, int64_t rows, int64_t cols)
{
    const int64_t n = rows * cols;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t s = i / cols, j = i - s * cols;
        const double gv = gu[s * 2 * cols + j];
        y[i] = float(gv / (1.0 + exp(-gv)) * double(gu[s * 2 * cols + cols + j]));
    }
}

__global__ void add_kernel(const float *a, const float *b, float *y, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        y[i] = a[i] + b[i];
}

// ------------------------------------------------------------------ sampled verify

constexpr int kSampleThreads = 1024;
constexpr int kSampleWaves = kSampleThreads / 64;

// One workgroup per stream draws that stream's token.  Sums are taken in a
// fixed order that never decreases along the index: each thread owns a
// contiguous chunk of the vocabulary and sums it in index order; chunk sums
// are prefixed sequentially within a wave, then wave totals sequentially.
// The drawn index is the first one, in that order, whose running sum exceeds
// u * Z among indices of nonzero weight; if rounding leaves none, the last
// index of nonzero weight in the chunk that holds the target.  No positive
// weight (non-finite logits) draws -1.
__global__ __launch_bounds__(kSampleThreads) void sample_draw_kernel(const float *__restrict__ logits,
                                                                     const double *__restrict__ uniforms,
                                                                     double temperature,
                                                                     int32_t *__restrict__ tokens_out, int64_t vocab)
{
    __shared__ double loc_s[kSampleThreads];
    __shared__ double pre_s[kSampleThreads];
    __shared__ double wbase[kSampleWaves + 1];
    __shared__ float wmax[kSampleWaves];
    __shared__ int owner;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, s = blockIdx.x;
    const int64_t chunk = (vocab + kSampleThreads - 1) / kSampleThreads;
    const int64_t j0 = min(vocab, int64_t(tid) * chunk), j1 = min(vocab, j0 + chunk);
    const float *v = logits + (int64_t)s * vocab;
    float m = -__builtin_inff();
    for (int64_t j = j0; j < j1; j++)
        m = fmaxf(m, v[j]);
    m = wave_max_f32(m);
    if (lane == 0)
        wmax[wv] = m;
    __syncthreads();
    m = wmax[0];
    for (int i = 1; i < kSampleWaves; i++)
        m = fmaxf(m, wmax[i]);
    const double md = m;
    double loc = 0.0;
    for (int64_t j = j0; j < j1; j++)
        loc += exp((double(v[j]) - md) / temperature);
    loc_s[tid] = loc;
    if (tid == 0)
        owner = -1;
    __syncthreads();
    if (lane == 0) {
        double run = 0.0;
        for (int i = 0; i < 64; i++) {
            pre_s[tid + i] = run;
            run += loc_s[tid + i];
        }
        wbase[wv + 1] = run;  // wave total, prefixed below
    }
    __syncthreads();
    if (tid == 0) {
        double run = 0.0;
        for (int w = 0; w < kSampleWaves; w++) {
            const double tot = wbase[w + 1];
            wbase[w] = run;
            run += tot;
        }
        wbase[kSampleWaves] = run;  // Z
    }
    __syncthreads();
    const double Z = wbase[kSampleWaves];
    const double target = uniforms[s] * Z;
    const double excl = wbase[wv] + pre_s[tid];
    if (loc > 0.0 && excl <= target)
        atomicMax(&owner, tid);
    __syncthreads();
    if (tid == 0 && owner < 0)  // no positive weight: non-finite logits
        tokens_out[s] = -1;
    if (tid == owner) {
        double run = excl;
        int64_t pick = -1, last = -1;
        for (int64_t j = j0; j < j1; j++) {
            const double e = exp((double(v[j]) - md) / temperature);
            if (e > 0.0) {
                last = j;
                run += e;
                if (run > target) {
                    pick = j;
                    break;
                }
            }
        }
        if (pick < 0)
            pick = last;
        tokens_out[s] = int32_t(pick);
    }
}

// The accept count from the draws: 1 + the leading run of i >= 1 with
// tokens_in[i] == tokens_out[i - 1].
__global__ void accept_kernel(const int32_t *__restrict__ tokens_in, const int32_t *__restrict__ tokens_out,
                              int32_t *__restrict__ accept_out, int n)
{
    if (threadIdx.x == 0) {
        int a = 1;
        for (int i = 1; i < n; i++) {
            if (tokens_in[i] != tokens_out[i - 1])
                break;
            a++;
        }
        accept_out[0] = a;
    }
}

int launch_status()
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        pti::set_hip_error(e);
        return PTI_ERR_HIP;
    }
    return PTI_OK;
}

bool elem_ok(int64_t n) { return n >= 1 && n <= PTI_MAX_ELEMS; }

}  // namespace

extern "C" int pti_embed_q8(const void *w_q8, const int32_t *tokens, float *x, int64_t vocab, int64_t hidden,
                            int n_streams, void *stream)
{
    if (!w_q8 || !tokens || !x)
        return PTI_ERR_NULL;
    if (!pti::shape_ok(vocab, hidden))
        return PTI_ERR_SHAPE;
    if (n_streams < 1 || n_streams > PTI_MAX_STREAMS)
        return PTI_ERR_NSTREAMS;
    if (!pti::aligned(tokens, 4) || !pti::aligned(x, 4))
        return PTI_ERR_ALIGN;
    const pti::Range X{x, size_t(n_streams) * size_t(hidden) * 4};
    if (pti::overlap(X, {w_q8, size_t(vocab) * size_t(hidden / 32) * PTI_Q8_BLOCK_BYTES}) ||
        pti::overlap(X, {tokens, size_t(n_streams) * 4}))
        return PTI_ERR_OVERLAP;
    const dim3 grid((unsigned)((hidden + 255) / 256), (unsigned)n_streams);
    hipLaunchKernelGGL(embed_q8_kernel, grid, dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint8_t *>(w_q8), tokens, x, vocab, hidden);
    return launch_status();
}

extern "C" int pti_embed_ssq(const void *w_ssq, const int32_t *tokens, float *x, int64_t vocab, int64_t hidden,
                             void *stream)
{
    if (!w_ssq || !tokens || !x)
        return PTI_ERR_NULL;
    if (!pti::shape_ok(vocab, hidden))
        return PTI_ERR_SHAPE;
    if (!pti::aligned(tokens, 4) || !pti::aligned(x, 4))
        return PTI_ERR_ALIGN;
    const pti::Range X{x, size_t(2) * size_t(hidden) * 4};
    if (pti::overlap(X, {w_ssq, size_t(vocab) * size_t(hidden / 32) * PTI_SSQ_BLOCK_BYTES}) ||
        pti::overlap(X, {tokens, 8}))
        return PTI_ERR_OVERLAP;
    const dim3 grid((unsigned)((hidden + 255) / 256), 2u);
    hipLaunchKernelGGL(embed_ssq_kernel, grid, dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint8_t *>(w_ssq), tokens, x, vocab, hidden);
    return launch_status();
}

extern "C" int pti_rmsnorm(const float *x, float *y, int64_t dim, int n_streams, float eps, void *stream)
{
    if (!x || !y)
        return PTI_ERR_NULL;
    if (!elem_ok(dim) || !(eps >= 0.0f) || !std::isfinite(eps))
        return PTI_ERR_SHAPE;
    if (n_streams < 1 || n_streams > PTI_MAX_STREAMS)
        return PTI_ERR_NSTREAMS;
    if (!pti::aligned(x, 4) || !pti::aligned(y, 4))
        return PTI_ERR_ALIGN;
    const size_t bytes = size_t(n_streams) * size_t(dim) * 4;
    if (x != y && pti::overlap({x, bytes}, {y, bytes}))
        return PTI_ERR_OVERLAP;
    hipLaunchKernelGGL(rmsnorm_kernel, dim3((unsigned)n_streams), dim3(kNormThreads), 0,
                       static_cast<hipStream_t>(stream), x, y, dim, double(eps));
    return launch_status();
}

namespace {
// Elementwise ops allow y to be one of the inputs exactly, not a shifted overlap.
bool elementwise_overlap(const float *in, const float *y, size_t bytes)
{
    return in != y && pti::overlap({in, bytes}, {y, bytes});
}

unsigned elementwise_grid(int64_t n)
{
    const int64_t blocks = (n + 255) / 256;
    return (unsigned)(blocks < 4096 ? blocks : 4096);
}
}  // namespace

extern "C" int pti_silu_mul(const float *g, const float *u, float *y, int64_t n, void *stream)
{
    if (!g || !u || !y)
        return PTI_ERR_NULL;
    if (!elem_ok(n))
        return PTI_ERR_SHAPE;
    if (!pti::aligned(g, 4) || !pti::aligned(u, 4) || !pti::aligned(y, 4))
        return PTI_ERR_ALIGN;
    const size_t bytes = size_t(n) * 4;
    if (elementwise_overlap(g, y, bytes) || elementwise_overlap(u, y, bytes))
        return PTI_ERR_OVERLAP;
    hipLaunchKernelGGL(silu_mul_kernel, dim3(elementwise_grid(n)), dim3(256), 0, static_cast<hipStream_t>(stream), g,
                       u, y, n);
    return launch_status();
}

namespace pti {
int launch_silu_mul_rows(const float *gu, float *y, int64_t rows, int64_t cols, void *stream)
{
    hipLaunchKernelGGL(silu_mul_rows_kernel, dim3(elementwise_grid(rows * cols)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), gu, y, rows, cols);
    return launch_status();
}
}  // namespace pti

extern "C" int pti_add(const float *a, const float *b, float *y, int64_t n, void *stream)
{
    if (!a || !b || !y)
        return PTI_ERR_NULL;
    if (!elem_ok(n))
        return PTI_ERR_SHAPE;
    if (!pti::aligned(a, 4) || !pti::aligned(b, 4) || !pti::aligned(y, 4))
        return PTI_ERR_ALIGN;
    const size_t bytes = size_t(n) * 4;
    if (elementwise_overlap(a, y, bytes) || elementwise_overlap(b, y, bytes))
        return PTI_ERR_OVERLAP;
    hipLaunchKernelGGL(add_kernel, dim3(elementwise_grid(n)), dim3(256), 0, static_cast<hipStream_t>(stream), a, b, y,
                       n);
    return launch_status();
}

extern "C" int pti_sample_verify(const float *logits, const int32_t *tokens_in, const double *uniforms,
                                 double temperature, int32_t *tokens_out, int32_t *accept_out, int64_t vocab,
                                 int n_streams, void *stream)
{
    if (!logits || !tokens_in || !uniforms || !tokens_out || !accept_out)
        return PTI_ERR_NULL;
    if (vocab < 1 || vocab > PTI_MAX_VOCAB || !(temperature > 0.0) || !std::isfinite(temperature))
        return PTI_ERR_SHAPE;
    if (n_streams < 1 || n_streams > PTI_MAX_STREAMS)
        return PTI_ERR_NSTREAMS;
    if (!pti::aligned(logits, 4) || !pti::aligned(tokens_in, 4) || !pti::aligned(uniforms, 8) ||
        !pti::aligned(tokens_out, 4) || !pti::aligned(accept_out, 4))
        return PTI_ERR_ALIGN;
    const size_t ns = size_t(n_streams);
    const pti::Range L{logits, ns * size_t(vocab) * 4}, T{tokens_in, ns * 4}, U{uniforms, ns * 8},
        O{tokens_out, ns * 4}, C{accept_out, 4};
    for (const pti::Range &out : {O, C})
        if (pti::overlap(out, L) || pti::overlap(out, T) || pti::overlap(out, U))
            return PTI_ERR_OVERLAP;
    if (pti::overlap(O, C))
        return PTI_ERR_OVERLAP;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(sample_draw_kernel, dim3((unsigned)n_streams), dim3(kSampleThreads), 0, st, logits, uniforms,
                       temperature, tokens_out, vocab);
    hipLaunchKernelGGL(accept_kernel, dim3(1), dim3(64), 0, st, tokens_in, tokens_out, accept_out, n_streams);
    return launch_status();
}

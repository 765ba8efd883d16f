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
//   * rmsnorm: y = x / sqrt(mean(x^2) + eps), one workgroup per stream; x is
//     multiplied by the fp64 reciprocal of the root, so y is within one fp32
//     ulp of the formula (the GEMV that fuses the norm gives the same bits).
//   * silu_mul: y = g / (1 + exp(-g)) * u, elementwise.
//   * add: y = a + b in fp32, elementwise.
//   * sample_verify: per stream, weights w_j = exp((l_j - max) / t) in fp64 and
//     the smallest index whose running sum of weights exceeds u * sum(w); then
//     the accept count of the drawn tokens.
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cmath>

#include "pti_internal.h"
#include "pti_norm.h"
#include "pti_silu.h"

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

__device__ __forceinline__ float wave_max_f32(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

// ------------------------------------------------------------------ rmsnorm

constexpr int kNormThreads = pti_norm::kGroup;

__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(const float *__restrict__ x, float *__restrict__ y,
                                                               int64_t dim, double eps)
{
    __shared__ double part[kNormThreads / 64];
    __shared__ double root;  // 1 / the root
    const int tid = threadIdx.x;
    const float *xs = x + blockIdx.x * dim;
    float *ys = y + blockIdx.x * dim;
    double acc = 0.0;
    for (int64_t c = tid; c < dim; c += kNormThreads)
        acc = pti_norm::sq_acc(acc, xs[c]);
    acc = pti_norm::wave_sum_f64(acc);
    if ((tid & 63) == 0)
        part[tid >> 6] = acc;
    __syncthreads();
    if (tid == 0)
        root = pti_norm::inv_root(part, dim, eps);
    __syncthreads();
    const double r = root;
    for (int64_t c = tid; c < dim; c += kNormThreads)
        ys[c] = pti_norm::apply(xs[c], r);
}

// The same arithmetic in the same order for dim <= PER * kNormThreads, with
// the thread's elements read once, all loads in flight together, and kept in
// registers for the second pass (a loop with one dependent load per element
// pays the memory latency once per element).
template <int PER>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_reg_kernel(const float *__restrict__ x,
                                                                   float *__restrict__ y, int64_t dim, double eps)
{
    __shared__ double part[kNormThreads / 64];
    __shared__ double root;  // 1 / the root
    const int tid = threadIdx.x;
    const float *xs = x + blockIdx.x * dim;
    float *ys = y + blockIdx.x * dim;
    // buffer loads bounded by the row: past dim they read zeros, with no
    // branch, so all PER loads are in flight at once
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(xs), (short)0, (int)(dim * 4), 0x00020000);
    float v[PER];
#pragma unroll
    for (int i = 0; i < PER; i++)
        v[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (tid + i * kNormThreads) * 4, 0, 0));
    double acc = 0.0;
#pragma unroll
    for (int i = 0; i < PER; i++)
        if (tid + (int64_t)i * kNormThreads < dim)
            acc = pti_norm::sq_acc(acc, v[i]);
    acc = pti_norm::wave_sum_f64(acc);
    if ((tid & 63) == 0)
        part[tid >> 6] = acc;
    __syncthreads();
    if (tid == 0)
        root = pti_norm::inv_root(part, dim, eps);
    __syncthreads();
    const double r = root;
#pragma unroll
    for (int i = 0; i < PER; i++) {
        const int64_t c = tid + (int64_t)i * kNormThreads;
        if (c < dim)
            ys[c] = pti_norm::apply(v[i], r);
    }
}

// ------------------------------------------------------------------ elementwise

__global__ void silu_mul_kernel(const float *g, const float *u, float *y, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        y[i] = pti_silu::silu_mul(g[i], u[i]);
    }
}

// The same arithmetic on the rows of a stacked gate|up output: g = gu[s][j],
// u = gu[s][cols + j].  Row s = blockIdx.y.
__global__ void silu_mul_rows_kernel(const float *gu, float *y, int64_t cols)
{
    const int64_t s = blockIdx.y;
    const float *g = gu + s * 2 * cols, *u = g + cols;
    float *ys = y + s * cols;
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < cols; j += (int64_t)gridDim.x * blockDim.x) {
        ys[j] = pti_silu::silu_mul(g[j], u[j]);
    }
}

__global__ void add_kernel(const float *a, const float *b, float *y, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        y[i] = a[i] + b[i];
}

// ------------------------------------------------------------------ sampled verify

// A stream's vocabulary is cut into parts of kSvPart consecutive indices.
// Pass 1 (one workgroup per part and stream): the part's max m_b and
// S_b = sum_j exp((l_j - m_b) / T) in fp64.  Pass 2 (one workgroup per
// stream): M = max_b m_b; part weights W_b = S_b exp((m_b - M) / T); the
// running sum over parts in index order locates the part that holds u * Z
// (Z = sum_b W_b); inside it, the weights w_j = exp((l_j - m_b) / T)
// exp((m_b - M) / T) are summed in index order from the part's start to find
// the index.  Every sum runs in a fixed order that never decreases along the
// index: within a workgroup each thread owns a contiguous run and the runs
// are prefixed sequentially within a wave, then across waves.  The drawn index
// is the first of nonzero weight whose running sum exceeds u * Z; if rounding
// leaves none in the thread run that holds the target, the last index of
// nonzero weight in that run.  No positive weight (non-finite logits) draws -1.
constexpr int kSvPart = 2048;
constexpr int kSvThreads = 256;
constexpr int kSvWaves = kSvThreads / 64;
constexpr int kSvRun = kSvPart / kSvThreads;  // a thread's run of indices within a part

struct SvPart {
    double m, s;  // the part's max logit and its exp-sum relative to that max
};

__global__ __launch_bounds__(kSvThreads) void sv_part_kernel(const float *__restrict__ logits, double temperature,
                                                             SvPart *__restrict__ parts, int64_t vocab, int64_t nparts)
{
    __shared__ float wmax[kSvWaves];
    __shared__ double wsum[kSvWaves];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t b = blockIdx.x, s = blockIdx.y;
    const int64_t j0 = b * kSvPart;
    const int n = (int)min<int64_t>(kSvPart, vocab - j0);
    // the thread's kSvRun strided logits, all loads in flight at once
    // (buffer loads bounded by the part; entries past it are masked below)
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(logits + s * vocab + j0), (short)0, n * 4, 0x00020000);
    float x[kSvRun];
#pragma unroll
    for (int k = 0; k < kSvRun; k++)
        x[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (tid + k * kSvThreads) * 4, 0, 0));
    float m = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < kSvRun; k++)
        if (tid + k * kSvThreads < n)
            m = fmaxf(m, x[k]);
    m = wave_max_f32(m);
    if (lane == 0)
        wmax[wv] = m;
    __syncthreads();
    m = wmax[0];
    for (int i = 1; i < kSvWaves; i++)
        m = fmaxf(m, wmax[i]);
    const double md = m;
    double acc = 0.0;
    if (m > -__builtin_inff())
#pragma unroll
        for (int k = 0; k < kSvRun; k++)
            if (tid + k * kSvThreads < n)
                acc += exp((double(x[k]) - md) / temperature);
    acc = pti_norm::wave_sum_f64(acc);
    if (lane == 0)
        wsum[wv] = acc;
    __syncthreads();
    if (tid == 0) {
        double t = wsum[0];
        for (int i = 1; i < kSvWaves; i++)
            t += wsum[i];
        parts[s * nparts + b] = SvPart{md, t};
    }
}

// Index-monotone exclusive prefix of the threads' values `loc` (thread tid
// owns a contiguous run): sequential over the 64 lanes of a wave, then over
// the waves.  Returns this thread's exclusive prefix; *total gets the sum.
__device__ __forceinline__ double block_prefix(double loc, double *loc_s, double *pre_s, double *wbase, double *total)
{
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    loc_s[tid] = loc;
    __syncthreads();
    if (lane == 0) {
        // the wave's 64 values into registers, the sequential prefix there,
        // then back (LDS round trips pipelined instead of one per element)
        double v[64];
#pragma unroll
        for (int i = 0; i < 64; i += 2) {
            const double2 t = *reinterpret_cast<const double2 *>(&loc_s[tid + i]);
            v[i] = t.x, v[i + 1] = t.y;
        }
        double run = 0.0;
#pragma unroll
        for (int i = 0; i < 64; i++) {
            const double t = v[i];
            v[i] = run;
            run += t;
        }
#pragma unroll
        for (int i = 0; i < 64; i += 2)
            *reinterpret_cast<double2 *>(&pre_s[tid + i]) = make_double2(v[i], v[i + 1]);
        wbase[wv + 1] = run;
    }
    __syncthreads();
    if (tid == 0) {
        double run = 0.0;
        for (int w = 0; w < kSvWaves; w++) {
            const double t = wbase[w + 1];
            wbase[w] = run;
            run += t;
        }
        wbase[kSvWaves] = run;
    }
    __syncthreads();
    *total = wbase[kSvWaves];
    return wbase[wv] + pre_s[tid];
}

__global__ __launch_bounds__(kSvThreads) void sv_draw_kernel(const float *__restrict__ logits,
                                                             const double *__restrict__ uniforms, double temperature,
                                                             const SvPart *__restrict__ parts,
                                                             int32_t *__restrict__ tokens_out, int64_t vocab,
                                                             int64_t nparts)
{
    __shared__ __attribute__((aligned(16))) double loc_s[kSvThreads];
    __shared__ __attribute__((aligned(16))) double pre_s[kSvThreads];
    __shared__ double wbase[kSvWaves + 1];
    __shared__ float wmax[kSvWaves];
    __shared__ int owner;
    __shared__ int64_t own_part;
    __shared__ double own_excl;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t s = blockIdx.x;
    const SvPart *ps = parts + s * nparts;
    // M = max over the parts
    float M = -__builtin_inff();
    for (int64_t i = tid; i < nparts; i += kSvThreads)
        M = fmaxf(M, (float)ps[i].m);
    M = wave_max_f32(M);
    if (lane == 0)
        wmax[wv] = M;
    __syncthreads();
    M = wmax[0];
    for (int i = 1; i < kSvWaves; i++)
        M = fmaxf(M, wmax[i]);
    const double Md = M;
    auto factor = [&](double mb) { return mb > -__builtin_inff() ? exp((mb - Md) / temperature) : 0.0; };

    // parts: thread tid owns the contiguous run [p0, p1)
    const int64_t cp = (nparts + kSvThreads - 1) / kSvThreads;
    const int64_t p0 = min(nparts, tid * cp), p1 = min(nparts, p0 + cp);
    double loc = 0.0;
    for (int64_t p = p0; p < p1; p++)
        loc += ps[p].s * factor(ps[p].m);
    if (tid == 0)
        owner = -1;
    double Z;
    const double excl = block_prefix(loc, loc_s, pre_s, wbase, &Z);
    const double target = uniforms[s] * Z;
    if (loc > 0.0 && excl <= target)
        atomicMax(&owner, tid);
    __syncthreads();
    if (owner < 0) {  // no positive weight: non-finite logits
        if (tid == 0)
            tokens_out[s] = -1;
        return;
    }
    if (tid == owner) {
        double run = excl;
        int64_t pick = -1, last = -1;
        double pick_excl = 0.0, last_excl = 0.0;
        for (int64_t p = p0; p < p1; p++) {
            const double w = ps[p].s * factor(ps[p].m);
            if (w > 0.0) {
                last = p, last_excl = run;
                if (run + w > target) {
                    pick = p, pick_excl = run;
                    break;
                }
                run += w;
            }
        }
        own_part = pick >= 0 ? pick : last;
        own_excl = pick >= 0 ? pick_excl : last_excl;
    }
    __syncthreads();

    // inside the part: thread tid owns the contiguous run [q0, q1)
    const int64_t b = own_part;
    const int64_t j0 = b * kSvPart;
    const int n = (int)min<int64_t>(kSvPart, vocab - j0);
    const double mb = ps[b].m, fb = factor(mb);
    const int cq = (n + kSvThreads - 1) / kSvThreads;  // at most kSvRun
    const int q0 = min(n, tid * cq), q1 = min(n, q0 + cq);
    // the run's logits, all loads in flight at once (bounded by the part)
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(logits + s * vocab + j0), (short)0, n * 4, 0x00020000);
    float x[kSvRun];
#pragma unroll
    for (int k = 0; k < kSvRun; k++)
        x[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (q0 + k) * 4, 0, 0));
    double e[kSvRun];  // this thread's weights, kept for the owner's scan
    double loc2 = 0.0;
#pragma unroll
    for (int k = 0; k < kSvRun; k++) {
        e[k] = q0 + k < q1 ? exp((double(x[k]) - mb) / temperature) * fb : 0.0;
        loc2 += e[k];
    }
    if (tid == 0)
        owner = -1;
    double Zp;
    const double excl2 = own_excl + block_prefix(loc2, loc_s, pre_s, wbase, &Zp);
    if (loc2 > 0.0 && excl2 <= target)
        atomicMax(&owner, tid);
    __syncthreads();
    const int own2 = owner;
    if (own2 < 0) {  // cannot happen when the part's weight is positive; keep the part's first index
        if (tid == 0)
            tokens_out[s] = (int32_t)j0;
        return;
    }
    if (tid == own2) {
        double run = excl2;
        int pick = -1, last = -1;
#pragma unroll
        for (int k = 0; k < kSvRun; k++) {
            if (pick < 0 && e[k] > 0.0) {  // entries past q1 are 0
                last = q0 + k;
                run += e[k];
                if (run > target)
                    pick = q0 + k;
            }
        }
        tokens_out[s] = (int32_t)(j0 + (pick >= 0 ? pick : last));
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

// A pass's inputs written from kernel arguments: the tokens, and the
// uniforms when sampling (no host-to-device copy on the decode loop's path).
struct PassInputs {
    int32_t tok[PTI_MAX_STREAMS];
    double uni[PTI_MAX_STREAMS];
};

__global__ void set_inputs_kernel(PassInputs in, int32_t *tok, int n_tok, double *uni, int n_uni)
{
    const int i = threadIdx.x;
    if (i < n_tok)
        tok[i] = in.tok[i];
    if (uni && i < n_uni)
        uni[i] = in.uni[i];
}

int64_t sv_parts(int64_t vocab) { return (vocab + kSvPart - 1) / kSvPart; }

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
    const dim3 grid((unsigned)n_streams), block(kNormThreads);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (dim <= 8 * kNormThreads)
        hipLaunchKernelGGL(rmsnorm_reg_kernel<8>, grid, block, 0, st, x, y, dim, double(eps));
    else if (dim <= 32 * kNormThreads)
        hipLaunchKernelGGL(rmsnorm_reg_kernel<32>, grid, block, 0, st, x, y, dim, double(eps));
    else
        hipLaunchKernelGGL(rmsnorm_kernel, grid, block, 0, st, x, y, dim, double(eps));
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
    hipLaunchKernelGGL(silu_mul_rows_kernel, dim3(elementwise_grid(cols), (unsigned)rows), dim3(256), 0,
                       static_cast<hipStream_t>(stream), gu, y, cols);
    return launch_status();
}

int launch_set_inputs(int32_t *tok, const int32_t *tok_host, int n_tok, double *uni, const double *uni_host, int n_uni,
                      void *stream)
{
    PassInputs in{};
    for (int i = 0; i < n_tok; i++)
        in.tok[i] = tok_host[i];
    for (int i = 0; uni_host && i < n_uni; i++)
        in.uni[i] = uni_host[i];
    hipLaunchKernelGGL(set_inputs_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), in, tok, n_tok,
                       uni_host ? uni : nullptr, n_uni);
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

extern "C" size_t pti_sample_verify_workspace_bytes(int64_t vocab, int n_streams)
{
    if (vocab < 1 || vocab > PTI_MAX_VOCAB || n_streams < 1 || n_streams > PTI_MAX_STREAMS)
        return 0;
    return size_t(n_streams) * size_t(sv_parts(vocab)) * sizeof(SvPart);
}

namespace {

// Checks every argument of the sampled verify except the workspace, which
// each entry point checks its own way.
int sample_verify_args(const float *logits, const int32_t *tokens_in, const double *uniforms, double temperature,
                       const int32_t *tokens_out, const int32_t *accept_out, int64_t vocab, int n_streams)
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
    return PTI_OK;
}

// The three kernels of a sampled verify, with the part sums in `parts`.
int launch_sample_verify(const float *logits, const int32_t *tokens_in, const double *uniforms, double temperature,
                         int32_t *tokens_out, int32_t *accept_out, int64_t vocab, int n_streams, SvPart *parts,
                         void *stream)
{
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t np = sv_parts(vocab);
    hipLaunchKernelGGL(sv_part_kernel, dim3((unsigned)np, (unsigned)n_streams), dim3(kSvThreads), 0, st, logits,
                       temperature, parts, vocab, np);
    hipLaunchKernelGGL(sv_draw_kernel, dim3((unsigned)n_streams), dim3(kSvThreads), 0, st, logits, uniforms,
                       temperature, parts, tokens_out, vocab, np);
    hipLaunchKernelGGL(accept_kernel, dim3(1), dim3(64), 0, st, tokens_in, tokens_out, accept_out, n_streams);
    return launch_status();
}

// Scratch of the allocation-free sampled verify: the part sums, in device
// memory that the library owns.  Each GPU the library runs on holds its own
// copy until the process ends; host code reaches it only through the
// per-device address from hipGetSymbolAddress (the array's name is a host-side
// stand-in, not a device address).  Every call on a GPU shares that GPU's copy.
constexpr size_t kStaticScratchBytes = PTI_STATIC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch, looked up once per device
// (with that device current) and kept; nullptr with the HIP error recorded if
// the lookup fails.
void *scratch_ptr()
{
    int dev = 0;
    if (hipError_t e = hipGetDevice(&dev); e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        pti::set_hip_error(e != hipSuccess ? e : hipErrorInvalidDevice);
        return nullptr;
    }
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        // two threads racing both look it up and store the same address
        if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)); e != hipSuccess || !p) {
            pti::set_hip_error(e != hipSuccess ? e : hipErrorInvalidSymbol);
            return nullptr;
        }
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace

extern "C" int pti_sample_verify_static(const float *logits, const int32_t *tokens_in, const double *uniforms,
                                        double temperature, int32_t *tokens_out, int32_t *accept_out, int64_t vocab,
                                        int n_streams, void *stream)
{
    if (const int rc = sample_verify_args(logits, tokens_in, uniforms, temperature, tokens_out, accept_out, vocab,
                                          n_streams);
        rc != PTI_OK)
        return rc;
    if (pti_sample_verify_workspace_bytes(vocab, n_streams) > kStaticScratchBytes)
        return PTI_ERR_SHAPE;  // more part sums than the library's scratch holds
    void *p = scratch_ptr();
    if (!p)
        return PTI_ERR_HIP;
    return launch_sample_verify(logits, tokens_in, uniforms, temperature, tokens_out, accept_out, vocab, n_streams,
                                static_cast<SvPart *>(p), stream);
}

extern "C" int pti_sample_verify(const float *logits, const int32_t *tokens_in, const double *uniforms,
                                 double temperature, int32_t *tokens_out, int32_t *accept_out, int64_t vocab,
                                 int n_streams, void *work, size_t work_bytes, void *stream)
{
    if (!work)
        return PTI_ERR_NULL;
    if (const int rc = sample_verify_args(logits, tokens_in, uniforms, temperature, tokens_out, accept_out, vocab,
                                          n_streams);
        rc != PTI_OK)
        return rc;
    if (work_bytes < pti_sample_verify_workspace_bytes(vocab, n_streams))
        return PTI_ERR_SHAPE;
    if (!pti::aligned(work, 16))
        return PTI_ERR_ALIGN;
    const size_t ns = size_t(n_streams);
    const pti::Range L{logits, ns * size_t(vocab) * 4}, T{tokens_in, ns * 4}, U{uniforms, ns * 8},
        O{tokens_out, ns * 4}, C{accept_out, 4}, W{work, pti_sample_verify_workspace_bytes(vocab, n_streams)};
    if (pti::overlap(W, L) || pti::overlap(W, T) || pti::overlap(W, U) || pti::overlap(W, O) || pti::overlap(W, C))
        return PTI_ERR_OVERLAP;
    return launch_sample_verify(logits, tokens_in, uniforms, temperature, tokens_out, accept_out, vocab, n_streams,
                                static_cast<SvPart *>(work), stream);
}

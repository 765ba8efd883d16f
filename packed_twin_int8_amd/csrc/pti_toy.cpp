// Decoder-stack forward pass and the staggered multi-stream decode loop.
//
// [Digest = "Packed Twin Inference：无需草稿模型的推测解码新方案，实现2倍吞吐量提升",
// section "技术实现架构" (implementation architecture): a forward pass in which one
// weight load serves the confirmed and the speculative streams, a verify that
// compares their outputs, and state that grows on accept and is reset on
// reject; README = "打包双子推理（PTI）", section "接受机制如何工作" (how
// acceptance works): stream i runs i positions ahead on a guess the same model
// produced one step earlier.]
//
// Everything here is host code enqueuing the library's own kernels on one
// stream; the only synchronisation is the read-back of each pass's drawn
// tokens, which decide the next pass's inputs.  The caller owns every buffer:
// the workspace holds the activations of one pass,
//   h [N][hidden]  residual stream         r [N][hidden]  normalised input
//   g [N][ffn]     gate, then silu(g)*u    u [N][ffn]     up projection
//   d [N][hidden]  down projection         logits [N][vocab]
//   tokens, drawn tokens, accept count (int32), uniforms (fp64)
// each region 256-byte aligned (the GEMVs read activations with 16-byte loads).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>

#include "pti_internal.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

struct Layout {
    size_t h, r, gu, x, logits, tok, uni, sv, keys, total;
};

// Workgroups of the LM head whose greedy-verify keys the workspace holds (a
// head launch over more takes the separate verify).
constexpr int64_t kMaxKeyGroups = 1024;

Layout layout(const pti_toy_model &m, int n)
{
    Layout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes);
        return o;
    };
    const size_t N = size_t(n);
    L.h = take(N * size_t(m.hidden) * 4);
    L.r = take(N * size_t(m.hidden) * 4);
    L.gu = take(N * 2 * size_t(m.ffn) * 4);  // stacked gate|up outputs, [N][2F]
    L.x = take(N * size_t(m.ffn) * 4);
    L.logits = take(N * size_t(m.vocab) * 4);
    L.tok = take(PTI_MAX_STREAMS * 4);
    L.uni = take(PTI_MAX_STREAMS * 8);
    L.sv = take(pti_sample_verify_workspace_bytes(m.vocab, n));  // the sampled verify's part sums
    L.keys = take(size_t(kMaxKeyGroups) * pti::kVerifyKeyStride * 8);  // the head's greedy-verify keys
    L.total = off;
    return L;
}

bool weights_ok(const void *p) { return p != nullptr && pti::aligned(p, 4); }

int check_model(const pti_toy_model *m)
{
    if (!m || !m->embed || !m->head || !m->gate || !m->up || !m->down)
        return PTI_ERR_NULL;
    if (m->format != PTI_FMT_Q8 && m->format != PTI_FMT_SSQ)
        return PTI_ERR_SHAPE;
    if (m->n_layers < 1 || m->n_layers > PTI_TOY_MAX_LAYERS)
        return PTI_ERR_SHAPE;
    if (!pti::shape_ok(m->vocab, m->hidden) || !pti::shape_ok(m->ffn, m->hidden) ||
        !pti::shape_ok(m->hidden, m->ffn))
        return PTI_ERR_SHAPE;
    if (!(m->eps >= 0.0f) || !std::isfinite(m->eps))
        return PTI_ERR_SHAPE;
    for (int l = 0; l < m->n_layers; l++)
        if (!m->gate[l] || !m->up[l] || !m->down[l])
            return PTI_ERR_NULL;
    if (!weights_ok(m->embed) || !weights_ok(m->head))
        return PTI_ERR_ALIGN;
    for (int l = 0; l < m->n_layers; l++)
        if (!weights_ok(m->gate[l]) || !weights_ok(m->up[l]) || !weights_ok(m->down[l]))
            return PTI_ERR_ALIGN;
    return PTI_OK;
}

int check_streams(const pti_toy_model *m, int n)
{
    if (m->format == PTI_FMT_SSQ)
        return n == 2 ? PTI_OK : PTI_ERR_NSTREAMS;
    return (n >= 1 && n <= PTI_MAX_STREAMS) ? PTI_OK : PTI_ERR_NSTREAMS;
}

#define PTI_TRY(call)            \
    do {                         \
        const int st_ = (call);  \
        if (st_ != PTI_OK)       \
            return st_;          \
    } while (0)

// y [N][rows] = W x for x [N][cols]; the SSQ form runs twin A on x[0], twin B on x[1].
int gemv(const pti_toy_model &m, const void *w, const float *x, float *y, int64_t rows, int64_t cols, int n,
         void *stream)
{
    if (m.format == PTI_FMT_SSQ)
        return pti_gemv_ssq(w, x, x + cols, y, y + rows, rows, cols, stream);
    return pti_gemv_q8_multi(w, x, y, rows, cols, n, stream);
}

// Enqueues one pass; logits may point into the workspace or outside it.
// Per layer: rmsnorm; gate and up in one grouped launch (outputs stacked per
// stream); silu(gate) * up; down with the residual added as the rows are
// stored.  In Q8 the first three are one launch where the gate|up GEMV takes
// the per-wave-row kernel.  Each step's results are bitwise those of the
// separate calls (rmsnorm, gate, up, silu_mul, down, add).
//
// keyed (optional): ask the Q8 head for greedy-verify keys in the workspace;
// *keyed is set to whether it wrote them (the head took the per-wave-row
// kernel with the norm fused and its workgroups fit the key region).
int forward(const pti_toy_model &m, const Layout &L, char *work, const int32_t *tokens, float *logits, int n,
            void *stream, bool *keyed = nullptr)
{
    if (keyed)
        *keyed = false;
    float *h = reinterpret_cast<float *>(work + L.h), *r = reinterpret_cast<float *>(work + L.r);
    float *gu = reinterpret_cast<float *>(work + L.gu), *x = reinterpret_cast<float *>(work + L.x);
    const int64_t H = m.hidden, F = m.ffn;
    const bool ssq = m.format == PTI_FMT_SSQ;
    if (ssq)
        PTI_TRY(pti_embed_ssq(m.embed, tokens, h, m.vocab, H, stream));
    else
        PTI_TRY(pti_embed_q8(m.embed, tokens, h, m.vocab, H, n, stream));
    const int64_t rows2[2] = {F, F};
    for (int l = 0; l < m.n_layers; l++) {
        const void *gate_up[2] = {m.gate[l], m.up[l]};
        // Q8, where the gate|up GEMV takes the per-wave-row kernel: the norm
        // inside its staging and silu(gate) * up applied to its row pairs,
        // one launch (same bits as the separate norm, GEMV and activation)
        const int fused = ssq ? pti::kNormNotFused
                              : pti::q8_gate_up_silu(m.gate[l], m.up[l], F, h, x, H, n, m.eps, stream);
        if (fused != pti::kNormNotFused) {
            PTI_TRY(fused);
        } else {
            PTI_TRY(pti_rmsnorm(h, r, H, n, m.eps, stream));
            if (ssq)
                PTI_TRY(pti_gemv_ssq_grouped(gate_up, rows2, 2, r, r + H, gu, gu + 2 * F, H, stream));
            else
                PTI_TRY(pti_gemv_q8_multi_grouped(gate_up, rows2, 2, r, gu, H, n, stream));
            PTI_TRY(pti::launch_silu_mul_rows(gu, x, n, F, stream));
        }
        if (ssq)
            PTI_TRY(pti::gemv_ssq_res(m.down[l], x, x + F, h, h + H, h, h + H, H, F, stream));
        else
            PTI_TRY(pti::gemv_q8_res(m.down[l], x, h, h, H, F, n, stream));
    }
    if (!ssq) {
        const void *head[1] = {m.head};
        const int64_t vrows[1] = {m.vocab};
        const int64_t groups = pti::rowwise_groups(m.vocab);
        unsigned long long *keys = keyed && groups > 0 && groups <= kMaxKeyGroups
                                       ? reinterpret_cast<unsigned long long *>(work + L.keys)
                                       : nullptr;
        const int fused = pti::q8_gemv_rmsnorm(head, vrows, 1, h, logits, H, n, m.eps, stream, keys);
        if (fused != pti::kNormNotFused) {
            if (keyed)
                *keyed = fused == PTI_OK && keys != nullptr;
            return fused;
        }
    }
    PTI_TRY(pti_rmsnorm(h, r, H, n, m.eps, stream));
    return gemv(m, m.head, r, logits, m.vocab, H, n, stream);
}

int hip_status(hipError_t e)
{
    if (e != hipSuccess) {
        pti::set_hip_error(e);
        return PTI_ERR_HIP;
    }
    return PTI_OK;
}

// The decode loop's state and its passes.
struct Decoder {
    const pti_toy_model &m;
    Layout L;
    char *work;
    int N;                   // streams of a step
    int npass;               // streams of a multi-stream pass's forward (N; 2 for SSQ)
    double temp;
    const double *uniforms;  // host
    int32_t *log;            // host, 5 ints per draw, or null
    int64_t nlog = 0;
    hipStream_t st;
    // pinned host memory the verify kernels write the draws (ints
    // 0 .. PTI_MAX_STREAMS - 1) and the accept count (int PTI_MAX_STREAMS)
    // into, so that a pass's results reach the host without a copy command
    volatile int32_t *back = nullptr;

    int32_t *dev_tok() const { return reinterpret_cast<int32_t *>(work + L.tok); }
    double *dev_uni() const { return reinterpret_cast<double *>(work + L.uni); }
    float *dev_logits() const { return reinterpret_cast<float *>(work + L.logits); }

    void record(int step, int slot, int stream, int32_t in, int32_t out)
    {
        if (log) {
            int32_t *e = log + 5 * nlog;
            e[0] = step, e[1] = slot, e[2] = stream, e[3] = in, e[4] = out;
        }
        nlog++;
    }

    // Draws n tokens from logits rows [row0, row0 + n) with the uniforms of
    // slots slot0 ...; the accept count compares them with the pass inputs
    // already in dev_tok() (read only when n >= 2, i.e. for row0 == 0).
    // The pass's inputs: tokens x[0..nx-1] and, when sampling, the uniforms of
    // the n draws of slots slot0 ..., written by one small kernel.
    int set_inputs(const int32_t *x, int nx, int step, int slot0, int n)
    {
        const double *u = temp == 0.0 ? nullptr : uniforms + (size_t(step) * 2 * N + size_t(slot0));
        return pti::launch_set_inputs(dev_tok(), x, nx, dev_uni(), u, n, st);
    }

    // Draws n tokens from logits rows [row0, row0 + n) with the uniforms set
    // for the pass; the accept count compares them with the pass inputs in
    // dev_tok() (read only when n >= 2, i.e. for row0 == 0).  The draws and
    // the accept count arrive in the readback page when the stream is synchronised.
    // keyed: the pass's head left greedy-verify keys (row0 is then 0), which
    // one wave reduces instead of a pass over the logits.
    int draw(int row0, int n, int32_t *out, int32_t *accept, bool keyed)
    {
        void *s = st;
        const float *lg = dev_logits() + int64_t(row0) * m.vocab;
        int32_t *o = const_cast<int32_t *>(back), *a = o + PTI_MAX_STREAMS;
        if (temp == 0.0 && keyed)
            PTI_TRY(pti::launch_verify_keys_n(reinterpret_cast<const unsigned long long *>(work + L.keys),
                                              (int)pti::rowwise_groups(m.vocab), n, dev_tok(), o, a, s));
        else if (temp == 0.0)
            PTI_TRY(pti_verify_argmax(lg, dev_tok(), o, a, m.vocab, n, s));
        else
            PTI_TRY(pti_sample_verify(lg, dev_tok(), dev_uni(), temp, o, a, m.vocab, n, work + L.sv,
                                      pti_sample_verify_workspace_bytes(m.vocab, n), s));
        PTI_TRY(hip_status(hipStreamSynchronize(st)));
        for (int i = 0; i < n; i++)
            out[i] = back[i];
        *accept = back[PTI_MAX_STREAMS];
        return PTI_OK;
    }

    // One pass of every stream on inputs x[0..N-1]: outputs o[], accept count.
    int multi(int step, const int32_t *x, int32_t *o, int32_t *a)
    {
        PTI_TRY(set_inputs(x, N, step, 0, N));
        bool keyed = false;
        PTI_TRY(forward(m, L, work, dev_tok(), dev_logits(), npass, st, temp == 0.0 ? &keyed : nullptr));
        PTI_TRY(draw(0, N, o, a, keyed));
        for (int s = 0; s < N; s++)
            record(step, s, s, x[s], o[s]);
        return PTI_OK;
    }

    // Single-stream pass of `stream` on token t in pass slot `slot`.  In the
    // SSQ format both twins run on t and twin B's logits are drawn from
    // (single-stream passes are always of a stream >= 1, the drafter).
    int single(int step, int slot, int stream, int32_t t, int32_t *o)
    {
        const int32_t in[2] = {t, t};
        const int n = m.format == PTI_FMT_SSQ ? 2 : 1;
        int32_t a;
        PTI_TRY(set_inputs(in, n, step, slot, 1));
        bool keyed = false;
        PTI_TRY(forward(m, L, work, dev_tok(), dev_logits(), n, st, temp == 0.0 ? &keyed : nullptr));
        const int row = (m.format == PTI_FMT_SSQ && stream >= 1) ? 1 : 0;
        PTI_TRY(draw(row, 1, o, &a, keyed && row == 0));
        record(step, slot, stream, t, *o);
        return PTI_OK;
    }
};

// The readback page of the calling thread: pinned, coherent host memory that
// kernels write into directly (one page per thread that decodes, allocated at
// its first call and kept until the process ends, so that calls on
// different threads never share it and nothing is freed while a kernel may
// still write to it).
int readback_page(volatile int32_t **out)
{
    static thread_local void *page = nullptr;
    if (!page) {
        void *p = nullptr;
        PTI_TRY(hip_status(hipHostMalloc(&p, 4096, hipHostMallocCoherent)));
        page = p;
    }
    *out = static_cast<volatile int32_t *>(page);
    return PTI_OK;
}

int check_work(const Layout &L, const void *work, size_t work_bytes)
{
    if (!work)
        return PTI_ERR_NULL;
    if (!pti::aligned(work, kAlign))
        return PTI_ERR_ALIGN;
    if (work_bytes < L.total)
        return PTI_ERR_SHAPE;
    return PTI_OK;
}

}  // namespace

extern "C" size_t pti_toy_workspace_bytes(const pti_toy_model *m, int n_streams)
{
    if (check_model(m) != PTI_OK || check_streams(m, n_streams) != PTI_OK)
        return 0;
    return layout(*m, n_streams).total;
}

extern "C" int pti_toy_forward(const pti_toy_model *m, const int32_t *tokens, float *logits, void *work,
                               size_t work_bytes, int n_streams, void *stream)
{
    PTI_TRY(check_model(m));
    PTI_TRY(check_streams(m, n_streams));
    if (!tokens || !logits)
        return PTI_ERR_NULL;
    if (!pti::aligned(tokens, 4) || !pti::aligned(logits, 4))
        return PTI_ERR_ALIGN;
    const Layout L = layout(*m, n_streams);
    PTI_TRY(check_work(L, work, work_bytes));
    const pti::Range W{work, L.total}, T{tokens, size_t(n_streams) * 4},
        O{logits, size_t(n_streams) * size_t(m->vocab) * 4};
    if (pti::overlap(W, T) || pti::overlap(W, O) || pti::overlap(T, O))
        return PTI_ERR_OVERLAP;
    return forward(*m, L, static_cast<char *>(work), tokens, logits, n_streams, stream);
}

extern "C" int pti_toy_forward_graph(const pti_toy_model *m, const int32_t *tokens, float *logits, void *work,
                                     size_t work_bytes, int n_streams, void **graph_out)
{
    if (!graph_out)
        return PTI_ERR_NULL;
    *graph_out = nullptr;
    PTI_TRY(check_model(m));
    PTI_TRY(check_streams(m, n_streams));
    if (!tokens || !logits)
        return PTI_ERR_NULL;
    if (!pti::aligned(tokens, 4) || !pti::aligned(logits, 4))
        return PTI_ERR_ALIGN;
    const Layout L = layout(*m, n_streams);
    PTI_TRY(check_work(L, work, work_bytes));
    const pti::Range W{work, L.total}, T{tokens, size_t(n_streams) * 4},
        O{logits, size_t(n_streams) * size_t(m->vocab) * 4};
    if (pti::overlap(W, T) || pti::overlap(W, O) || pti::overlap(T, O))
        return PTI_ERR_OVERLAP;
    // Capture one pass on a private stream (default priority); the graph
    // keeps the kernels and their arguments, so replays read tokens and write
    // logits and work at these addresses.
    hipStream_t cs = nullptr;
    PTI_TRY(hip_status(hipStreamCreateWithFlags(&cs, hipStreamNonBlocking)));
    hipGraph_t g = nullptr;
    int rc = hip_status(hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal));
    if (rc == PTI_OK) {
        const int frc = forward(*m, L, static_cast<char *>(work), tokens, logits, n_streams, cs);
        const int erc = hip_status(hipStreamEndCapture(cs, &g));  // always ends the capture
        rc = frc != PTI_OK ? frc : erc;
    }
    hipGraphExec_t exec = nullptr;
    if (rc == PTI_OK)
        rc = hip_status(hipGraphInstantiate(&exec, g, nullptr, nullptr, 0));
    if (g)
        (void)hipGraphDestroy(g);
    (void)hipStreamDestroy(cs);
    if (rc == PTI_OK)
        *graph_out = exec;
    return rc;
}

extern "C" int pti_graph_launch(void *graph, void *stream)
{
    if (!graph)
        return PTI_ERR_NULL;
    return hip_status(hipGraphLaunch(static_cast<hipGraphExec_t>(graph), static_cast<hipStream_t>(stream)));
}

extern "C" int pti_graph_destroy(void *graph)
{
    if (!graph)
        return PTI_OK;
    return hip_status(hipGraphExecDestroy(static_cast<hipGraphExec_t>(graph)));
}

extern "C" int pti_toy_decode(const pti_toy_model *m, int32_t first_token, int n_streams, int n_steps,
                              double temperature, const double *uniforms, void *work, size_t work_bytes,
                              int32_t *committed, int32_t *accepts, int32_t *passes, int64_t *n_passes, void *stream)
{
    PTI_TRY(check_model(m));
    PTI_TRY(check_streams(m, n_streams));
    if (n_steps < 0 || first_token < 0 || first_token >= m->vocab)
        return PTI_ERR_SHAPE;
    if (!(temperature >= 0.0) || !std::isfinite(temperature))
        return PTI_ERR_SHAPE;
    if ((n_steps > 0 && (!committed || !accepts)) || (temperature > 0.0 && !uniforms))
        return PTI_ERR_NULL;
    const Layout L = layout(*m, n_streams);
    PTI_TRY(check_work(L, work, work_bytes));

    const int N = n_streams;
    Decoder D{*m, L, static_cast<char *>(work), N, m->format == PTI_FMT_SSQ ? 2 : N, temperature, uniforms, passes,
              0, static_cast<hipStream_t>(stream)};
    PTI_TRY(readback_page(&D.back));
    int32_t x[PTI_MAX_STREAMS], o[PTI_MAX_STREAMS], nxt[PTI_MAX_STREAMS];
    x[0] = first_token;
    for (int i = 1; i < N; i++)
        PTI_TRY(D.single(0, N + i - 1, i, x[i - 1], &x[i]));
    for (int k = 1; k <= n_steps; k++) {
        int32_t a = 0;
        PTI_TRY(D.multi(k, x, o, &a));
        if (a < 1 || a > N)
            return PTI_ERR_HIP;  // cannot happen with a working device; guards the indexing below
        committed[k - 1] = o[0];
        accepts[k - 1] = a;
        std::memcpy(nxt, o, sizeof(int32_t) * size_t(N));
        int32_t prev = o[a - 1];
        for (int j = a; j < N; j++) {
            PTI_TRY(D.single(k, N + j - a, j, prev, &prev));
            nxt[j] = prev;
        }
        std::memcpy(x, nxt, sizeof(int32_t) * size_t(N));
    }
    if (n_passes)
        *n_passes = D.nlog;
    return PTI_OK;
}

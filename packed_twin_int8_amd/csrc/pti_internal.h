// Internal declarations shared by the library's translation units.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "pti.h"

namespace pti {

// Records a HIP error code for pti_last_hip_error() on this thread.
void set_hip_error(int err);

inline bool shape_ok(int64_t rows, int64_t cols)
{
    return rows >= 1 && rows <= PTI_MAX_ROWS && cols >= PTI_BLOCK && cols <= PTI_MAX_COLS &&
           cols % PTI_BLOCK == 0;
}

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Half-open byte range [p, p + n).
struct Range {
    const void *p;
    size_t n;
};

// The rows of up to PTI_MAX_STREAMS streams (one pointer each).
struct StreamRows {
    const float *p[PTI_MAX_STREAMS];
};

// Greedy verify over streams whose logits need not be contiguous; arguments
// already validated by the caller.  Enqueues on `stream`.
int launch_verify_rows(const StreamRows &lg, const int32_t *tokens_in, int32_t *argmax_out, int32_t *accept_out,
                       int64_t vocab, int n_streams, void *stream);

// GEMVs whose outputs add a residual: y[s][r] = res[s][r] + (W x_s)[r], the
// same fp32 addition pti_add makes; res may be y itself (each element is read
// before it is written, by the same thread).  Arguments already validated.
int gemv_q8_res(const void *w, const float *x, float *y, const float *res, int64_t rows, int64_t cols, int n,
                void *stream);
int gemv_ssq_res(const void *w, const float *x_a, const float *x_b, float *y_a, float *y_b, const float *res_a,
                 const float *res_b, int64_t rows, int64_t cols, void *stream);

// y[s] = W rmsnorm(x[s]) for the Q8 matrices w[0..n_mats) stacked into one
// row space (as pti_gemv_q8_multi_grouped stacks them), s < n: the
// per-wave-row GEMV normalises x while staging it, with the bits pti_rmsnorm
// gives.  Returns kNormNotFused, launching nothing, when the shape takes the
// row-split kernel at every stream count or x does not fit in LDS at once (the
// caller then runs pti_rmsnorm and the plain GEMV).  Arguments already validated, except that
// the matrices are checked as a grouped launch checks them.
constexpr int kNormNotFused = 1;
// keys (optional): the launch also writes, per workgroup, the largest greedy
// verify key of each stream (kVerifyKeyStride per workgroup, stream s at s;
// rowwise_groups(sum of rows) workgroups), for launch_verify_keys_n.
constexpr int kVerifyKeyStride = 4;
int q8_gemv_rmsnorm(const void *const *w, const int64_t *rows, int n_mats, const float *x, float *y, int64_t cols,
                    int n, float eps, void *stream, unsigned long long *keys = nullptr);

// Workgroups of a per-wave-row launch over `rows` rows (0 if the device
// cannot be queried).
int64_t rowwise_groups(int64_t rows);

// argmax_out[s] (s < n) and accept_out[0] from the keys of a q8_gemv_rmsnorm
// launch, the results pti_verify_argmax gives on that launch's outputs.
int launch_verify_keys_n(const unsigned long long *keys, int n_groups, int n, const int32_t *tokens_in,
                         int32_t *argmax_out, int32_t *accept_out, void *stream);

// y[s][j] = silu(g[s][j]) * u[s][j], j < ffn, s < n, for g = G rmsnorm(x[s])
// and u = U rmsnorm(x[s]) (Q8 matrices gate and up of ffn rows each, cols
// columns): one launch of the per-wave-row GEMV in which each wave takes row
// j of both matrices and applies the activation to the pair, so g and u are
// never stored.  Each of g, u has the bits q8_gemv_rmsnorm gives for the
// stacked gate|up, and y those of launch_silu_mul_rows on that output.
// Returns kNormNotFused, launching nothing, where q8_gemv_rmsnorm would.
int q8_gate_up_silu(const void *gate, const void *up, int64_t ffn, const float *x, float *y, int64_t cols, int n,
                    float eps, void *stream);

// y[s][j] = silu(gu[s][j]) * gu[s][cols + j] for s < rows, j < cols (rows of
// 2 cols: the stacked output of a grouped gate|up GEMV), as pti_silu_mul
// computes it.  Arguments already validated.
int launch_silu_mul_rows(const float *gu, float *y, int64_t rows, int64_t cols, void *stream);

// tok[i] = tok_host[i] (i < n_tok) and, when uni_host is set, uni[i] =
// uni_host[i] (i < n_uni), written on the device from kernel arguments (one
// launch, no host-to-device copy).  n_tok, n_uni <= PTI_MAX_STREAMS.
int launch_set_inputs(int32_t *tok, const int32_t *tok_host, int n_tok, double *uni, const double *uni_host, int n_uni,
                      void *stream);

inline bool overlap(Range a, Range b)
{
    if (a.n == 0 || b.n == 0)
        return false;
    uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.n && b0 < a0 + a.n;
}

}  // namespace pti

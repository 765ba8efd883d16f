/*
 * pti.h -- C ABI of libpti.so: the packed-twin (PTI) decode hot path on
 * AMD Instinct MI355X (gfx950).
 *
 * Pages cited (by title and section):
 *   [Digest]  "Packed Twin Inference：无需草稿模型的推测解码新方案，实现2倍吞吐量提升"
 *             (zingnex.cn forum digest of the packed-twin-inference project)
 *   [README]  "打包双子推理（PTI）" (bittide.aicompass.dev; the project README in
 *             Chinese translation)
 *
 * The operations: a matrix-vector product (GEMV) over int8 weights that are
 * read from memory once per call and shared by several token streams.
 *   - SSQ ("side-by-side quantization") packs the int8 weights of two models,
 *     the twins A and B, into one uint16 per position, A in the high byte and
 *     B in the low byte, in 68-byte blocks [scale_A f16][scale_B f16][32 x uint16]
 *     [Digest, section "PTI的核心创新：SSQ打包技术" (SSQ packing)].  One load of a
 *     slot feeds both twins' accumulations
 *     [README, section "与 SSQ（Side-by-Side Quantization）的关系" (relation to SSQ)].
 *   - Q8 stores one model as 34-byte blocks [scale f16][32 x int8] (two of them
 *     have the size of one SSQ block [Digest, SSQ packing]); one read of a block
 *     is shared by n_streams activation vectors [README, section
 *     "带宽分析：为什么会有开销" (bandwidth analysis), the multi-stream kernel
 *     that reads four activation vectors per weight load].
 *   - Verify takes each stream's greedy token and counts how many streams'
 *     speculative inputs are confirmed [README, section "接受机制如何工作" (how
 *     acceptance works); Digest, section "技术实现架构" (implementation
 *     architecture), the verify step].
 *
 * Conventions shared by every call
 *   - Return value: PTI_OK (0) or a negative PTI_ERR_* code.  Nothing aborts,
 *     throws or exits.  Arguments are validated before anything is written or
 *     launched; on a validation error nothing is written.
 *   - Matrices are row-major, little-endian, with no header or padding: row r
 *     holds cols/32 consecutive blocks, block b covering columns 32b..32b+31.
 *     A weight's value is scale * int8 (symmetric, no zero point).
 *   - Ownership: the caller owns every buffer.  The library makes no device
 *     allocation calls; its only device memory of its own is the 64 KB
 *     file-scope array of pti_sample_verify_static (one per GPU, from load
 *     time).  Its only host allocation is pti_toy_decode's readback page
 *     (4 KB of pinned host memory per calling thread, see there).  Its other
 *     state: a thread-local copy of the last HIP error, a thread-local cache
 *     of the current device's CU count, per-kernel flags of the devices whose
 *     launch attributes are set, and that array's address per device.  It
 *     may be called from several threads.
 *   - Device calls take device pointers and a HIP stream (a hipStream_t passed
 *     as void*, NULL = the default stream).  They enqueue work and return
 *     without synchronising; outputs are overwritten, never accumulated into.
 *     A HIP launch failure returns PTI_ERR_HIP (see pti_last_hip_error).
 *   - Device calls need: w 4-byte aligned, activations 16-byte aligned, every
 *     other device pointer 4-byte aligned; outputs must not overlap any input
 *     or each other.  Inputs may alias each other (e.g. x_a == x_b).
 *   - Sizes: 1 <= rows <= PTI_MAX_ROWS, 32 <= cols <= PTI_MAX_COLS,
 *     cols % 32 == 0, 1 <= vocab <= PTI_MAX_VOCAB.
 *   - Numerics: fp32 accumulation.  For every output, the error against the
 *     exact result is below 1e-5 * sum_c |scale * q_c * x_c| for finite inputs.
 *     The result of one stream depends only on that stream's inputs, on
 *     (rows, cols) and on the format: it is bitwise the same whatever
 *     n_streams, the stream's slot or the call, so A == B twins fed equal
 *     activations give bitwise equal outputs.  An SSQ twin and a Q8 GEMV of the
 *     same model's weights agree within the bound above (their lanes group the
 *     columns differently).  Non-finite scales or activations give unspecified
 *     (non-finite or finite) outputs for the affected rows.
 */
#ifndef PTI_H
#define PTI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PTI_BLOCK 32            /* weights per scale block, both formats */
#define PTI_SSQ_BLOCK_BYTES 68  /* [scale_A f16][scale_B f16][32 x uint16] */
#define PTI_Q8_BLOCK_BYTES 34   /* [scale f16][32 x int8] */
#define PTI_MAX_STREAMS 4
#define PTI_MAX_GROUP 4         /* matrices per grouped GEMV launch */
#define PTI_MAX_ROWS 2147483647LL
#define PTI_MAX_COLS (1LL << 24)
#define PTI_MAX_VOCAB 2147483647LL
#define PTI_MAX_ELEMS (1LL << 40)  /* element count limit of the elementwise and norm calls */
#define PTI_SSQ_VERIFY_WORK_BYTES 16384  /* workspace of pti_gemv_ssq_verify */
#define PTI_MAX_ATTN_LEN (1LL << 24)      /* KV cache positions per stream */

enum pti_status {
    PTI_OK = 0,
    PTI_ERR_NULL = -1,     /* a required pointer is NULL */
    PTI_ERR_SHAPE = -2,    /* rows/cols/vocab outside the limits above, or cols % 32 != 0 */
    PTI_ERR_NSTREAMS = -3, /* n_streams outside [1, PTI_MAX_STREAMS] */
    PTI_ERR_ALIGN = -4,    /* a device pointer is not aligned as required */
    PTI_ERR_HIP = -5,      /* the HIP runtime reported an error; see pti_last_hip_error() */
    PTI_ERR_OVERLAP = -6   /* an output range overlaps an input range or another output */
};

/* Static text for a status code ("unknown status" for other values). */
const char *pti_status_str(int status);

/* hipError_t value of the last PTI_ERR_HIP returned on the calling thread
 * (0 if none). */
int pti_last_hip_error(void);

/* ABI version of this header: 1. */
int pti_abi_version(void);

/* ------------------------------------------------------------------------- */
/* Host-side packing [Digest, SSQ packing; Digest, implementation architecture:
 * the packing, unpacking and format-conversion tools].  CPU, synchronous; all
 * buffers are caller-owned host memory.  Bit-preserving for every int8 value
 * (including -128) and every f16 bit pattern.                              */

/* Bytes of a packed rows x cols matrix: rows*(cols/32)*68 (SSQ) or
 * rows*(cols/32)*34 (Q8); 0 if the shape is invalid. */
size_t pti_ssq_bytes(int64_t rows, int64_t cols);
size_t pti_q8_bytes(int64_t rows, int64_t cols);

/* a, b: int8 [rows][cols] (twin A, twin B); scale_a, scale_b: f16 bit patterns
 * [rows][cols/32]; out: pti_ssq_bytes(rows, cols) bytes.  Block (r, k) is at
 * byte (r*cols/32 + k)*68: bytes 0..1 scale_a, 2..3 scale_b, then slot j
 * (= A_j << 8 | B_j as uint16) at bytes 4+2j (B_j) and 5+2j (A_j). */
int pti_pack_ssq(const int8_t *a, const int8_t *b, const uint16_t *scale_a, const uint16_t *scale_b,
                 int64_t rows, int64_t cols, uint8_t *out);
/* Inverse of pti_pack_ssq. */
int pti_unpack_ssq(const uint8_t *in, int64_t rows, int64_t cols, int8_t *a, int8_t *b,
                   uint16_t *scale_a, uint16_t *scale_b);

/* q: int8 [rows][cols]; scale: f16 bits [rows][cols/32]; out: pti_q8_bytes bytes.
 * Block (r, k) at byte (r*cols/32 + k)*34: bytes 0..1 scale, bytes 2+j q_j. */
int pti_pack_q8(const int8_t *q, const uint16_t *scale, int64_t rows, int64_t cols, uint8_t *out);
/* Inverse of pti_pack_q8. */
int pti_unpack_q8(const uint8_t *in, int64_t rows, int64_t cols, int8_t *q, uint16_t *scale);

/* Split an SSQ matrix into the two twins' Q8 matrices ([scale_a][A x 32] and
 * [scale_b][B x 32] per block); join is the exact inverse.  q8_a, q8_b:
 * pti_q8_bytes each; ssq: pti_ssq_bytes.  Inputs and outputs must not overlap. */
int pti_ssq_split(const uint8_t *ssq, int64_t rows, int64_t cols, uint8_t *q8_a, uint8_t *q8_b);
int pti_ssq_join(const uint8_t *q8_a, const uint8_t *q8_b, int64_t rows, int64_t cols, uint8_t *ssq);

/* ------------------------------------------------------------------------- */
/* Device calls                                                              */

/* SSQ twin GEMV [README, relation to SSQ: one slot load, unpack high and low
 * byte, accumulate scale_A*A*x_A and scale_B*B*x_B]:
 *   y_a[r] = sum_c scale_A(r, c/32) * A[r][c] * x_a[c]
 *   y_b[r] = sum_c scale_B(r, c/32) * B[r][c] * x_b[c]
 * w_ssq: device, pti_ssq_bytes(rows, cols) bytes (4-byte aligned);
 * x_a, x_b: device fp32 [cols] (16-byte aligned; may be the same buffer);
 * y_a, y_b: device fp32 [rows], distinct, not overlapping any input. */
int pti_gemv_ssq(const void *w_ssq, const float *x_a, const float *x_b, float *y_a, float *y_b,
                 int64_t rows, int64_t cols, void *stream);

/* SSQ twin GEMV with n_per_twin streams per twin [README, relation to SSQ
 * (one slot load feeds both twins) combined with the bandwidth analysis (one
 * weight read feeds several activation vectors)]: one pass over the packed
 * matrix computes, for j < n_per_twin,
 *   y_a[j][r] = sum_c scale_A(r, c/32) * A[r][c] * x_a[j][c]
 *   y_b[j][r] = sum_c scale_B(r, c/32) * B[r][c] * x_b[j][c]
 * Each (twin, j) output is bitwise the one pti_gemv_ssq gives for
 * (x_a[j], x_b[j]).  x_a, x_b: device fp32 [n_per_twin][cols] contiguous
 * (16-byte aligned); y_a, y_b: device fp32 [n_per_twin][rows] contiguous, not
 * overlapping each other or any input; 1 <= n_per_twin <= 2 (else
 * PTI_ERR_NSTREAMS). */
int pti_gemv_ssq_multi(const void *w_ssq, const float *x_a, const float *x_b, float *y_a, float *y_b,
                       int64_t rows, int64_t cols, int n_per_twin, void *stream);

/* SSQ twin GEMV fused with the greedy verify of its two outputs [README,
 * relation to SSQ; README, how acceptance works]: the results of
 * pti_gemv_ssq (y_a, y_b bitwise the same) and those of pti_verify_argmax
 * over the streams (y_a, y_b) with vocab = rows, without a second pass over
 * y: argmax_out[0] = argmax y_a, argmax_out[1] = argmax y_b (lowest index wins
 * a tie; -0 equals +0; NaN ordering unspecified), accept_out[0] = 1 +
 * (tokens_in[1] == argmax_out[0]).  For the twin decode rows is the
 * vocabulary and y_a, y_b are the twins' logits; tokens_in[1] is the guess
 * twin B ran on, tokens_in[0] is not read.  The GEMV's workgroups keep the
 * largest output each; a one-workgroup kernel enqueued after it on the same
 * stream reduces those.
 * Arguments as in pti_gemv_ssq, plus: tokens_in: device int32 [2];
 * argmax_out: device int32 [2]; accept_out: device int32 [1] (4-byte aligned);
 * work: device scratch of at least PTI_SSQ_VERIFY_WORK_BYTES bytes, 16-byte
 * aligned, caller-owned, any contents (overwritten; calls that may run at the
 * same time need separate workspaces); work_bytes below
 * PTI_SSQ_VERIFY_WORK_BYTES gives PTI_ERR_SHAPE.  No output (y_a, y_b,
 * argmax_out, accept_out, work) may overlap an input or another output. */
int pti_gemv_ssq_verify(const void *w_ssq, const float *x_a, const float *x_b, float *y_a, float *y_b,
                        int64_t rows, int64_t cols, const int32_t *tokens_in, int32_t *argmax_out,
                        int32_t *accept_out, void *work, size_t work_bytes, void *stream);

/* Q8 multi-stream GEMV [README, bandwidth analysis: one weight read serves the
 * activation vectors of all streams]:
 *   y[n][r] = sum_c scale(r, c/32) * q[r][c] * x[n][c]   for n < n_streams
 * w_q8: device, pti_q8_bytes(rows, cols) bytes (4-byte aligned);
 * x: device fp32 [n_streams][cols], contiguous (16-byte aligned);
 * y: device fp32 [n_streams][rows], contiguous, not overlapping w or x;
 * 1 <= n_streams <= 4. */
int pti_gemv_q8_multi(const void *w_q8, const float *x, float *y, int64_t rows, int64_t cols,
                      int n_streams, void *stream);

/* Grouped GEMVs [README, bandwidth analysis: the per-token dispatch path is
 * where the pages' own implementation lost its time]: n_mats matrices with
 * the same column count and the same activations (q|k|v, gate|up) in one
 * launch, as if their rows were stacked in order into one matrix of
 * sum(rows) rows.  Every output is bitwise the one the single-matrix call
 * gives for its matrix.
 * w_ssq / w_q8: HOST array [n_mats] of device pointers, each 4-byte aligned,
 * matrix m of rows[m] rows (HOST array [n_mats], each >= 1);
 * 1 <= n_mats <= PTI_MAX_GROUP (else PTI_ERR_SHAPE), sum(rows) <=
 * PTI_MAX_ROWS.  Outputs over the stacked rows: matrix m's rows start at
 * row rows[0] + ... + rows[m-1].
 *   pti_gemv_ssq_grouped: y_a, y_b: device fp32 [sum(rows)]; x_a, x_b as in
 *     pti_gemv_ssq.
 *   pti_gemv_q8_multi_grouped: y: device fp32 [n_streams][sum(rows)]
 *     contiguous; x as in pti_gemv_q8_multi.
 * No output may overlap a matrix, an activation vector or the other output. */
int pti_gemv_ssq_grouped(const void *const *w_ssq, const int64_t *rows, int n_mats, const float *x_a,
                         const float *x_b, float *y_a, float *y_b, int64_t cols, void *stream);
int pti_gemv_q8_multi_grouped(const void *const *w_q8, const int64_t *rows, int n_mats, const float *x, float *y,
                              int64_t cols, int n_streams, void *stream);

/* Greedy verify [README, how acceptance works; Digest, implementation
 * architecture, step 3]: per stream n, argmax_out[n] = the index of the largest
 * logits[n][*] (the lowest index wins a tie; -0 equals +0; NaN ordering is
 * unspecified).  Stream 0 runs on the confirmed token; tokens_in[i] (i >= 1) is
 * the guess stream i ran on, checked against argmax_out[i-1].  accept_out[0] =
 * 1 + the number of leading checks i = 1, 2, ... that pass (a failed check
 * voids every later stream); tokens_in[0] is not read.
 * logits: device fp32 [n_streams][vocab] contiguous; tokens_in: device int32
 * [n_streams]; argmax_out: device int32 [n_streams]; accept_out: device int32
 * [1]; outputs must not overlap inputs or each other. */
int pti_verify_argmax(const float *logits, const int32_t *tokens_in, int32_t *argmax_out,
                      int32_t *accept_out, int64_t vocab, int n_streams, void *stream);

/* Sampled verify [README, how acceptance works: at temperature > 0 a guess is
 * confirmed when it equals the token the stream before it samples, which
 * happens with the collision probability sum_x p(x)^2; Digest, implementation
 * architecture: the softmax and verify kernels]: per stream n, weights
 * w_j = exp((logits[n][j] - max_j logits[n][j]) / temperature) in fp64, and
 * tokens_out[n] = the first index j of nonzero weight at which a running sum
 * of the weights exceeds uniforms[n] * sum_j w_j (if rounding leaves none, the
 * last index of nonzero weight before the target).  The vocabulary is cut
 * into parts of 2048 indices: a part's weights are exp((l_j - m_b) / T)
 * exp((m_b - M) / T) with m_b the part's max and M the stream's.  The running
 * sum is taken in a fixed, index-monotone order (over the parts in index
 * order, then inside the part that holds the target in index order), so the
 * draw equals an in-order sequential inverse-CDF draw except where u * sum
 * lies within a few fp64 ulps of a cumulative sum.  accept_out[0] as in
 * pti_verify_argmax, with the drawn tokens in place of the argmaxes.
 * logits: device fp32 [n_streams][vocab] (finite; otherwise tokens_out is
 * unspecified and may be -1); tokens_in: device int32 [n_streams];
 * uniforms: device fp64 [n_streams] in [0, 1) (8-byte aligned); temperature:
 * finite, > 0; tokens_out: device int32 [n_streams]; accept_out: device int32
 * [1]; work: device scratch of at least
 * pti_sample_verify_workspace_bytes(vocab, n_streams) bytes (16-byte aligned,
 * any contents; 0 for invalid sizes).  Outputs and work must not overlap
 * inputs or each other.  Three kernels are enqueued on `stream` (the parts'
 * sums, one workgroup per stream for the draw, the accept count); calls
 * sharing a workspace must not run at the same time. */
size_t pti_sample_verify_workspace_bytes(int64_t vocab, int n_streams);
int pti_sample_verify(const float *logits, const int32_t *tokens_in, const double *uniforms, double temperature,
                      int32_t *tokens_out, int32_t *accept_out, int64_t vocab, int n_streams, void *work,
                      size_t work_bytes, void *stream);

/* pti_sample_verify without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The part sums go to a scratch array the
 * library keeps in device memory: PTI_STATIC_SCRATCH_BYTES per GPU, held from
 * the first call on that GPU until the process ends; the call itself
 * allocates nothing.  Arguments, results and errors as pti_sample_verify,
 * plus PTI_ERR_SHAPE when pti_sample_verify_workspace_bytes(vocab,
 * n_streams) exceeds PTI_STATIC_SCRATCH_BYTES (at most 4096 parts of 2048
 * logits over all streams: vocab up to 2,097,152 at four streams), and
 * PTI_ERR_HIP if the scratch's device address cannot be obtained.  Every call
 * on one GPU shares that GPU's scratch: calls that overlap in time on one GPU
 * (on different streams or host threads) race and give wrong draws; calls
 * enqueued on one stream are ordered and safe.  Nothing needs to start at
 * zero: each call writes every part sum before reading it. */
#define PTI_STATIC_SCRATCH_BYTES 65536
int pti_sample_verify_static(const float *logits, const int32_t *tokens_in, const double *uniforms,
                             double temperature, int32_t *tokens_out, int32_t *accept_out, int64_t vocab,
                             int n_streams, void *stream);

/* ------------------------------------------------------------------------- */
/* Decoder-stack glue [Digest, implementation architecture: the forward pass in
 * which one weight load serves every stream].  Device calls, conventions as
 * above; they compute in fp64 internally and round once to fp32, so each
 * output is within 1 fp32 ulp of the exact value of its formula on the given
 * fp32 inputs (bit-exact for pti_embed_* and pti_add).                      */

/* x[n][c] = scale(tokens[n], c/32) * q[tokens[n]][c]: row tokens[n] of a Q8
 * matrix [vocab][hidden], dequantised.  tokens: device int32 [n_streams];
 * x: device fp32 [n_streams][hidden].  A token outside [0, vocab) yields a row
 * of NaN. */
int pti_embed_q8(const void *w_q8, const int32_t *tokens, float *x, int64_t vocab, int64_t hidden, int n_streams,
                 void *stream);
/* Two-stream form over an SSQ matrix [vocab][hidden]: x[0] = twin A's row
 * tokens[0], x[1] = twin B's row tokens[1].  tokens: device int32 [2];
 * x: device fp32 [2][hidden]. */
int pti_embed_ssq(const void *w_ssq, const int32_t *tokens, float *x, int64_t vocab, int64_t hidden, void *stream);

/* y[n][c] = x[n][c] / sqrt(mean_c x[n][c]^2 + eps) (no gain), for
 * n < n_streams; x, y: device fp32 [n_streams][dim]; y may equal x (in place)
 * but not overlap it otherwise; eps finite, >= 0; 1 <= dim <= PTI_MAX_ELEMS.
 * Sums in fp64, then x times the fp64 reciprocal of the root: each output is
 * within one fp32 ulp of the formula. */
int pti_rmsnorm(const float *x, float *y, int64_t dim, int n_streams, float eps, void *stream);

/* y[i] = g[i] / (1 + exp(-g[i])) * u[i] (SiLU gate times up projection), i < n.
 * y may equal g or u (in place) but not overlap them otherwise. */
int pti_silu_mul(const float *g, const float *u, float *y, int64_t n, void *stream);

/* y[i] = a[i] + b[i] in fp32 (the residual add), i < n.  y may equal a or b. */
int pti_add(const float *a, const float *b, float *y, int64_t n, void *stream);

/* ------------------------------------------------------------------------- */
/* Twin-KV decode attention [Digest, implementation architecture: twins A and
 * B keep separate KV caches, one pass serves both streams, an accept extends
 * B's cache and a reject resets B's state; Notes (the LLM-inference page),
 * from naive inference to the KV cache: a decode step appends the new key
 * and value and attends over the cache].
 *
 * For each stream s < n_streams (each with its own cache):
 *   1. store: K_s[g][pos[s]] = binary16(k_new[s][g]) and likewise V (round to
 *      nearest even), replacing the entry there -- a reject's redraw runs at
 *      the same position and so replaces the stale speculative entry;
 *   2. attend: out[s][h] = sum_{j <= pos[s]} softmax_j(q[s][h] . K_s[g][j] /
 *      sqrt(head_dim)) V_s[g][j], with kv head g = h / (n_heads / n_kv_heads).
 * Accuracy is that of fp32 arithmetic: both products run on the matrix
 * cores with q (scaled per head by a power of two) and the softmax weights
 * each split into a high and a low binary16 part, and every binary16 product
 * is exact in fp32.  Finite inputs of any magnitude are handled; binary16
 * subnormals in the caches are used as they are.
 * q: device fp32 [n_streams][n_heads][head_dim]; k_new, v_new: device fp32
 * [n_streams][n_kv_heads][head_dim]; k_cache, v_cache: HOST arrays
 * [n_streams] of device binary16 caches [n_kv_heads][max_len][head_dim]
 * (16-byte aligned, caller-owned, distinct); pos: device int32 [n_streams]
 * (read on the device, so a captured graph can replay with new positions; a
 * position outside [0, max_len) makes that stream's outputs NaN and touches
 * no cache); out: device fp32 [n_streams][n_heads][head_dim]; work: device
 * scratch of at least pti_attn_workspace_bytes bytes (16-byte aligned), any
 * contents.
 * Limits: head_dim 64 or 128; n_heads a multiple of n_kv_heads, at most 8
 * query heads per kv head; 1 <= max_len <= PTI_MAX_ATTN_LEN.  No output
 * (out, work, any cache) may overlap an input or another output.  Two
 * kernels are enqueued on `stream`; calls sharing a workspace must not run
 * at the same time. */
size_t pti_attn_workspace_bytes(int n_streams, int n_heads, int n_kv_heads, int head_dim, int64_t max_len);
int pti_attn_decode(const float *q, const float *k_new, const float *v_new, uint16_t *const *k_cache,
                    uint16_t *const *v_cache, const int32_t *pos, float *out, int n_streams, int n_heads,
                    int n_kv_heads, int head_dim, int64_t max_len, void *work, size_t work_bytes, void *stream);

/* ------------------------------------------------------------------------- */
/* Toy decoder stack and the staggered multi-stream decode loop.
 *
 * The pages run one model as N staggered streams that share every weight load
 * [README, how acceptance works; Digest, implementation architecture].  The
 * stand-in model is an MLP-residual stack:
 *   h_0 = embed row of the token;
 *   h_{l+1} = h_l + down_l(silu(gate_l r_l) * up_l r_l), r_l = rmsnorm(h_l);
 *   logits = head rmsnorm(h_L).
 * All matrices share one format.  PTI_FMT_Q8: each pass serves n_streams in
 * 1..4 through the multi-stream GEMV.  PTI_FMT_SSQ: a twin pair packed side by
 * side; a pass serves exactly 2 streams, stream 0 on twin A (the verifier) and
 * stream 1 on twin B (the drafter).                                          */

#define PTI_FMT_Q8 0
#define PTI_FMT_SSQ 1
#define PTI_TOY_MAX_LAYERS 64

typedef struct pti_toy_model {
    int32_t format;   /* PTI_FMT_Q8 or PTI_FMT_SSQ */
    int32_t n_layers; /* 1 .. PTI_TOY_MAX_LAYERS */
    int64_t hidden;   /* multiple of 32 */
    int64_t ffn;      /* multiple of 32 */
    int64_t vocab;
    float eps;        /* RMSNorm epsilon, finite, >= 0 */
    const void *embed;       /* device, [vocab][hidden] */
    const void *head;        /* device, [vocab][hidden] */
    const void *const *gate; /* host array of n_layers device pointers, [ffn][hidden] each */
    const void *const *up;   /* same */
    const void *const *down; /* host array of n_layers device pointers, [hidden][ffn] each */
} pti_toy_model;

/* Device workspace bytes needed by pti_toy_forward / pti_toy_decode for this
 * model and stream count; 0 if the model or n_streams is invalid. */
size_t pti_toy_workspace_bytes(const pti_toy_model *m, int n_streams);

/* One pass: logits[n][*] for tokens[n], n < n_streams (2 for SSQ).
 * tokens: device int32 [n_streams]; logits: device fp32 [n_streams][vocab];
 * work: device, >= pti_toy_workspace_bytes bytes, 256-byte aligned, not
 * overlapping tokens or logits.  Enqueued on `stream`, no synchronisation. */
int pti_toy_forward(const pti_toy_model *m, const int32_t *tokens, float *logits, void *work, size_t work_bytes,
                    int n_streams, void *stream);

/* One pass of pti_toy_forward captured into an instantiated HIP graph
 * [README, bandwidth analysis: the per-token dispatch path], so that a pass
 * is one launch call however many kernels it has.  Arguments as in
 * pti_toy_forward; the graph reads tokens and writes logits and work at
 * these addresses on every replay (write new tokens into the same buffer).
 * *graph_out: an opaque handle for pti_graph_launch (NULL on error); the
 * caller owns it and frees it with pti_graph_destroy.  Nothing is enqueued
 * or run by this call (the capture uses a private stream). */
int pti_toy_forward_graph(const pti_toy_model *m, const int32_t *tokens, float *logits, void *work,
                          size_t work_bytes, int n_streams, void **graph_out);
/* Enqueue one replay of a graph on `stream`. */
int pti_graph_launch(void *graph, void *stream);
/* Free a graph handle (NULL is a no-op). */
int pti_graph_destroy(void *graph);

/* The staggered decode loop, n_steps steps after first_token.
 *   - Ramp-up (step 0): stream i >= 1 gets its first input from single-stream
 *     passes, x_i = draw(x_{i-1}), pass slots N .. 2N-2.
 *   - Step k = 1 .. n_steps: one N-stream pass (slots 0 .. N-1) draws o_0 ..
 *     o_{N-1}; accepts[k-1] = 1 + leading run of x_i == o_{i-1};
 *     committed[k-1] = o_0; stream i's next input is o_i.
 *   - When accepts[k-1] = a < N, streams a .. N-1 ran on stale guesses: their
 *     next inputs are drawn again by single-stream passes starting from
 *     o_{a-1} (slots N .. 2N-1-a).
 * A draw is the argmax of the logits (temperature == 0) or the sampled-verify
 * draw at that temperature with uniform uniforms[k * 2N + slot].  A greedy
 * pass whose Q8 LM head runs the per-wave-row kernel with the norm fused
 * takes the argmaxes from per-workgroup keys that the head writes into
 * `work` (the same argmax, lowest index among equals, without a second pass
 * over the logits); any other pass runs pti_verify_argmax.  A
 * single-stream pass of stream i >= 1 runs twin B in the SSQ format.
 * uniforms: host fp64 [(n_steps + 1) * 2 * N], may be NULL when temperature
 * is 0.  committed, accepts: host int32 [n_steps].  passes: host int32
 * [(N - 1) + n_steps * (2N - 1)][5] or NULL; each executed draw appends
 * (step, slot, stream, input token, output token) and *n_passes (host, may be
 * NULL) receives their count.  Synchronises `stream` after every pass (the
 * next inputs depend on the accept count).  The pass's verify kernel writes
 * the draws and the accept count straight into a page of pinned, coherent
 * host memory (no copy command per pass); the page belongs to the calling
 * thread, is allocated at its first call (an allocation failure returns
 * PTI_ERR_HIP) and is kept until the process ends. */
int pti_toy_decode(const pti_toy_model *m, int32_t first_token, int n_streams, int n_steps, double temperature,
                   const double *uniforms, void *work, size_t work_bytes, int32_t *committed, int32_t *accepts,
                   int32_t *passes, int64_t *n_passes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PTI_H */

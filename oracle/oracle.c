/*
 * oracle.c -- plain, slow, scalar fp64 CPU oracle for the packed-twin decode path.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
 * baseline may load or call this code.  It shares nothing with the HIP library:
 * its own f16 decoder, its own block packer and unpacker, its own dot products.
 * Built with gcc -O2 -ffp-contract=off (no fast-math, no FMA contraction).
 *
 * Pages cited (by title and section):
 *   [Digest]  "Packed Twin Inference：无需草稿模型的推测解码新方案，实现2倍吞吐量提升"
 *             (zingnex.cn forum digest of the packed-twin-inference project).
 *   [README]  "打包双子推理（PTI）" (bittide.aicompass.dev page carrying the
 *             project README in Chinese translation).
 *
 * Formats (little-endian throughout):
 *   SSQ mode-16 block, 68 bytes, 32 weights of each twin
 *     [Digest, section "PTI的核心创新：SSQ打包技术" (SSQ packing), block layout]:
 *       bytes 0..1   scale of twin A (IEEE binary16)
 *       bytes 2..3   scale of twin B (IEEE binary16)
 *       bytes 4+2j, 5+2j  slot j (uint16): twin A's int8 in the high byte,
 *                         twin B's int8 in the low byte, so in memory the low
 *                         byte (twin B) comes first
 *                         [README, section "与 SSQ（Side-by-Side Quantization）的关系",
 *                          the unpack arithmetic: A = slot >> 8, B = slot & 0xFF]
 *   Q8 block, 34 bytes: bytes 0..1 scale (binary16), bytes 2+j the int8 weight j.
 *     (Two Q8 blocks have the byte count of one SSQ block [Digest, SSQ packing].)
 *   Matrices are row-major: row r holds cols/32 consecutive blocks, row r+1
 *   follows with no padding; output index = row, block b covers columns
 *   32b .. 32b+31.
 *
 * Every value here is computed in double.  A product scale*q*x is exact in double
 * (11 + 8 + 24 significant bits); only the running sums round.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#define ORC_BLOCK 32
#define ORC_SSQ_BYTES 68
#define ORC_Q8_BYTES 34

/* IEEE 754 binary16 -> double, written from the format's definition:
 * sign bit, 5 exponent bits (bias 15), 10 fraction bits; exponent 0 encodes
 * zero and subnormals (fraction * 2^-24), exponent 31 encodes Inf/NaN. */
double orc_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1f;
    int fr = h & 0x3ff;
    double v;
    if (ex == 0)
        v = ldexp((double)fr, -24);
    else if (ex == 31)
        v = fr ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + fr), ex - 25);
    return sign ? -v : v;
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static void wr16(uint8_t *p, uint16_t v)
{
    p[0] = (uint8_t)(v & 0xff);
    p[1] = (uint8_t)(v >> 8);
}

size_t orc_ssq_bytes(int64_t rows, int64_t cols) { return (size_t)(rows * (cols / ORC_BLOCK) * ORC_SSQ_BYTES); }
size_t orc_q8_bytes(int64_t rows, int64_t cols) { return (size_t)(rows * (cols / ORC_BLOCK) * ORC_Q8_BYTES); }

/* ---- packing [Digest, SSQ packing; README, relation to SSQ] ------------------ */

void orc_pack_ssq(const int8_t *a, const int8_t *b, const uint16_t *sa, const uint16_t *sb,
                  int64_t rows, int64_t cols, uint8_t *out)
{
    int64_t nb = cols / ORC_BLOCK;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t k = 0; k < nb; k++) {
            uint8_t *blk = out + (r * nb + k) * ORC_SSQ_BYTES;
            wr16(blk + 0, sa[r * nb + k]);
            wr16(blk + 2, sb[r * nb + k]);
            for (int j = 0; j < ORC_BLOCK; j++) {
                int64_t c = k * ORC_BLOCK + j;
                uint16_t slot = (uint16_t)(((uint8_t)a[r * cols + c] << 8) | (uint8_t)b[r * cols + c]);
                wr16(blk + 4 + 2 * j, slot);
            }
        }
}

void orc_unpack_ssq(const uint8_t *in, int64_t rows, int64_t cols, int8_t *a, int8_t *b,
                    uint16_t *sa, uint16_t *sb)
{
    int64_t nb = cols / ORC_BLOCK;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t k = 0; k < nb; k++) {
            const uint8_t *blk = in + (r * nb + k) * ORC_SSQ_BYTES;
            sa[r * nb + k] = rd16(blk + 0);
            sb[r * nb + k] = rd16(blk + 2);
            for (int j = 0; j < ORC_BLOCK; j++) {
                uint16_t slot = rd16(blk + 4 + 2 * j);
                a[r * cols + k * ORC_BLOCK + j] = (int8_t)(uint8_t)(slot >> 8);
                b[r * cols + k * ORC_BLOCK + j] = (int8_t)(uint8_t)(slot & 0xff);
            }
        }
}

void orc_pack_q8(const int8_t *q, const uint16_t *s, int64_t rows, int64_t cols, uint8_t *out)
{
    int64_t nb = cols / ORC_BLOCK;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t k = 0; k < nb; k++) {
            uint8_t *blk = out + (r * nb + k) * ORC_Q8_BYTES;
            wr16(blk, s[r * nb + k]);
            for (int j = 0; j < ORC_BLOCK; j++)
                blk[2 + j] = (uint8_t)q[r * cols + k * ORC_BLOCK + j];
        }
}

void orc_unpack_q8(const uint8_t *in, int64_t rows, int64_t cols, int8_t *q, uint16_t *s)
{
    int64_t nb = cols / ORC_BLOCK;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t k = 0; k < nb; k++) {
            const uint8_t *blk = in + (r * nb + k) * ORC_Q8_BYTES;
            s[r * nb + k] = rd16(blk);
            for (int j = 0; j < ORC_BLOCK; j++)
                q[r * cols + k * ORC_BLOCK + j] = (int8_t)blk[2 + j];
        }
}

/* ---- GEMV: y[r] = sum_c scale(r, c/32) * q[r][c] * x[c] ----------------------
 * The per-weight form of the twin accumulation in [README, relation to SSQ]
 * (acc += scale * weight * x for each twin), summed in column order.
 * t[r] = sum_c |scale| * |q| * |x| is the magnitude the error bound is measured
 * against.  One pass per (row, stream). */

static void dot_q8_row(const uint8_t *row, int64_t nb, const float *x, double *y, double *t)
{
    double acc = 0.0, mag = 0.0;
    for (int64_t k = 0; k < nb; k++) {
        const uint8_t *blk = row + k * ORC_Q8_BYTES;
        double d = orc_f16_to_f64(rd16(blk));
        for (int j = 0; j < ORC_BLOCK; j++) {
            double w = d * (double)(int8_t)blk[2 + j];
            double xv = (double)x[k * ORC_BLOCK + j];
            acc += w * xv;
            mag += fabs(w) * fabs(xv);
        }
    }
    *y = acc;
    *t = mag;
}

/* Q8 GEMV over n activation vectors x[n][cols] -> y[n][rows], t[n][rows]. */
void orc_gemv_q8(const uint8_t *w, int64_t rows, int64_t cols, const float *x, int n,
                 double *y, double *t)
{
    int64_t nb = cols / ORC_BLOCK;
    for (int s = 0; s < n; s++)
        for (int64_t r = 0; r < rows; r++)
            dot_q8_row(w + r * nb * ORC_Q8_BYTES, nb, x + (int64_t)s * cols, y + (int64_t)s * rows + r,
                       t + (int64_t)s * rows + r);
}

/* Same as orc_gemv_q8 for the listed rows only (sampled checks of big shapes);
 * y and t are [n][n_idx]. */
void orc_gemv_q8_rows(const uint8_t *w, int64_t rows, int64_t cols, const float *x, int n,
                      const int64_t *row_idx, int64_t n_idx, double *y, double *t)
{
    int64_t nb = cols / ORC_BLOCK;
    (void)rows;
    for (int s = 0; s < n; s++)
        for (int64_t i = 0; i < n_idx; i++)
            dot_q8_row(w + row_idx[i] * nb * ORC_Q8_BYTES, nb, x + (int64_t)s * cols,
                       y + (int64_t)s * n_idx + i, t + (int64_t)s * n_idx + i);
}

static void dot_ssq_row(const uint8_t *row, int64_t nb, const float *xa, const float *xb,
                        double *ya, double *yb, double *ta, double *tb)
{
    double acc_a = 0.0, acc_b = 0.0, mag_a = 0.0, mag_b = 0.0;
    for (int64_t k = 0; k < nb; k++) {
        const uint8_t *blk = row + k * ORC_SSQ_BYTES;
        double da = orc_f16_to_f64(rd16(blk + 0));
        double db = orc_f16_to_f64(rd16(blk + 2));
        for (int j = 0; j < ORC_BLOCK; j++) {
            uint16_t slot = rd16(blk + 4 + 2 * j);
            double wa = da * (double)(int8_t)(uint8_t)(slot >> 8);
            double wb = db * (double)(int8_t)(uint8_t)(slot & 0xff);
            double xav = (double)xa[k * ORC_BLOCK + j];
            double xbv = (double)xb[k * ORC_BLOCK + j];
            acc_a += wa * xav;
            acc_b += wb * xbv;
            mag_a += fabs(wa) * fabs(xav);
            mag_b += fabs(wb) * fabs(xbv);
        }
    }
    *ya = acc_a;
    *yb = acc_b;
    *ta = mag_a;
    *tb = mag_b;
}

/* SSQ twin GEMV: one pass over the packed twin matrix feeds both outputs. */
void orc_gemv_ssq(const uint8_t *w, int64_t rows, int64_t cols, const float *xa, const float *xb,
                  double *ya, double *yb, double *ta, double *tb)
{
    int64_t nb = cols / ORC_BLOCK;
    for (int64_t r = 0; r < rows; r++)
        dot_ssq_row(w + r * nb * ORC_SSQ_BYTES, nb, xa, xb, ya + r, yb + r, ta + r, tb + r);
}

void orc_gemv_ssq_rows(const uint8_t *w, int64_t rows, int64_t cols, const float *xa, const float *xb,
                       const int64_t *row_idx, int64_t n_idx, double *ya, double *yb, double *ta,
                       double *tb)
{
    int64_t nb = cols / ORC_BLOCK;
    (void)rows;
    for (int64_t i = 0; i < n_idx; i++)
        dot_ssq_row(w + row_idx[i] * nb * ORC_SSQ_BYTES, nb, xa, xb, ya + i, yb + i, ta + i, tb + i);
}

/* ---- greedy verify [README, section "接受机制如何工作" (how acceptance works);
 *      Digest, section "技术实现架构" step 3] -----------------------------------
 * Stream 0 runs on the last confirmed token; stream i >= 1 runs on a guess for
 * the position that stream i-1 predicts.  The guess fed to stream i is accepted
 * when it equals stream i-1's greedy output; a failed check voids every stream
 * after it, so the accept count is 1 plus the length of the leading run of
 * successful checks. */

/* Index of the largest value; the first (lowest) index wins a tie.  Plain
 * comparison, so -0 and +0 are equal. */
int64_t orc_argmax(const float *v, int64_t n)
{
    int64_t best = 0;
    for (int64_t i = 1; i < n; i++)
        if (v[i] > v[best])
            best = i;
    return best;
}

int orc_accept_count(const int32_t *tokens_in, const int32_t *argmax, int n)
{
    int a = 1;
    for (int i = 1; i < n; i++) {
        if (tokens_in[i] != argmax[i - 1])
            break;
        a++;
    }
    return a;
}

/* argmax per stream of logits[n][vocab], then the accept count. */
int orc_verify_argmax(const float *logits, const int32_t *tokens_in, int32_t *argmax_out,
                      int64_t vocab, int n)
{
    for (int s = 0; s < n; s++)
        argmax_out[s] = (int32_t)orc_argmax(logits + (int64_t)s * vocab, vocab);
    return orc_accept_count(tokens_in, argmax_out, n);
}

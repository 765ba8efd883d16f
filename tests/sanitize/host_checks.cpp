// Host checks of libpti and the oracle, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (tests/test_sanitize.py builds
// and runs it; no GPU is used).
//
//   * the packer, unpacker, split and join against the oracle's packer, over
//     odd shapes, int8 -128 and every binary16 scale pattern;
//   * the argument checks of every device entry point (null pointers, shapes,
//     stream counts, alignment, overlaps): each call must return its status
//     before it touches memory (the device pointers are fake addresses);
//   * the oracle's f16 decode, GEMVs, argmax and verify on small inputs.
// Prints one line per group and exits 0 when every check held.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "pti.h"

extern "C" {
double orc_f16_to_f64(uint16_t h);
void orc_pack_ssq(const int8_t *a, const int8_t *b, const uint16_t *sa, const uint16_t *sb, int64_t rows,
                  int64_t cols, uint8_t *out);
void orc_pack_q8(const int8_t *q, const uint16_t *s, int64_t rows, int64_t cols, uint8_t *out);
void orc_gemv_q8(const uint8_t *w, int64_t rows, int64_t cols, const float *x, int n, double *y, double *t);
void orc_gemv_ssq(const uint8_t *w, int64_t rows, int64_t cols, const float *xa, const float *xb, double *ya,
                  double *yb, double *ta, double *tb);
int64_t orc_argmax(const float *v, int64_t n);
int orc_accept_count(const int32_t *tokens_in, const int32_t *argmax, int n);
int orc_verify_argmax(const float *logits, const int32_t *tokens_in, int32_t *argmax_out, int64_t vocab, int n);
}

static int g_fail = 0, g_checks = 0;

#define CHECK(cond)                                                                  \
    do {                                                                             \
        g_checks++;                                                                  \
        if (!(cond)) {                                                               \
            std::printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);              \
            g_fail++;                                                                \
        }                                                                            \
    } while (0)
#define EXPECT(call, want)                                                           \
    do {                                                                             \
        g_checks++;                                                                  \
        const int got_ = (call);                                                     \
        if (got_ != (want)) {                                                        \
            std::printf("FAIL %s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, #call, got_, (int)(want)); \
            g_fail++;                                                                \
        }                                                                            \
    } while (0)

static uint64_t g_rng = 0x9E3779B97F4A7C15ull;
static uint32_t rnd()
{
    g_rng ^= g_rng << 13;
    g_rng ^= g_rng >> 7;
    g_rng ^= g_rng << 17;
    return (uint32_t)(g_rng >> 16);
}

// fake, never dereferenced device addresses (every call fails validation first)
static void *F(uintptr_t a) { return reinterpret_cast<void *>(a); }
static float *FF(uintptr_t a) { return reinterpret_cast<float *>(a); }
static const uintptr_t A0 = 0x10000000, A1 = 0x20000000, A2 = 0x30000000, A3 = 0x40000000, A4 = 0x50000000;

static void packer(int64_t rows, int64_t cols, bool every_f16)
{
    const int64_t nb = cols / 32, n = rows * cols, ns = rows * nb;
    std::vector<int8_t> a(n), b(n);
    std::vector<uint16_t> sa(ns), sb(ns);
    for (int64_t i = 0; i < n; i++) {
        a[i] = (int8_t)(rnd() & 0xFF);
        b[i] = (int8_t)(rnd() & 0xFF);
    }
    a[0] = -128;
    b[n - 1] = -128;
    for (int64_t i = 0; i < ns; i++) {
        sa[i] = every_f16 ? (uint16_t)i : (uint16_t)rnd();
        sb[i] = every_f16 ? (uint16_t)(0xFFFF - i) : (uint16_t)rnd();
    }
    const size_t sz = pti_ssq_bytes(rows, cols), qz = pti_q8_bytes(rows, cols);
    CHECK(sz == (size_t)(ns * 68) && qz == (size_t)(ns * 34));
    std::vector<uint8_t> p(sz), o(sz), qa(qz), qb(qz), oq(qz), j(sz);
    EXPECT(pti_pack_ssq(a.data(), b.data(), sa.data(), sb.data(), rows, cols, p.data()), PTI_OK);
    orc_pack_ssq(a.data(), b.data(), sa.data(), sb.data(), rows, cols, o.data());
    CHECK(p == o);
    std::vector<int8_t> a2(n), b2(n);
    std::vector<uint16_t> sa2(ns), sb2(ns);
    EXPECT(pti_unpack_ssq(p.data(), rows, cols, a2.data(), b2.data(), sa2.data(), sb2.data()), PTI_OK);
    CHECK(a2 == a && b2 == b && sa2 == sa && sb2 == sb);
    EXPECT(pti_ssq_split(p.data(), rows, cols, qa.data(), qb.data()), PTI_OK);
    orc_pack_q8(a.data(), sa.data(), rows, cols, oq.data());
    CHECK(qa == oq);
    orc_pack_q8(b.data(), sb.data(), rows, cols, oq.data());
    CHECK(qb == oq);
    EXPECT(pti_ssq_join(qa.data(), qb.data(), rows, cols, j.data()), PTI_OK);
    CHECK(j == p);
    std::vector<uint8_t> q(qz);
    EXPECT(pti_pack_q8(a.data(), sa.data(), rows, cols, q.data()), PTI_OK);
    orc_pack_q8(a.data(), sa.data(), rows, cols, oq.data());
    CHECK(q == oq);
    EXPECT(pti_unpack_q8(q.data(), rows, cols, a2.data(), sa2.data()), PTI_OK);
    CHECK(a2 == a && sa2 == sa);
}

static void packer_errors()
{
    std::vector<uint8_t> buf(8192);
    uint8_t *p = buf.data();
    const int8_t *i8 = reinterpret_cast<const int8_t *>(p);
    const uint16_t *u16 = reinterpret_cast<const uint16_t *>(p);
    EXPECT(pti_pack_ssq(nullptr, i8, u16, u16, 1, 32, p), PTI_ERR_NULL);
    EXPECT(pti_pack_ssq(i8, i8, u16, u16, 1, 33, p), PTI_ERR_SHAPE);
    EXPECT(pti_pack_ssq(i8, i8, u16, u16, 0, 32, p), PTI_ERR_SHAPE);
    EXPECT(pti_pack_ssq(i8, i8, u16, u16, 1, 0, p), PTI_ERR_SHAPE);
    EXPECT(pti_pack_q8(i8, u16, 1, 16, p), PTI_ERR_SHAPE);
    EXPECT(pti_pack_q8(i8, nullptr, 1, 32, p), PTI_ERR_NULL);
    EXPECT(pti_unpack_q8(p, -1, 32, reinterpret_cast<int8_t *>(p), reinterpret_cast<uint16_t *>(p)), PTI_ERR_SHAPE);
    EXPECT(pti_unpack_ssq(p, 1, 32, nullptr, nullptr, nullptr, nullptr), PTI_ERR_NULL);
    EXPECT(pti_ssq_split(p, 1, 32, p, p + 2000), PTI_ERR_OVERLAP);
    EXPECT(pti_ssq_split(p, 1, 32, p + 100, p + 100), PTI_ERR_OVERLAP);
    EXPECT(pti_ssq_join(p, p + 100, 1, 32, p + 50), PTI_ERR_OVERLAP);
    EXPECT(pti_ssq_join(p, nullptr, 1, 32, p + 500), PTI_ERR_NULL);
    CHECK(pti_ssq_bytes(1, 31) == 0 && pti_q8_bytes(0, 32) == 0 && pti_ssq_bytes(-5, 64) == 0);
    CHECK(pti_ssq_bytes(2, 64) == 272 && pti_q8_bytes(2, 64) == 136);
    CHECK(pti_ssq_bytes(1, (int64_t(1) << 24) + 32) == 0);
    for (int s = -8; s <= 8; s++)
        CHECK(pti_status_str(s) != nullptr);
    CHECK(std::strcmp(pti_status_str(7), "unknown status") == 0);
    CHECK(pti_abi_version() == 1);
}

static void device_errors()
{
    // SSQ twin GEMV
    EXPECT(pti_gemv_ssq(nullptr, FF(A1), FF(A1), FF(A2), FF(A3), 8, 64, nullptr), PTI_ERR_NULL);
    EXPECT(pti_gemv_ssq(F(A0), FF(A1), FF(A1), nullptr, FF(A3), 8, 64, nullptr), PTI_ERR_NULL);
    EXPECT(pti_gemv_ssq(F(A0), FF(A1), FF(A1), FF(A2), FF(A3), 0, 64, nullptr), PTI_ERR_SHAPE);
    EXPECT(pti_gemv_ssq(F(A0), FF(A1), FF(A1), FF(A2), FF(A3), 8, 48, nullptr), PTI_ERR_SHAPE);
    EXPECT(pti_gemv_ssq(F(A0), FF(A1), FF(A1), FF(A2), FF(A3), 8, (int64_t(1) << 24) + 32, nullptr), PTI_ERR_SHAPE);
    EXPECT(pti_gemv_ssq(F(A0 + 2), FF(A1), FF(A1), FF(A2), FF(A3), 8, 64, nullptr), PTI_ERR_ALIGN);
    EXPECT(pti_gemv_ssq(F(A0), FF(A1 + 4), FF(A1), FF(A2), FF(A3), 8, 64, nullptr), PTI_ERR_ALIGN);
    EXPECT(pti_gemv_ssq(F(A0), FF(A1), FF(A1), FF(A2), FF(A2 + 16), 8, 64, nullptr), PTI_ERR_OVERLAP);
    EXPECT(pti_gemv_ssq(F(A0), FF(A1), FF(A1), FF(A0 + 64), FF(A3), 8, 64, nullptr), PTI_ERR_OVERLAP);
    // two streams per twin
    EXPECT(pti_gemv_ssq_multi(F(A0), nullptr, FF(A1), FF(A2), FF(A3), 8, 64, 1, nullptr), PTI_ERR_NULL);
    EXPECT(pti_gemv_ssq_multi(F(A0), FF(A1), FF(A1), FF(A2), FF(A3), 8, 64, 0, nullptr), PTI_ERR_NSTREAMS);
    EXPECT(pti_gemv_ssq_multi(F(A0), FF(A1), FF(A1), FF(A2), FF(A3), 8, 64, 3, nullptr), PTI_ERR_NSTREAMS);
    EXPECT(pti_gemv_ssq_multi(F(A0), FF(A1), FF(A1), FF(A2), FF(A2 + 32), 8, 64, 2, nullptr), PTI_ERR_OVERLAP);
    // fused SSQ + verify
    const uintptr_t T = 0x60000000, AM = 0x61000000, AC = 0x62000000, WK = 0x63000000;
    const size_t W = PTI_SSQ_VERIFY_WORK_BYTES;
    auto fv = [&](uintptr_t w, uintptr_t ya, uintptr_t yb, uintptr_t t, uintptr_t am, uintptr_t ac, uintptr_t wk,
                  size_t wb, int64_t rows) {
        return pti_gemv_ssq_verify(w ? F(w) : nullptr, FF(A1), FF(A1), FF(ya), FF(yb), rows, 64,
                                   t ? reinterpret_cast<const int32_t *>(t) : nullptr,
                                   am ? reinterpret_cast<int32_t *>(am) : nullptr,
                                   ac ? reinterpret_cast<int32_t *>(ac) : nullptr, wk ? F(wk) : nullptr, wb, nullptr);
    };
    EXPECT(fv(0, A2, A3, T, AM, AC, WK, W, 8), PTI_ERR_NULL);
    EXPECT(fv(A0, A2, A3, 0, AM, AC, WK, W, 8), PTI_ERR_NULL);
    EXPECT(fv(A0, A2, A3, T, AM, AC, 0, W, 8), PTI_ERR_NULL);
    EXPECT(fv(A0, A2, A3, T, AM, AC, WK, W, 0), PTI_ERR_SHAPE);
    EXPECT(fv(A0, A2, A3, T, AM, AC, WK, W - 1, 8), PTI_ERR_SHAPE);
    EXPECT(fv(A0, A2, A3, T, AM, AC, WK + 8, W, 8), PTI_ERR_ALIGN);
    EXPECT(fv(A0, A2, A3, T, AM, AM + 4, WK, W, 8), PTI_ERR_OVERLAP);
    EXPECT(fv(A0, A2, A3, T, AM, AC, A2 - 1024, W, 8), PTI_ERR_OVERLAP);
    EXPECT(fv(A0, A2, A0 + 128, T, AM, AC, WK, W, 8), PTI_ERR_OVERLAP);
    // Q8 multi-stream
    EXPECT(pti_gemv_q8_multi(F(A0), nullptr, FF(A2), 8, 64, 1, nullptr), PTI_ERR_NULL);
    EXPECT(pti_gemv_q8_multi(F(A0), FF(A1), FF(A2), 8, 64, 0, nullptr), PTI_ERR_NSTREAMS);
    EXPECT(pti_gemv_q8_multi(F(A0), FF(A1), FF(A2), 8, 64, 5, nullptr), PTI_ERR_NSTREAMS);
    EXPECT(pti_gemv_q8_multi(F(A0), FF(A1), FF(A2), 8, 0, 1, nullptr), PTI_ERR_SHAPE);
    EXPECT(pti_gemv_q8_multi(F(A0), FF(A1 + 8), FF(A2), 8, 64, 1, nullptr), PTI_ERR_ALIGN);
    EXPECT(pti_gemv_q8_multi(F(A0), FF(A1), FF(A1 - 64), 8, 64, 4, nullptr), PTI_ERR_OVERLAP);
    // grouped
    const void *ws[3] = {F(A0), F(A0 + 0x100000), F(A0 + 0x200000)};
    const void *wbad[3] = {F(A0), nullptr, F(A0)};
    const void *wmis[3] = {F(A0), F(A0 + 0x100002), F(A0)};
    const int64_t R[3] = {8, 4, 4}, Rbad[3] = {8, 0, 4};
    EXPECT(pti_gemv_q8_multi_grouped(nullptr, R, 3, FF(A1), FF(A2), 64, 1, nullptr), PTI_ERR_NULL);
    EXPECT(pti_gemv_q8_multi_grouped(ws, nullptr, 3, FF(A1), FF(A2), 64, 1, nullptr), PTI_ERR_NULL);
    EXPECT(pti_gemv_q8_multi_grouped(ws, R, 0, FF(A1), FF(A2), 64, 1, nullptr), PTI_ERR_SHAPE);
    EXPECT(pti_gemv_q8_multi_grouped(ws, R, 5, FF(A1), FF(A2), 64, 1, nullptr), PTI_ERR_SHAPE);  // arrays not read
    EXPECT(pti_gemv_q8_multi_grouped(ws, R, 3, FF(A1), FF(A2), 64, 0, nullptr), PTI_ERR_NSTREAMS);
    EXPECT(pti_gemv_q8_multi_grouped(wbad, R, 3, FF(A1), FF(A2), 64, 1, nullptr), PTI_ERR_NULL);
    EXPECT(pti_gemv_q8_multi_grouped(ws, Rbad, 3, FF(A1), FF(A2), 64, 1, nullptr), PTI_ERR_SHAPE);
    EXPECT(pti_gemv_q8_multi_grouped(wmis, R, 3, FF(A1), FF(A2), 64, 1, nullptr), PTI_ERR_ALIGN);
    EXPECT(pti_gemv_q8_multi_grouped(ws, R, 3, FF(A1), FF(A0 + 0x100000 + 64), 64, 1, nullptr), PTI_ERR_OVERLAP);
    EXPECT(pti_gemv_ssq_grouped(ws, R, 3, FF(A1), nullptr, FF(A2), FF(A3), 64, nullptr), PTI_ERR_NULL);
    EXPECT(pti_gemv_ssq_grouped(ws, R, 5, FF(A1), FF(A1), FF(A2), FF(A3), 64, nullptr), PTI_ERR_SHAPE);
    EXPECT(pti_gemv_ssq_grouped(ws, R, 3, FF(A1), FF(A1), FF(A2), FF(A2 + 16), 64, nullptr), PTI_ERR_OVERLAP);
    // row counts that overflow a sum: rejected, with no signed overflow on the way
    const int64_t Rbig[3] = {INT64_MAX, INT64_MAX, INT64_MAX};
    EXPECT(pti_gemv_q8_multi_grouped(ws, Rbig, 3, FF(A1), FF(A2), 64, 1, nullptr), PTI_ERR_SHAPE);
    EXPECT(pti_gemv_ssq_grouped(ws, Rbig, 3, FF(A1), FF(A1), FF(A2), FF(A3), 64, nullptr), PTI_ERR_SHAPE);
    // verify
    const int32_t *ti = reinterpret_cast<const int32_t *>(A1);
    EXPECT(pti_verify_argmax(nullptr, ti, reinterpret_cast<int32_t *>(A2), reinterpret_cast<int32_t *>(A3), 100, 2,
                             nullptr), PTI_ERR_NULL);
    EXPECT(pti_verify_argmax(FF(A0), ti, reinterpret_cast<int32_t *>(A2), reinterpret_cast<int32_t *>(A3), 0, 2,
                             nullptr), PTI_ERR_SHAPE);
    EXPECT(pti_verify_argmax(FF(A0), ti, reinterpret_cast<int32_t *>(A2), reinterpret_cast<int32_t *>(A3), 100, 5,
                             nullptr), PTI_ERR_NSTREAMS);
    EXPECT(pti_verify_argmax(FF(A0), ti, reinterpret_cast<int32_t *>(A2 + 2), reinterpret_cast<int32_t *>(A3), 100, 2,
                             nullptr), PTI_ERR_ALIGN);
    EXPECT(pti_verify_argmax(FF(A0), ti, reinterpret_cast<int32_t *>(A2), reinterpret_cast<int32_t *>(A2 + 4), 100, 2,
                             nullptr), PTI_ERR_OVERLAP);
    // sampled verify
    const double *u = reinterpret_cast<const double *>(A2);
    int32_t *to = reinterpret_cast<int32_t *>(A3);
    int32_t *ao = reinterpret_cast<int32_t *>(A4);
    CHECK(pti_sample_verify_workspace_bytes(100, 2) == 32 && pti_sample_verify_workspace_bytes(0, 1) == 0);
    EXPECT(pti_sample_verify(FF(A0), ti, nullptr, 0.7, to, ao, 100, 2, F(A4 + 0x1000), 32, nullptr), PTI_ERR_NULL);
    EXPECT(pti_sample_verify(FF(A0), ti, u, 0.0, to, ao, 100, 2, F(A4 + 0x1000), 32, nullptr), PTI_ERR_SHAPE);
    EXPECT(pti_sample_verify(FF(A0), ti, u, NAN, to, ao, 100, 2, F(A4 + 0x1000), 32, nullptr), PTI_ERR_SHAPE);
    EXPECT(pti_sample_verify(FF(A0), ti, u, 0.7, to, ao, 100, 5, F(A4 + 0x1000), 32, nullptr), PTI_ERR_NSTREAMS);
    EXPECT(pti_sample_verify(FF(A0), ti, u, 0.7, to, ao, 100, 2, F(A4 + 0x1000), 31, nullptr), PTI_ERR_SHAPE);
    EXPECT(pti_sample_verify(FF(A0), ti, u, 0.7, reinterpret_cast<int32_t *>(A2 + 8), ao, 100, 2, F(A4 + 0x1000),
                             32, nullptr), PTI_ERR_OVERLAP);
    // glue
    EXPECT(pti_embed_q8(nullptr, ti, FF(A2), 100, 64, 1, nullptr), PTI_ERR_NULL);
    EXPECT(pti_embed_q8(F(A0), ti, FF(A2), 100, 48, 1, nullptr), PTI_ERR_SHAPE);
    EXPECT(pti_embed_q8(F(A0), ti, FF(A2), 100, 64, 5, nullptr), PTI_ERR_NSTREAMS);
    EXPECT(pti_embed_ssq(F(A0), ti, FF(A1 + 4), 100, 64, nullptr), PTI_ERR_OVERLAP);
    EXPECT(pti_rmsnorm(FF(A0), FF(A1), 0, 1, 1e-6f, nullptr), PTI_ERR_SHAPE);
    EXPECT(pti_rmsnorm(FF(A0), FF(A1), 64, 1, -1.0f, nullptr), PTI_ERR_SHAPE);
    EXPECT(pti_rmsnorm(FF(A0), FF(A1), 64, 0, 1e-6f, nullptr), PTI_ERR_NSTREAMS);
    EXPECT(pti_rmsnorm(FF(A0), FF(A0 + 4), 64, 1, 1e-6f, nullptr), PTI_ERR_OVERLAP);
    EXPECT(pti_silu_mul(FF(A0), FF(A1), FF(A0 + 4), 64, nullptr), PTI_ERR_OVERLAP);
    EXPECT(pti_silu_mul(FF(A0), FF(A1 + 2), FF(A2), 64, nullptr), PTI_ERR_ALIGN);
    EXPECT(pti_add(nullptr, FF(A1), FF(A2), 64, nullptr), PTI_ERR_NULL);
    EXPECT(pti_add(FF(A0), FF(A1), FF(A1 + 8), 64, nullptr), PTI_ERR_OVERLAP);
    // attention
    CHECK(pti_attn_workspace_bytes(0, 8, 2, 128, 16) == 0 && pti_attn_workspace_bytes(1, 8, 2, 96, 16) == 0);
    uint16_t *kp[1] = {reinterpret_cast<uint16_t *>(0x70000000)}, *vp[1] = {reinterpret_cast<uint16_t *>(0x71000000)};
    uint16_t *kbad[1] = {reinterpret_cast<uint16_t *>(0x70000008)};
    const int32_t *pos = reinterpret_cast<const int32_t *>(A3);
    EXPECT(pti_attn_decode(nullptr, FF(A1), FF(A2), kp, vp, pos, FF(A4), 1, 8, 2, 64, 16, F(0x72000000), 1 << 20,
                           nullptr), PTI_ERR_NULL);
    EXPECT(pti_attn_decode(FF(A0), FF(A1), FF(A2), kp, vp, pos, FF(A4), 0, 8, 2, 64, 16, F(0x72000000), 1 << 20,
                           nullptr), PTI_ERR_NSTREAMS);
    EXPECT(pti_attn_decode(FF(A0), FF(A1), FF(A2), kp, vp, pos, FF(A4), 1, 8, 2, 96, 16, F(0x72000000), 1 << 20,
                           nullptr), PTI_ERR_SHAPE);
    EXPECT(pti_attn_decode(FF(A0), FF(A1), FF(A2), kbad, vp, pos, FF(A4), 1, 8, 2, 64, 16, F(0x72000000), 1 << 20,
                           nullptr), PTI_ERR_ALIGN);
    EXPECT(pti_attn_decode(FF(A0), FF(A1), FF(A2), kp, vp, pos, FF(A0 + 64), 1, 8, 2, 64, 16, F(0x72000000), 1 << 20,
                           nullptr), PTI_ERR_OVERLAP);
    // toy stack
    const void *lay[2] = {F(A0), F(A0)};
    pti_toy_model m{PTI_FMT_Q8, 2, 64, 96, 100, 1e-6f, F(A0), F(A0), lay, lay, lay};
    const size_t n = pti_toy_workspace_bytes(&m, 4);
    CHECK(n > 0 && pti_toy_workspace_bytes(&m, 5) == 0 && pti_toy_workspace_bytes(nullptr, 1) == 0);
    pti_toy_model bad = m;
    bad.hidden = 48;
    CHECK(pti_toy_workspace_bytes(&bad, 1) == 0);
    bad = m;
    bad.n_layers = 65;
    CHECK(pti_toy_workspace_bytes(&bad, 1) == 0);
    EXPECT(pti_toy_forward(nullptr, ti, FF(A2), F(A3), n, 4, nullptr), PTI_ERR_NULL);
    EXPECT(pti_toy_forward(&m, ti, FF(A2), F(A3), n - 1, 4, nullptr), PTI_ERR_SHAPE);
    EXPECT(pti_toy_forward(&m, ti, FF(A2), F(A3 + 16), n, 4, nullptr), PTI_ERR_ALIGN);
    EXPECT(pti_toy_forward(&m, ti, FF(A3 + 512), F(A3), n, 4, nullptr), PTI_ERR_OVERLAP);
    int32_t hbuf[64];
    int64_t npass = -1;
    EXPECT(pti_toy_decode(&m, -1, 4, 5, 0.0, nullptr, F(A3), n, hbuf, hbuf, nullptr, &npass, nullptr), PTI_ERR_SHAPE);
    EXPECT(pti_toy_decode(&m, 3, 4, 5, 0.7, nullptr, F(A3), n, hbuf, hbuf, nullptr, &npass, nullptr), PTI_ERR_NULL);
    EXPECT(pti_toy_decode(&m, 3, 4, 5, NAN, nullptr, F(A3), n, hbuf, hbuf, nullptr, &npass, nullptr), PTI_ERR_SHAPE);
    CHECK(npass == -1);
    void *graph = nullptr;
    EXPECT(pti_toy_forward_graph(nullptr, ti, FF(A2), F(A3), n, 1, &graph), PTI_ERR_NULL);
    CHECK(graph == nullptr);
    EXPECT(pti_graph_launch(nullptr, nullptr), PTI_ERR_NULL);
    EXPECT(pti_graph_destroy(nullptr), PTI_OK);
}

// The oracle on small inputs: binary16 decode of every pattern against its
// definition, the GEMVs against a direct double loop, argmax and verify.
static void oracle_checks()
{
    for (uint32_t h = 0; h < 65536; h++) {
        const int s = h >> 15, e = (h >> 10) & 31, f = h & 1023;
        const double v = orc_f16_to_f64((uint16_t)h);
        double want = e == 0 ? std::ldexp((double)f, -24) : e == 31 ? (f ? NAN : INFINITY) : std::ldexp(1.0 + f / 1024.0, e - 15);
        want = s ? -want : want;
        CHECK(std::isnan(want) ? std::isnan(v) : (v == want && std::signbit(v) == std::signbit(want)));
    }
    const int64_t rows = 5, cols = 96, nb = cols / 32;
    std::vector<int8_t> a(rows * cols), b(rows * cols);
    std::vector<uint16_t> sa(rows * nb), sb(rows * nb);
    for (auto &v : a) v = (int8_t)(rnd() & 0xFF);
    for (auto &v : b) v = (int8_t)(rnd() & 0xFF);
    for (auto &v : sa) v = (uint16_t)(rnd() % 0x7C00);
    for (auto &v : sb) v = (uint16_t)(rnd() % 0x7C00);
    a[3] = -128;
    std::vector<float> xa(cols), xb(cols);
    for (auto &v : xa) v = (float)((int)(rnd() % 2001) - 1000) / 37.0f;
    for (auto &v : xb) v = (float)((int)(rnd() % 2001) - 1000) / 53.0f;
    std::vector<uint8_t> p(rows * nb * 68), q(rows * nb * 34);
    orc_pack_ssq(a.data(), b.data(), sa.data(), sb.data(), rows, cols, p.data());
    orc_pack_q8(a.data(), sa.data(), rows, cols, q.data());
    std::vector<double> ya(rows), yb(rows), ta(rows), tb(rows), y(rows), t(rows);
    orc_gemv_ssq(p.data(), rows, cols, xa.data(), xb.data(), ya.data(), yb.data(), ta.data(), tb.data());
    orc_gemv_q8(q.data(), rows, cols, xa.data(), 1, y.data(), t.data());
    for (int64_t r = 0; r < rows; r++) {
        double wa = 0, wb = 0, aa = 0;
        for (int64_t c = 0; c < cols; c++) {
            const double da = orc_f16_to_f64(sa[r * nb + c / 32]) * a[r * cols + c] * xa[c];
            const double db = orc_f16_to_f64(sb[r * nb + c / 32]) * b[r * cols + c] * xb[c];
            wa += da, wb += db, aa += std::fabs(da);
        }
        CHECK(std::fabs(ya[r] - wa) <= 1e-12 * aa && std::fabs(y[r] - ya[r]) <= 1e-12 * aa);
        CHECK(std::fabs(ta[r] - aa) <= 1e-12 * aa && std::fabs(yb[r] - wb) <= 1e-9 * (std::fabs(wb) + tb[r]));
    }
    const float v[6] = {1.f, 3.f, 3.f, -0.f, 0.f, 2.f};
    CHECK(orc_argmax(v, 6) == 1 && orc_argmax(v + 3, 2) == 0);
    const int32_t am[4] = {1, 2, 0, 1};
    int32_t tin[4] = {9, 1, 2, 5};
    CHECK(orc_accept_count(tin, am, 4) == 3);
    tin[1] = 7;
    CHECK(orc_accept_count(tin, am, 4) == 1 && orc_accept_count(tin, am, 1) == 1);
    float lg[2 * 5] = {0, 1, 5, 5, 2, -1, -2, -3, -0.5f, -0.5f};
    int32_t out[2];
    const int32_t tk[2] = {0, 2};
    CHECK(orc_verify_argmax(lg, tk, out, 5, 2) == 2 && out[0] == 2 && out[1] == 3);
}

int main()
{
    packer(1, 32, false);
    packer(3, 96, false);
    packer(7, 160, false);
    packer(33, 1024, false);
    packer(5, 5632, false);
    packer(256, 8192, true);  // 65536 blocks: every binary16 pattern in each twin's scales
    packer(1024, 5120, false);  // the threaded path
    std::printf("packer: %d checks, %d failed\n", g_checks, g_fail);
    packer_errors();
    device_errors();
    std::printf("argument errors: %d checks, %d failed\n", g_checks, g_fail);
    oracle_checks();
    std::printf("oracle: %d checks, %d failed\n", g_checks, g_fail);
    std::printf(g_fail ? "FAILED\n" : "ALL OK\n");
    return g_fail ? 1 : 0;
}

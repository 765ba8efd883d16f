// Host-side part of libpti: status codes and the SSQ / Q8 block packer.
//
// Block formats [Digest = "Packed Twin Inference：无需草稿模型的推测解码新方案，
// 实现2倍吞吐量提升", section "PTI的核心创新：SSQ打包技术" (SSQ packing);
// README = "打包双子推理（PTI）", section "与 SSQ（Side-by-Side Quantization）的关系"]:
//   SSQ block (68 B): f16 scale of twin A, f16 scale of twin B, then 32 uint16
//   slots, each holding twin A's int8 in its high byte and twin B's in its low
//   byte (little-endian memory, so the B byte comes first).
//   Q8 block (34 B): f16 scale, then 32 int8.
// Large matrices are packed with rows split across std::thread workers.
#include <algorithm>
#include <cstring>
#include <thread>
#include <vector>

#include "pti_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int kSsqBytes = PTI_SSQ_BLOCK_BYTES;
constexpr int kQ8Bytes = PTI_Q8_BLOCK_BYTES;

// Runs fn(r0, r1) over [0, rows) split across hardware threads when the matrix
// is big enough to pay for them.
template <class Fn>
void for_rows(int64_t rows, int64_t cols, Fn fn)
{
    const int64_t work = rows * cols;
    unsigned hw = std::max(1u, std::thread::hardware_concurrency());
    unsigned nt = work < (int64_t(1) << 22) ? 1u : std::min<unsigned>(hw, 32u);
    nt = unsigned(std::min<int64_t>(nt, rows));
    if (nt <= 1) {
        fn(int64_t(0), rows);
        return;
    }
    std::vector<std::thread> th;
    th.reserve(nt);
    for (unsigned t = 0; t < nt; t++) {
        int64_t r0 = rows * t / nt, r1 = rows * (t + 1) / nt;
        th.emplace_back([=] { fn(r0, r1); });
    }
    for (auto &t : th)
        t.join();
}

inline void put_u16(uint8_t *p, uint16_t v)
{
    p[0] = uint8_t(v);
    p[1] = uint8_t(v >> 8);
}
inline uint16_t get_u16(const uint8_t *p) { return uint16_t(p[0]) | uint16_t(p[1]) << 8; }

int check_host(const void *a, const void *b, const void *c, const void *d, const void *e, int64_t rows,
               int64_t cols)
{
    if (!a || !b || !c || !d || !e)
        return PTI_ERR_NULL;
    if (!pti::shape_ok(rows, cols))
        return PTI_ERR_SHAPE;
    return PTI_OK;
}

const uint8_t kDummy = 0;

}  // namespace

namespace pti {
void set_hip_error(int err) { g_last_hip_error = err; }
}  // namespace pti

extern "C" {

const char *pti_status_str(int status)
{
    switch (status) {
    case PTI_OK: return "ok";
    case PTI_ERR_NULL: return "null pointer";
    case PTI_ERR_SHAPE: return "invalid shape (rows >= 1, 32 <= cols <= 2^24, cols % 32 == 0, vocab >= 1)";
    case PTI_ERR_NSTREAMS: return "n_streams must be in [1, 4]";
    case PTI_ERR_ALIGN: return "misaligned pointer (weights 4 B, activations 16 B, others 4 B)";
    case PTI_ERR_HIP: return "HIP runtime error";
    case PTI_ERR_OVERLAP: return "output buffer overlaps an input or another output";
    default: return "unknown status";
    }
}

int pti_last_hip_error(void) { return g_last_hip_error; }

int pti_abi_version(void) { return 1; }

size_t pti_ssq_bytes(int64_t rows, int64_t cols)
{
    return pti::shape_ok(rows, cols) ? size_t(rows) * size_t(cols / PTI_BLOCK) * kSsqBytes : 0;
}

size_t pti_q8_bytes(int64_t rows, int64_t cols)
{
    return pti::shape_ok(rows, cols) ? size_t(rows) * size_t(cols / PTI_BLOCK) * kQ8Bytes : 0;
}

int pti_pack_ssq(const int8_t *a, const int8_t *b, const uint16_t *scale_a, const uint16_t *scale_b,
                 int64_t rows, int64_t cols, uint8_t *out)
{
    if (int st = check_host(a, b, scale_a, scale_b, out, rows, cols))
        return st;
    const int64_t nb = cols / PTI_BLOCK;
    for_rows(rows, cols, [&](int64_t r0, int64_t r1) {
        for (int64_t r = r0; r < r1; r++) {
            const uint8_t *ra = reinterpret_cast<const uint8_t *>(a + r * cols);
            const uint8_t *rb = reinterpret_cast<const uint8_t *>(b + r * cols);
            uint8_t *dst = out + r * nb * kSsqBytes;
            for (int64_t k = 0; k < nb; k++, dst += kSsqBytes, ra += PTI_BLOCK, rb += PTI_BLOCK) {
                put_u16(dst, scale_a[r * nb + k]);
                put_u16(dst + 2, scale_b[r * nb + k]);
                // interleave: memory order per slot is (B byte, A byte)
                for (int j = 0; j < PTI_BLOCK; j++) {
                    dst[4 + 2 * j] = rb[j];
                    dst[5 + 2 * j] = ra[j];
                }
            }
        }
    });
    return PTI_OK;
}

int pti_unpack_ssq(const uint8_t *in, int64_t rows, int64_t cols, int8_t *a, int8_t *b,
                   uint16_t *scale_a, uint16_t *scale_b)
{
    if (!in)
        return PTI_ERR_NULL;
    if (int st = check_host(a, b, scale_a, scale_b, in, rows, cols))
        return st;
    const int64_t nb = cols / PTI_BLOCK;
    for_rows(rows, cols, [&](int64_t r0, int64_t r1) {
        for (int64_t r = r0; r < r1; r++) {
            const uint8_t *src = in + r * nb * kSsqBytes;
            uint8_t *ra = reinterpret_cast<uint8_t *>(a + r * cols);
            uint8_t *rb = reinterpret_cast<uint8_t *>(b + r * cols);
            for (int64_t k = 0; k < nb; k++, src += kSsqBytes, ra += PTI_BLOCK, rb += PTI_BLOCK) {
                scale_a[r * nb + k] = get_u16(src);
                scale_b[r * nb + k] = get_u16(src + 2);
                for (int j = 0; j < PTI_BLOCK; j++) {
                    rb[j] = src[4 + 2 * j];
                    ra[j] = src[5 + 2 * j];
                }
            }
        }
    });
    return PTI_OK;
}

int pti_pack_q8(const int8_t *q, const uint16_t *scale, int64_t rows, int64_t cols, uint8_t *out)
{
    if (int st = check_host(q, scale, out, &kDummy, &kDummy, rows, cols))
        return st;
    const int64_t nb = cols / PTI_BLOCK;
    for_rows(rows, cols, [&](int64_t r0, int64_t r1) {
        for (int64_t r = r0; r < r1; r++) {
            uint8_t *dst = out + r * nb * kQ8Bytes;
            const int8_t *src = q + r * cols;
            for (int64_t k = 0; k < nb; k++, dst += kQ8Bytes, src += PTI_BLOCK) {
                put_u16(dst, scale[r * nb + k]);
                std::memcpy(dst + 2, src, PTI_BLOCK);
            }
        }
    });
    return PTI_OK;
}

int pti_unpack_q8(const uint8_t *in, int64_t rows, int64_t cols, int8_t *q, uint16_t *scale)
{
    if (int st = check_host(in, q, scale, &kDummy, &kDummy, rows, cols))
        return st;
    const int64_t nb = cols / PTI_BLOCK;
    for_rows(rows, cols, [&](int64_t r0, int64_t r1) {
        for (int64_t r = r0; r < r1; r++) {
            const uint8_t *src = in + r * nb * kQ8Bytes;
            int8_t *dst = q + r * cols;
            for (int64_t k = 0; k < nb; k++, src += kQ8Bytes, dst += PTI_BLOCK) {
                scale[r * nb + k] = get_u16(src);
                std::memcpy(dst, src + 2, PTI_BLOCK);
            }
        }
    });
    return PTI_OK;
}

int pti_ssq_split(const uint8_t *ssq, int64_t rows, int64_t cols, uint8_t *q8_a, uint8_t *q8_b)
{
    if (int st = check_host(ssq, q8_a, q8_b, &kDummy, &kDummy, rows, cols))
        return st;
    const size_t ns = pti_ssq_bytes(rows, cols), nq = pti_q8_bytes(rows, cols);
    if (pti::overlap({ssq, ns}, {q8_a, nq}) || pti::overlap({ssq, ns}, {q8_b, nq}) ||
        pti::overlap({q8_a, nq}, {q8_b, nq}))
        return PTI_ERR_OVERLAP;
    const int64_t nblk = rows * (cols / PTI_BLOCK);
    for_rows(nblk, PTI_BLOCK, [&](int64_t b0, int64_t b1) {
        for (int64_t k = b0; k < b1; k++) {
            const uint8_t *s = ssq + k * kSsqBytes;
            uint8_t *qa = q8_a + k * kQ8Bytes, *qb = q8_b + k * kQ8Bytes;
            qa[0] = s[0], qa[1] = s[1];
            qb[0] = s[2], qb[1] = s[3];
            for (int j = 0; j < PTI_BLOCK; j++) {
                qb[2 + j] = s[4 + 2 * j];
                qa[2 + j] = s[5 + 2 * j];
            }
        }
    });
    return PTI_OK;
}

int pti_ssq_join(const uint8_t *q8_a, const uint8_t *q8_b, int64_t rows, int64_t cols, uint8_t *ssq)
{
    if (int st = check_host(q8_a, q8_b, ssq, &kDummy, &kDummy, rows, cols))
        return st;
    const size_t ns = pti_ssq_bytes(rows, cols), nq = pti_q8_bytes(rows, cols);
    if (pti::overlap({ssq, ns}, {q8_a, nq}) || pti::overlap({ssq, ns}, {q8_b, nq}))
        return PTI_ERR_OVERLAP;
    const int64_t nblk = rows * (cols / PTI_BLOCK);
    for_rows(nblk, PTI_BLOCK, [&](int64_t b0, int64_t b1) {
        for (int64_t k = b0; k < b1; k++) {
            uint8_t *s = ssq + k * kSsqBytes;
            const uint8_t *qa = q8_a + k * kQ8Bytes, *qb = q8_b + k * kQ8Bytes;
            s[0] = qa[0], s[1] = qa[1];
            s[2] = qb[0], s[3] = qb[1];
            for (int j = 0; j < PTI_BLOCK; j++) {
                s[4 + 2 * j] = qb[2 + j];
                s[5 + 2 * j] = qa[2 + j];
            }
        }
    });
    return PTI_OK;
}

}  // extern "C"

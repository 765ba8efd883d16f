// Decode attention over per-stream binary16 KV caches, for the twin decode.
//
// [Digest = "Packed Twin Inference：无需草稿模型的推测解码新方案，实现2倍吞吐量
// 提升", section "技术实现架构" (implementation architecture)]: twins A and B
// keep separate KV caches; one pass serves both streams; an accept extends
// B's cache and a reject resets B's state.  [Notes = the LLM-inference page,
// section "从朴素推理到 KV cache" (from naive inference to the KV cache)]: a
// decode step appends the new token's key and value and attends over the
// cache.
//
// Per stream s (independent caches, one query per head):
//   store  K_s[g][pos_s] = f16(k_new[s][g]), V_s[g][pos_s] = f16(v_new[s][g])
//          (round to nearest even), replacing what was there: a reject's
//          redraw at the same position overwrites the stale entry;
//   attend out[s][h] = sum_{j <= pos_s} softmax_j(q[s][h] . K_s[g][j] / sqrt(d)) V_s[g][j],
//          g = h / (n_heads / n_kv_heads) (grouped heads share a kv head).
//
// Mapped onto CDNA4 as a split-K "flash decode" with both products on the
// matrix cores (v_mfma_f32_16x16x32_f16):
//   * Pass 1, one workgroup of 256 threads per (key chunk of 128, kv head,
//     stream); each of its four waves owns 32 consecutive keys.  Cache rows
//     are read whole: d/8 lanes cover a row with 16-byte loads, so a load
//     instruction of a wave reads 64 / (d/8) consecutive rows as one
//     contiguous span, and all of a wave's K loads are in flight together
//     (its V loads follow once the scores are issued).  A wave's rows go to
//     its own LDS rows; the new entry, rounded as it is stored, replaces the
//     row at pos_s there.
//     Scores: the wave multiplies its 32 keys (16 per MFMA row block) by the
//     group's queries.  q is split exactly enough for fp32: per head it is
//     scaled by a power of two so that max |q| lies in [2^14, 2^15), then
//     written as a high binary16 part plus a low one (22 bits in all);
//     MFMA column 2h holds head h's high part and column 2h + 1 its low
//     part, and a DPP swap of neighbouring lanes adds the two.  Products of
//     binary16 values are exact in fp32, so the only roundings are the
//     accumulation's.  A key is read once for all heads that share it.
//     Softmax: the wave's max per head in registers, the chunk's max over
//     the four waves through LDS (the first barrier); the weights, in units
//     of 2^-15 (exact, so both of their binary16 parts stay normal), stay in
//     the lanes that computed them, which are already where the next
//     product's A operand needs them.
//     Weighted V: rows = head parts (row 2h high, 2h + 1 low), k = the
//     wave's 32 keys, columns = 16 dimensions read transposed from the
//     wave's V rows in LDS (ds_read_b64_tr_b16); each head's two rows sit in
//     one lane and are added there.  The four waves' weighted V meet in LDS
//     (the second barrier) and are added in wave order; the chunk's (max,
//     exp-sum, weighted V) per head go to the workspace.  The chunk holding
//     pos_s stores the new entry.
//   * Pass 2, one workgroup per (head, stream, 32 dimensions): the chunks up
//     to pos_s combine, rescaled by exp(m_c - M), in a fixed grouping of
//     chunks.
// Every sum runs in a fixed order that depends on the shapes and pos_s only.
// Chunks past a stream's position exit at once; the grid covers max_len so
// positions can live in device memory (capturable in a graph).
#include <hip/hip_runtime.h>

#include <cmath>

#include "pti_internal.h"

namespace {

constexpr int kChunk = 128;     // keys per pass-1 workgroup
constexpr int kThreads = 256;
constexpr int kMaxGroup = 8;    // query heads per kv head

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

struct AttnArgs {
    const float *q;       // [S][H][d]
    const float *k_new;   // [S][Hkv][d]
    const float *v_new;
    uint16_t *kc[PTI_MAX_STREAMS];  // [Hkv][max_len][d] binary16
    uint16_t *vc[PTI_MAX_STREAMS];
    const int32_t *pos;   // [S]
    float *out;           // [S][H][d]
    float *part;          // [S][H][n_chunks][d]: weighted V per chunk
    float *ml;            // [S][H][n_chunks][2]: max, exp-sum per chunk (after part)
    int H, Hkv, n_chunks;
    int64_t max_len;
    float scale;          // 1 / sqrt(d)
};

__device__ __forceinline__ uint16_t f2h(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }

// The value DPP moves into each lane under control CTRL (rows in ROW_MASK);
// lanes it does not write get `id`.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_or(float v, float id)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, id), __builtin_bit_cast(int, v),
                                                                 CTRL, ROW_MASK, 0xf, false));
}

// Max over the 64 lanes, in lane 63: a fixed DPP tree (row shifts by 1, 2,
// 4, 8, then the row broadcasts of lanes 15 and 31).
__device__ __forceinline__ float wave_max(float v)
{
    v = fmaxf(v, dpp_or<0x111, 0xf>(v, -INFINITY));
    v = fmaxf(v, dpp_or<0x112, 0xf>(v, -INFINITY));
    v = fmaxf(v, dpp_or<0x114, 0xf>(v, -INFINITY));
    v = fmaxf(v, dpp_or<0x118, 0xf>(v, -INFINITY));
    v = fmaxf(v, dpp_or<0x142, 0xa>(v, -INFINITY));
    v = fmaxf(v, dpp_or<0x143, 0xc>(v, -INFINITY));
    return v;
}

// Position of stream s, or -1 when outside the cache (the pass then writes
// NaN outputs and touches no cache memory).
__device__ __forceinline__ int64_t stream_pos(const AttnArgs &a, int s)
{
    const int64_t p = a.pos[s];
    return (p >= 0 && p < a.max_len) ? p : -1;
}

// 8 consecutive fp32 values (two float4) rounded to binary16, packed as they
// are stored.
__device__ __forceinline__ u32x4 pack8(float4 a, float4 b)
{
    return u32x4{(uint32_t)f2h(a.x) | ((uint32_t)f2h(a.y) << 16), (uint32_t)f2h(a.z) | ((uint32_t)f2h(a.w) << 16),
                 (uint32_t)f2h(b.x) | ((uint32_t)f2h(b.y) << 16), (uint32_t)f2h(b.z) | ((uint32_t)f2h(b.w) << 16)};
}

// c ? a : b by bit masks, so the compiler cannot move b's load into a branch
// (which would reorder the loads and make the first wait cover all of them).
__device__ __forceinline__ u32x4 pick(bool c, u32x4 a, u32x4 b)
{
    const uint32_t m = c ? 0xFFFFFFFFu : 0u;
    return (a & m) | (b & ~m);
}

// Max over the four 16-lane rows of a wave, per column (lane % 16), in every
// lane.
__device__ __forceinline__ float col_max(float v)
{
    v = fmaxf(v, __shfl_xor(v, 16, 64));
    return fmaxf(v, __shfl_xor(v, 32, 64));
}

// Pass 1.  Each wave owns 32 consecutive keys of the chunk and takes them
// through scores, softmax numerators and the weighted V on its own; the
// workgroup meets twice: for the chunk max of each head, and to add the four
// waves' weighted V.  The V rows are loaded once the scores are issued: with
// them in flight from the start the K rows arrived later (every chunk's K
// and V compete for HBM at once) and the registers allowed three waves per
// SIMD instead of four; both were slower, at 4K and at 32K positions.
template <int D, int G>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void attn_partial_kernel(AttnArgs a)
{
    static_assert(G >= 1 && G <= 8, "the high and low parts of at most 8 heads fill the 16 MFMA columns");
    constexpr int LPR = D / 8;                  // lanes per cache row: 16 bytes (8 halves) each
    constexpr int RPI = 64 / LPR;               // rows one load instruction of a wave covers
    constexpr int NW = kThreads / 64;
    constexpr int KPW = kChunk / NW;            // keys per wave
    constexpr int IT = KPW / RPI;               // loads per wave per tile
    constexpr int KSTEPS = D / 32;              // MFMA steps over the dimensions (scores)
    constexpr int NB = D / 16;                  // 16-dimension output blocks (weighted V)
    // LDS row pitch of the K and V rows, bytes: 8 banks (of 64) past a row's
    // length, so the K operand reads (8 lanes per cycle, 16 B each, one row
    // apiece) and the transposed V reads (16 lanes, 8 B each, over 4 rows) of a
    // cycle all fall in different banks
    constexpr int PITCH = 2 * D + 32;
    constexpr int OWP = D + 8;                  // park pitch per head, floats: the four k groups' heads
                                                // (2 apart) land 16 banks apart
    static_assert(KPW == 32, "tile shape");
    static_assert(G * OWP * 4 <= KPW * PITCH, "a wave's weighted V fits its own rows' LDS");
    // per wave: its 32 K rows, then its 32 V rows, then its weighted V [G][D]
    __shared__ __attribute__((aligned(16))) uint8_t tile[kChunk * PITCH];
    __shared__ float wred[2][NW][8];  // per wave and head: max, then exp-sum
    const int c = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t pos = stream_pos(a, s);
    if (pos < 0 || (int64_t)c * kChunk > pos)
        return;  // nothing of this stream in this chunk
    const int64_t j0 = (int64_t)c * kChunk;
    const int nk = (int)min<int64_t>(kChunk, pos + 1 - j0);  // keys in this chunk
    const bool has_new = pos < j0 + kChunk;                  // the new entry is in this chunk
    const uint16_t *K = a.kc[s] + ((size_t)g * a.max_len) * D;
    const uint16_t *V = a.vc[s] + ((size_t)g * a.max_len) * D;
    const float *kn = a.k_new + ((size_t)s * a.Hkv + g) * D;
    const float *vn = a.v_new + ((size_t)s * a.Hkv + g) * D;
    const int r = lane / LPR, seg = lane % LPR;  // row within a load, 8-dimension segment
    const int n = lane & 15, kg = lane >> 4;     // MFMA column / row (lane % 16) and k group (lane / 16)
    uint8_t *rows = tile + wv * KPW * PITCH;     // this wave's rows

    // ---- loads.  A wave's loads return in order, so the order they are
    // issued in sets what each step waits for: the new entry's and q's few
    // bytes first (no branch: every workgroup's k_new, v_new and q rows
    // exist), then the wave's K rows (its V rows follow the scores).  Rows are read
    // whole and in order (LPR lanes x 16 bytes) through buffer resources over
    // the chunk's valid rows (rows past them read 0 without a branch).
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(K + (size_t)j0 * D), (short)0, nk * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(V + (size_t)j0 * D), (short)0, nk * D * 2, 0x00020000);
    const int newkey = has_new ? (int)(pos - j0) : -1;  // chunk index of the new entry
    const float4 *knp = reinterpret_cast<const float4 *>(kn + 8 * seg);
    const float4 *vnp = reinterpret_cast<const float4 *>(vn + 8 * seg);
    const float4 kn0 = knp[0], kn1 = knp[1], vn0 = vnp[0], vn1 = vnp[1];
    const int hq = n >> 1;  // the head of MFMA column (and row) n; n & 1 picks its part
    const float4 *qrow = reinterpret_cast<const float4 *>(
        a.q + ((size_t)s * a.H + (size_t)g * G + (hq < G ? hq : 0)) * D + 8 * kg);
    float4 qv[KSTEPS][2];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ks++)
#pragma unroll
        for (int e4 = 0; e4 < 2; e4++)
            qv[ks][e4] = qrow[8 * ks + e4];
    u32x4 kt[IT], vt[IT];
#pragma unroll
    for (int it = 0; it < IT; it++)
        kt[it] = __builtin_amdgcn_raw_buffer_load_b128(krs, ((wv * KPW + it * RPI + r) * D + 8 * seg) * 2, 0, 0);
    __builtin_amdgcn_sched_barrier(0);  // keep the loads above issued first, in this order
    const u32x4 kn8 = pack8(kn0, kn1), vn8 = pack8(vn0, vn1);  // used only where has_new

    // ---- q as the MFMA's B operand: column 2h holds the high binary16 part
    // of head h, column 2h + 1 the low part (q' - high), for the k group's 8
    // dimensions per step.  q' = q 2^sh with sh chosen per head so that
    // max |q'| lies in [2^14, 2^15): both parts stay normal (or exactly
    // representable) and high + low carries 22 bits of each element.
    // Columns past the group's heads get zeros (a mask, not a branch).
    const uint32_t keep = hq < G ? 0xFFFFFFFFu : 0u;
    float qf[KSTEPS][8];
    float qmax = 0.f;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ks++)
#pragma unroll
        for (int e4 = 0; e4 < 2; e4++) {
            const float4 t = qv[ks][e4];
            const float e[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const float x = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, e[j]) & keep);
                qf[ks][4 * e4 + j] = x;
                qmax = fmaxf(qmax, fabsf(x));
            }
        }
    qmax = col_max(qmax);  // over the four k groups: the head's max |q|
    const int sh = qmax > 0.f ? 15 - __builtin_amdgcn_frexp_expf(qmax) : 0;
    f16x8 qb[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ks++)
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const float x = ldexpf(qf[ks][e], sh);
            const _Float16 hi = (_Float16)x;
            qb[ks][e] = (n & 1) ? (_Float16)(x - (float)hi) : hi;
        }

    // ---- the wave's 32 K rows to its LDS rows (the new entry, rounded as it
    // is stored, replaces the row at pos), then the scores on the matrix
    // cores: rows = keys (A, 16 per block), columns = head parts (B)
#pragma unroll
    for (int it = 0; it < IT; it++) {
        const int kk = it * RPI + r;
        *reinterpret_cast<u32x4 *>(rows + kk * PITCH + 16 * seg) = pick(wv * KPW + kk == newkey, kn8, kt[it]);
    }
    // the wave reads rows other lanes wrote: LDS serves a wave's accesses in
    // order, and the fence keeps the compiler from moving reads above writes
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    f32x4 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
        sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ks++) {
            const f16x8 ka = *reinterpret_cast<const f16x8 *>(rows + (16 * kb + n) * PITCH + 64 * ks + 16 * kg);
            sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qb[ks], sacc[kb], 0, 0, 0);
        }
    }
    // V rows now: their latency overlaps the softmax
#pragma unroll
    for (int it = 0; it < IT; it++)
        vt[it] = __builtin_amdgcn_raw_buffer_load_b128(vrs, ((wv * KPW + it * RPI + r) * D + 8 * seg) * 2, 0, 0);

    // ---- scores of the lane's 8 keys (wave key 16 kb + 4 kg + i) for head
    // n / 2: its column plus the partner column n ^ 1 (the other part of the
    // same head; both lanes of a pair get the same sum); keys past the
    // chunk's last get -inf.  Then the wave's max per head (over its 8
    // values, then the four k groups).
    float sc[8];
    float m = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
            // (a copy first: a bit cast of a vector element itself reads element 0)
            const float own = sacc[kb][i];
            const float other = __builtin_bit_cast(
                float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, own), 0xB1, 0xf, 0xf, false));
            const float v = ldexpf((n & 1) ? other + own : own + other, -sh) * a.scale;  // high + low
            sc[4 * kb + i] = wv * KPW + 16 * kb + 4 * kg + i < nk ? v : -INFINITY;
            m = fmaxf(m, sc[4 * kb + i]);
        }
    m = col_max(m);
    if (kg == 0 && (n & 1) == 0 && hq < G)
        wred[0][wv][hq] = m;
    __syncthreads();  // (1) every wave's max
    m = wred[0][0][hq & 7];
#pragma unroll
    for (int w = 1; w < NW; w++)
        m = fmaxf(m, wred[0][w][hq & 7]);

    // ---- weights in units of 2^-15 (exact; both binary16 parts below stay
    // normal), 0 for keys past the chunk and for columns past the heads; the
    // wave's exp-sum per head (its 8 values in order, then the k groups)
    float pw[8];
    float l = 0.f;
#pragma unroll
    for (int e = 0; e < 8; e++) {
        pw[e] = hq < G ? expf(sc[e] - m) * 32768.f : 0.f;
        l += pw[e];
    }
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (kg == 0 && (n & 1) == 0 && hq < G)
        wred[1][wv][hq] = l;

    // ---- the wave's V rows over its K rows (the scores have read them)
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int it = 0; it < IT; it++) {
        const int kk = it * RPI + r;
        *reinterpret_cast<u32x4 *>(rows + kk * PITCH + 16 * seg) = pick(wv * KPW + kk == newkey, vn8, vt[it]);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();

    // ---- weighted V of the wave's 32 keys on the matrix cores: rows = head
    // parts (A: row 2h the high binary16 part of head h's weights, row
    // 2h + 1 the low part -- lane n holds head n / 2's weights already),
    // k = the 32 keys in the scores' order (k group kg holds keys
    // 4 kg .. 4 kg + 3 and 16 + 4 kg .. 16 + 4 kg + 3), columns = 16
    // dimensions (B, read transposed from the V rows)
    f16x8 pa;
#pragma unroll
    for (int e = 0; e < 8; e++) {
        const _Float16 hi = (_Float16)pw[e];
        pa[e] = (n & 1) ? (_Float16)(pw[e] - (float)hi) : hi;
    }
    // A product's lane (column n, row group kg) holds rows 4 kg .. 4 kg + 3:
    // heads 2 kg and 2 kg + 1, high part then low part; each head's sum is
    // the wave's weighted V, parked over the wave's rows once every product
    // has read them
    float ov[NB][2];
#pragma unroll
    for (int j = 0; j < NB; j++) {
        const int col = 2 * (16 * j + 4 * (n & 3));  // byte offset of 4 dimensions
        const uint8_t *t0 = rows + (4 * kg + (n >> 2)) * PITCH + col;
        const s16x4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(t0));
        const s16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(t0 + 16 * PITCH));
        const f16x8 vb = __builtin_bit_cast(f16x8, s16x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]});
        const f32x4 o = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, vb, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        const float o0 = o[0], o1 = o[1], o2 = o[2], o3 = o[3];  // (copies first, as above)
        ov[j][0] = o0 + o1;
        ov[j][1] = o2 + o3;
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    float *ow = reinterpret_cast<float *>(rows);  // [G][OWP]
#pragma unroll
    for (int j = 0; j < NB; j++)
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const int h = 2 * kg + u;
            if (h < G)
                ow[h * OWP + 16 * j + n] = ov[j][u];
        }
    __syncthreads();  // (2) every wave's weighted V and exp-sums

    // ---- chunk partials: the four waves' weighted V added in wave order,
    // the max and exp-sum per head, all in units of 2^-15 (the combine
    // divides one by the other)
    for (int o = tid; o < G * D; o += kThreads) {
        const int h = o / D, dd = o % D;
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < NW; w++)
            v += reinterpret_cast<const float *>(tile + w * KPW * PITCH)[h * OWP + dd];
        a.part[(((size_t)s * a.H + (size_t)g * G + h) * a.n_chunks + c) * D + dd] = v;
    }
    if (tid < G) {
        float mm = wred[0][0][tid], ll = wred[1][0][tid];
#pragma unroll
        for (int w = 1; w < NW; w++)
            mm = fmaxf(mm, wred[0][w][tid]), ll += wred[1][w][tid];
        float *pp = a.ml + (((size_t)s * a.H + (size_t)g * G + tid) * a.n_chunks + c) * 2;
        pp[0] = mm;
        pp[1] = ll;
    }

    // ---- store the new entry (the chunk that holds pos; every reader of
    // this position in this pass used the rounded values above)
    if (has_new) {
        uint16_t *kd = a.kc[s] + ((size_t)g * a.max_len + pos) * D;
        uint16_t *vd = a.vc[s] + ((size_t)g * a.max_len + pos) * D;
        for (int i = tid; i < D; i += kThreads) {
            kd[i] = f2h(kn[i]);
            vd[i] = f2h(vn[i]);
        }
    }
}

// Pass 2: the chunks of (head, stream) combine, one workgroup per (head,
// stream, 32 dimensions).  The chunk maxima are read in parallel and reduced
// to M; then thread (cg, dg) sums, over chunks cg, cg + CG, ..., the 16-byte
// slice dg of the chunks' weighted V rows scaled by exp(m_c - M) (and the
// exp-sums likewise); the chunk groups add in order.
constexpr int kCombineDims = 32;

template <int D>
__global__ __launch_bounds__(kThreads) void attn_combine_kernel(AttnArgs a)
{
    constexpr int DG = kCombineDims / 4;  // float4 slices of the workgroup's dimensions
    constexpr int CG = kThreads / DG;     // chunk groups
    __shared__ float redm[kThreads / 64];
    __shared__ float4 vsum[CG][DG];
    __shared__ float lsum[CG];
    const int h = blockIdx.x, s = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int d0 = blockIdx.z * kCombineDims;
    float *o = a.out + ((size_t)s * a.H + h) * D + d0;
    const int64_t pos = stream_pos(a, s);
    if (pos < 0) {
        if (tid < kCombineDims)
            o[tid] = NAN;
        return;
    }
    const int nc = (int)(pos / kChunk) + 1;
    const float *pv = a.part + ((size_t)s * a.H + h) * a.n_chunks * D + d0;
    const float *pm = a.ml + ((size_t)s * a.H + h) * a.n_chunks * 2;
    float mx = -INFINITY;
    for (int c = tid; c < nc; c += kThreads)
        mx = fmaxf(mx, pm[2 * c]);
    mx = wave_max(mx);
    if (lane == 63)
        redm[wv] = mx;
    __syncthreads();
    float M = redm[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; w++)
        M = fmaxf(M, redm[w]);
    const int dg = tid % DG, cg = tid / DG;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float l = 0.f;
#pragma unroll 4
    for (int c = cg; c < nc; c += CG) {
        const float f = expf(pm[2 * c] - M);
        l = __builtin_fmaf(pm[2 * c + 1], f, l);
        const float4 v = reinterpret_cast<const float4 *>(pv + (size_t)c * D)[dg];
        acc.x = __builtin_fmaf(v.x, f, acc.x);
        acc.y = __builtin_fmaf(v.y, f, acc.y);
        acc.z = __builtin_fmaf(v.z, f, acc.z);
        acc.w = __builtin_fmaf(v.w, f, acc.w);
    }
    vsum[cg][dg] = acc;
    if (dg == 0)
        lsum[cg] = l;
    __syncthreads();
    if (tid < DG) {
        float4 t = vsum[0][tid];
        float L = lsum[0];
#pragma unroll
        for (int k = 1; k < CG; k++) {
            const float4 u = vsum[k][tid];
            t.x += u.x, t.y += u.y, t.z += u.z, t.w += u.w;
            L += lsum[k];
        }
        o[4 * tid] = t.x / L;
        o[4 * tid + 1] = t.y / L;
        o[4 * tid + 2] = t.z / L;
        o[4 * tid + 3] = t.w / L;
    }
}

template <int D, int G>
void launch_g(const AttnArgs &a, int S, hipStream_t st)
{
    hipLaunchKernelGGL((attn_partial_kernel<D, G>), dim3((unsigned)a.n_chunks, (unsigned)a.Hkv, (unsigned)S),
                       dim3(kThreads), 0, st, a);
    hipLaunchKernelGGL((attn_combine_kernel<D>), dim3((unsigned)a.H, (unsigned)S, (unsigned)(D / kCombineDims)),
                       dim3(kThreads), 0, st, a);
}

template <int D>
void launch_d(const AttnArgs &a, int G, int S, hipStream_t st)
{
    switch (G) {
    case 1: return launch_g<D, 1>(a, S, st);
    case 2: return launch_g<D, 2>(a, S, st);
    case 3: return launch_g<D, 3>(a, S, st);
    case 4: return launch_g<D, 4>(a, S, st);
    case 5: return launch_g<D, 5>(a, S, st);
    case 6: return launch_g<D, 6>(a, S, st);
    case 7: return launch_g<D, 7>(a, S, st);
    default: return launch_g<D, 8>(a, S, st);
    }
}

int64_t n_chunks(int64_t max_len) { return (max_len + kChunk - 1) / kChunk; }

bool attn_shape_ok(int n_streams, int n_heads, int n_kv_heads, int head_dim, int64_t max_len)
{
    return n_streams >= 1 && n_streams <= PTI_MAX_STREAMS && n_kv_heads >= 1 && n_heads >= n_kv_heads &&
           n_heads % n_kv_heads == 0 && n_heads / n_kv_heads <= kMaxGroup && n_heads <= 65535 &&
           (head_dim == 64 || head_dim == 128) && max_len >= 1 && max_len <= PTI_MAX_ATTN_LEN;
}

}  // namespace

extern "C" {

size_t pti_attn_workspace_bytes(int n_streams, int n_heads, int n_kv_heads, int head_dim, int64_t max_len)
{
    if (!attn_shape_ok(n_streams, n_heads, n_kv_heads, head_dim, max_len))
        return 0;
    return (size_t)n_streams * n_heads * (size_t)n_chunks(max_len) * ((size_t)head_dim + 2) * sizeof(float);
}

int pti_attn_decode(const float *q, const float *k_new, const float *v_new, uint16_t *const *k_cache,
                    uint16_t *const *v_cache, const int32_t *pos, float *out, int n_streams, int n_heads,
                    int n_kv_heads, int head_dim, int64_t max_len, void *work, size_t work_bytes, void *stream)
{
    if (!q || !k_new || !v_new || !k_cache || !v_cache || !pos || !out || !work)
        return PTI_ERR_NULL;
    if (n_streams < 1 || n_streams > PTI_MAX_STREAMS)
        return PTI_ERR_NSTREAMS;
    if (!attn_shape_ok(n_streams, n_heads, n_kv_heads, head_dim, max_len))
        return PTI_ERR_SHAPE;
    const size_t need = pti_attn_workspace_bytes(n_streams, n_heads, n_kv_heads, head_dim, max_len);
    if (work_bytes < need)
        return PTI_ERR_SHAPE;
    const size_t d = (size_t)head_dim, S = (size_t)n_streams;
    const size_t cache_bytes = (size_t)n_kv_heads * (size_t)max_len * d * 2;
    if (!pti::aligned(q, 4) || !pti::aligned(k_new, 4) || !pti::aligned(v_new, 4) || !pti::aligned(pos, 4) ||
        !pti::aligned(out, 4) || !pti::aligned(work, 16))
        return PTI_ERR_ALIGN;
    for (int s = 0; s < n_streams; s++) {
        if (!k_cache[s] || !v_cache[s])
            return PTI_ERR_NULL;
        if (!pti::aligned(k_cache[s], 16) || !pti::aligned(v_cache[s], 16))
            return PTI_ERR_ALIGN;
    }
    // outputs: out, work, every cache; inputs: q, k_new, v_new, pos
    const pti::Range ins[] = {{q, S * n_heads * d * 4}, {k_new, S * n_kv_heads * d * 4},
                              {v_new, S * n_kv_heads * d * 4}, {pos, S * 4}};
    pti::Range outs[2 + 2 * PTI_MAX_STREAMS];
    int no = 0;
    outs[no++] = {out, S * n_heads * d * 4};
    outs[no++] = {work, need};
    for (int s = 0; s < n_streams; s++) {
        outs[no++] = {k_cache[s], cache_bytes};
        outs[no++] = {v_cache[s], cache_bytes};
    }
    for (int i = 0; i < no; i++) {
        for (int j = i + 1; j < no; j++)
            if (pti::overlap(outs[i], outs[j]))
                return PTI_ERR_OVERLAP;
        for (const pti::Range &in : ins)
            if (pti::overlap(outs[i], in))
                return PTI_ERR_OVERLAP;
    }
    AttnArgs a{};
    a.q = q, a.k_new = k_new, a.v_new = v_new, a.pos = pos, a.out = out;
    for (int s = 0; s < n_streams; s++)
        a.kc[s] = k_cache[s], a.vc[s] = v_cache[s];
    a.H = n_heads, a.Hkv = n_kv_heads, a.n_chunks = (int)n_chunks(max_len), a.max_len = max_len;
    a.part = static_cast<float *>(work);
    a.ml = a.part + S * (size_t)n_heads * (size_t)a.n_chunks * d;
    a.scale = 1.0f / sqrtf((float)head_dim);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int G = n_heads / n_kv_heads;
    if (head_dim == 64)
        launch_d<64>(a, G, n_streams, st);
    else
        launch_d<128>(a, G, n_streams, st);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        pti::set_hip_error(e);
        return PTI_ERR_HIP;
    }
    return PTI_OK;
}

}  // extern "C"

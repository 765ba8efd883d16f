// Packed-weight decode GEMVs for gfx950: the SSQ twin GEMV (one or two
// streams per twin), the Q8 multi-stream GEMV, their grouped forms, and the
// SSQ GEMV fused with the greedy verify.
//
// Kernels.  The per-wave-row kernel below (gemv_kernel) serves Q8 matrices
// of more than 8192 rows (or of an odd block count, or more than 20 rounds)
// and SSQ rows of more than 40 rounds; the row-split kernel further down
// (gemv_ssq_split_kernel) serves the other SSQ shapes, and with VERIFY also
// keeps each workgroup's largest output per twin, which verify_keys_kernel
// then reduces; its Q8 form (gemv_q8_split_kernel) serves the other Q8
// shapes, and the tall Q8 shapes whose rows take one wave there when one or
// two streams run (where both kernels give the same bits).  A stream's result
// never depends on the stream count.  Both kernels read rows through a segment
// table (one matrix, or several with the same column count stacked into one
// row space) and can add a residual to the rows they store.
//
// What is computed [README = "打包双子推理（PTI）", section "与 SSQ（Side-by-Side
// Quantization）的关系" (relation to SSQ); section "带宽分析：为什么会有开销"
// (bandwidth analysis)]: every weight is read from HBM once per call; one SSQ
// slot feeds twin A (high byte) and twin B (low byte); one Q8 block feeds up to
// four activation vectors.  Output y[s][r] = sum_c scale(r, c/32) * q[r][c] * x[s][c].
//
// Per-wave-row kernel, mapped onto CDNA4 (gfx950: 256 CUs of 4 SIMDs, wave64,
// 160 KB LDS per CU):
//   * One workgroup per CU with a multiple of four wave64s.  Rows are dealt
//     round-robin to the SIMDs, so every SIMD gets the same number of rows (to
//     within one) whatever the row count -- no second dispatch wave, no SIMD
//     with twice the work -- and the GPU as a whole sweeps the matrix front to
//     back.  x is staged once per CU whatever the wave count.
//   * A wave owns its rows end to end: all 64 lanes share each row.  Each lane
//     owns a fixed set of columns ("units") in every row, so the activations it
//     needs are the same for all rows; R rows are computed together so each LDS
//     read of x serves R rows.
//       SSQ: 8-column units, four lanes per 68-byte block, lane q of the four
//            reading slots 8q..8q+7 -- so the four lanes' 16-byte loads cover
//            the block's 64 slot bytes contiguously (the address unit merges a
//            contiguous quad into one request; scattered 16-byte pieces cost
//            about 12% of bandwidth in measurements), plus the block's scale
//            dword.  16 blocks (1088 bytes) per round of 64 lanes.
//       Q8:  16-column units, two lanes per 34-byte block: the scale's dword and
//            the 16 quant bytes read as 4 + 1 dwords from dword-aligned
//            offsets and realigned with v_alignbyte (Q8 blocks sit at 2-byte
//            offsets half the time).  32 blocks (1088 bytes) per round.
//   * x is staged into LDS once per workgroup (per K-chunk when it does not
//     fit), never re-read from L2 per row block: the README's bandwidth analysis
//     traces the L2 thrash of its multi-stream kernel to that re-reading.  The
//     LDS layout makes each ds_read_b128 of a wave one contiguous 1 KB span.
//   * Weights are read with buffer loads through one buffer resource per row:
//     per-lane offsets are fixed, per-round offsets are scalar, and a read
//     past the row returns 0 instead of touching memory.
//   * Weight loads run D steps ahead of the compute (a step = one round of R
//     rows); every step issues the same loads (out-of-range steps through an
//     empty resource) and sched_barrier pins the order, so each wait covers
//     exactly one step.
//   * Signed bytes convert to fp32 with one SDWA v_cvt_f32_i32 each.  Per unit
//     and stream the products are summed in fp32 in column order, scaled by
//     the block's f16 scale with one FMA into the lane's accumulator, and the
//     64 lanes reduce by a fixed tree (tree_sums: all of a wave's sums in one
//     pass of DPP and lane swaps).  Finished rows park in one lane each of an
//     output register and are stored after the loop.  No MFMA: this is a
//     matrix-vector product, one FMA per weight and stream.
//   * A row's operation order depends only on (rows, cols) and the format: not
//     on the stream count, the stream's slot, R or the wave count, so a
//     stream's output is bitwise independent of those.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <utility>

#include "pti_internal.h"
#include "pti_norm.h"
#include "pti_silu.h"

// Per-wave-row kernel geometry by format and stream count: waves per
// workgroup (a multiple of 4), steps of loads in flight, rows per wave.  None
// of the three changes a row's arithmetic (they change which wave computes a
// row and when), so they may differ between stream counts; the values are
// measured optima and can be overridden at build time.
#ifndef PTI_Q8_N1_CFG
#define PTI_Q8_N1_CFG 12, 1, 1
#endif
#ifndef PTI_Q8_N2_CFG
#define PTI_Q8_N2_CFG 16, 1, 1
#endif
#ifndef PTI_Q8_N4_CFG
#define PTI_Q8_N4_CFG 16, 1, 2
#endif
// Stream counts up to which the Q8 row-split kernel takes the paired loads
// (fewer load instructions, four more VALU ops per 16 quants).
#ifndef PTI_Q8_PAIRED_MAX_NS
#define PTI_Q8_PAIRED_MAX_NS 2
#endif
#ifndef PTI_SSQ_ROWWISE_CFG
#define PTI_SSQ_ROWWISE_CFG 16, 3, 1
#endif
#ifndef PTI_LDS_BUDGET
#define PTI_LDS_BUDGET (160 * 1024)
#endif


namespace {

// LDS of the per-wave-row kernel: x (dynamic, at most kXLds bytes) and the
// fused norm's partial sums (static, within the rest of the CU's budget).
constexpr int kNormLds = 256;
constexpr int kXLds = PTI_LDS_BUDGET - kNormLds;

constexpr uint32_t kRoundBytes = 1088;  // bytes of a row one round of 64 lanes covers (both formats)
constexpr uint32_t kPastBuffer = 0x40000000u;  // a buffer load offset past every buffer here: reads 0, touches nothing

enum Fmt { kQ8 = 0, kSSQ = 1 };

template <int FMT>
constexpr int unit_cols() { return FMT == kSSQ ? 8 : 16; }

constexpr int kMaxSegs = PTI_MAX_GROUP;

// The matrix of a launch: one packed matrix, or up to kMaxSegs of them with
// the same column count stacked into one row space (a grouped launch).  Row
// r lives in segment m (rows [seg_end[m-1], seg_end[m])) and starts at
// seg_base[m] + r * row_bytes: seg_base[m] is segment m's pointer less its
// first row's offset, so one formula serves every segment.
struct GemvArgs {
    uintptr_t seg_base[kMaxSegs];
    int64_t seg_end[kMaxSegs];  // INT64_MAX from the last segment on
    const float *x[4];
    float *y[4];
    const float *res[4];   // when set: y[s][r] = res[s][r] + (W x[s])[r] (res may be y itself)
    int64_t rows;
    int64_t row_bytes;
    int32_t cols;
    int32_t units;         // units per row
    int32_t rounds;        // ceil(units / 64)
    int32_t chunk_rounds;  // rounds of x held in LDS at once
    int32_t norm;          // per-wave-row kernel, x staged at once: x[s] <- rmsnorm(x[s]) as it is staged
    double norm_eps;
    // per-wave-row kernel, greedy verify of the outputs (null: none): per
    // workgroup g the largest verify key of stream s at keys[kKeyStride g + s]
    unsigned long long *keys;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Address of row `row` (wave-uniform in every caller, so this is scalar work).
// A launch of one matrix has seg_end[0] = INT64_MAX and skips the segment
// search, whose 64-bit compares would otherwise run on the VALU at every pass.
__device__ __forceinline__ const uint8_t *row_addr(const GemvArgs &a, int64_t row)
{
    uintptr_t b = a.seg_base[0];
    if (a.seg_end[0] != INT64_MAX) {  // a grouped launch (uniform)
#pragma unroll
        for (int m = 1; m < kMaxSegs; m++)
            b = row >= a.seg_end[m - 1] ? a.seg_base[m] : b;
    }
    return reinterpret_cast<const uint8_t *>(b + (uintptr_t)row * (uintptr_t)a.row_bytes);
}

// Raw dwords of one unit of one row.
//   SSQ: sc = [scale_A | scale_B << 16]; d[0..3] = the unit's 8 slots (slot
//        2k in the low half of d[k]: B in byte 0, A in byte 1; slot 2k+1 in
//        the high half).
//   Q8:  sc = the dword holding the scale; d[0..4] = the dwords holding the 16
//        quants, starting at a byte offset of 0 or 2 in d[0].
struct Unit {
    uint32_t sc;
    uint32_t d[5];
};

// Per-lane byte offsets of the lane's unit within one round of a row,
// relative to the dword-aligned start of the row.  Q8 has two classes: rows
// whose start is dword-aligned (class 0) and rows starting 2 bytes into a
// dword (class 1, only when a row holds an odd number of blocks).
struct LaneOffsets {
    uint32_t ssq_sc, ssq_d;              // SSQ: scale dword, first slot dword
    uint32_t q_sc[2], q_ssh[2];          // Q8: scale dword, bit shift of the scale in it
    uint32_t q_d[2], q_sh[2], q_h[2];    // Q8: first quant dword, byte shift, 5th dword
};

__device__ __forceinline__ LaneOffsets lane_offsets(int lane)
{
    LaneOffsets o;
    o.ssq_sc = ((uint32_t)lane >> 2) * PTI_SSQ_BLOCK_BYTES;
    o.ssq_d = o.ssq_sc + 4 + 16 * ((uint32_t)lane & 3);
    const uint32_t pair = (uint32_t)lane >> 1, h = (uint32_t)lane & 1;  // Q8 block within the round, half
#pragma unroll
    for (int c = 0; c < 2; c++) {
        const uint32_t blk = 2 * c + pair * PTI_Q8_BLOCK_BYTES;  // block start
        const uint32_t q = blk + 2 + 16 * h;                      // first quant
        o.q_sc[c] = blk & ~3u;
        o.q_ssh[c] = (blk & 3u) * 8;
        o.q_d[c] = q & ~3u;
        o.q_sh[c] = q & 3u;
        // quant bytes 15-16 are only used when the run starts 2 bytes into a
        // dword (at d + 16); otherwise the read goes to the run's last dword
        // (d + 12), so it never leaves the row.  Rows with an odd block count
        // read just the halfword, at d + 16 or d + 14.
        o.q_h[c] = o.q_d[c] + 12 + 2 * o.q_sh[c];
    }
    return o;
}

// Entry c (0 or 1) of a two-entry offset table, by select: indexing the
// table with a runtime value would move it to scratch memory.
__device__ __forceinline__ uint32_t pick(const uint32_t (&t)[2], int c) { return c ? t[1] : t[0]; }

__device__ __forceinline__ float sbyte(uint32_t d, int k) { return (float)(int8_t)(d >> (8 * k)); }

__device__ __forceinline__ float f16_lo(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (unsigned short)v); }
__device__ __forceinline__ float f16_hi(uint32_t v)
{
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(v >> 16));
}

// LDS layout of one chunk of x (float4 elements), UC = unit columns:
//   xs[((round * (UC/4) + cg) * NSP + p) * 64 + (lane ^ swz(cg))]
// cg = column group (4 columns) of the lane's unit, p = piece.  Piece p of
// (lane, cg) holds stream p's four columns of the group, as x holds them (so
// staging stores each loaded float4 as it is); NSP = streams rounded up to
// 1, 2 or 4 (three streams are padded with a zero fourth).
// The lane slot is XOR-swizzled by the column group, swz(cg) = cg * 16 / CG
// (CG = UC / 4 groups per unit), so that both the loop's reads of one
// (round, cg, p) and the staging stores of consecutive column groups spread
// over all LDS banks.
template <int UC, int NSP>
__device__ __forceinline__ int lds_slot(int rd, int cg, int p, int l)
{
    constexpr int CG = UC / 4;
    return ((rd * CG + cg) * NSP + p) * 64 + (l ^ (cg * (16 / CG)));
}

// Staging item `it` is column group it of the chunk (columns 4 it .. 4 it + 3):
// unit u = it / CG (round u / 64, lane u % 64), group cg = it % CG of the
// unit.  Consecutive threads take consecutive 16-byte pieces of each x row,
// so a wave's staging loads read contiguous memory.
template <int UC>
__device__ __forceinline__ void stage_item(int it, int &rd, int &cg, int &l)
{
    constexpr int CG = UC / 4;
    const int u = it / CG;
    rd = u >> 6, cg = it % CG, l = u & 63;
}

// A thread loads its items of the chunk (it < nitems) with buffer loads; a
// column past the row or a padding stream (s >= NS) reads zeros through the
// buffer bounds.  An item past the chunk leaves v unset (stage_store never
// reads it), so no load's result is merged with a default, which would make
// each load wait for the one before.
template <int UC, int NSP, int NS, int BATCH, int THREADS>
__device__ __forceinline__ void stage_load(const GemvArgs &a, int item0, float4 (&v)[BATCH][NSP], int tid,
                                           int nitems)
{
    __amdgpu_buffer_rsrc_t rs[NSP];
#pragma unroll
    for (int s = 0; s < NSP; s++)
        rs[s] = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(s < NS ? a.x[s] : nullptr), (short)0,
                                                  s < NS ? (int)(a.cols * 4) : 0, 0x00020000);
#pragma unroll
    for (int i = 0; i < BATCH; i++) {
        const int it = item0 + i * THREADS + tid;
        if (it < nitems) {
#pragma unroll
            for (int s = 0; s < NSP; s++) {
                const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(rs[s], 16 * it, 0, 0);  // column 4 it
                v[i][s] = make_float4(
                    __builtin_bit_cast(float, (uint32_t)t.x), __builtin_bit_cast(float, (uint32_t)t.y),
                    __builtin_bit_cast(float, (uint32_t)t.z), __builtin_bit_cast(float, (uint32_t)t.w));
            }
        }
    }
}

template <int UC, int NSP, int BATCH, int THREADS>
__device__ __forceinline__ void stage_store(float4 *xs, int item0, const float4 (&v)[BATCH][NSP], int tid,
                                            int nitems)
{
#pragma unroll
    for (int i = 0; i < BATCH; i++) {
        const int it = item0 + i * THREADS + tid;
        if (it >= nitems)
            break;
        int rd, cg, l;
        stage_item<UC>(it, rd, cg, l);
        float4 *base = xs + lds_slot<UC, NSP>(rd, cg, 0, l);
#pragma unroll
        for (int p = 0; p < NSP; p++)
            base[p * 64] = v[i][p];
    }
}

// Element (column c, stream s) of x in the LDS layout above (all of x staged).
template <int UC, int NSP>
__device__ __forceinline__ float *staged_elem(float4 *xs, int c, int s)
{
    const int rd = c / (64 * UC), l = (c / UC) % 64, cg = (c % UC) / 4;
    return reinterpret_cast<float *>(xs + lds_slot<UC, NSP>(rd, cg, s, l)) + c % 4;
}

// x[s] <- rmsnorm(x[s]) in LDS after all of x was staged and a barrier: the
// sum of squares by the first 256 threads in pti_rmsnorm's order (so the
// result has the same bits), then every thread scales the elements of the
// items it staged.  Ends with a barrier.
template <int UC, int NSP, int NS, int BATCH, int THREADS>
__device__ __forceinline__ void norm_staged(const GemvArgs &a, float4 *xs, int tid, int nitems)
{
    static_assert(THREADS >= pti_norm::kGroup, "the sum of squares takes 256 threads");
    __shared__ double part[NS][pti_norm::kGroup / 64];
    static_assert(sizeof(part) <= kNormLds, "the norm's LDS");
    if (tid < pti_norm::kGroup) {
        // B elements of every stream read at once (4 at three or four
        // streams: 8 would spill), then summed in order
        constexpr int B = NS >= 3 ? 4 : 8, G = pti_norm::kGroup;
        double acc[NS];
#pragma unroll
        for (int s = 0; s < NS; s++)
            acc[s] = 0.0;
        for (int c0 = tid; c0 < a.cols; c0 += B * G) {
            float v[NS][B];
#pragma unroll
            for (int k = 0; k < B; k++)
#pragma unroll
                for (int s = 0; s < NS; s++)
                    v[s][k] = c0 + k * G < a.cols ? *staged_elem<UC, NSP>(xs, c0 + k * G, s) : 0.f;
#pragma unroll
            for (int k = 0; k < B; k++)
                if (c0 + k * G < a.cols)
#pragma unroll
                    for (int s = 0; s < NS; s++)
                        acc[s] = pti_norm::sq_acc(acc[s], v[s][k]);
        }
#pragma unroll
        for (int s = 0; s < NS; s++) {
            const double t = pti_norm::wave_sum_f64(acc[s]);
            if ((tid & 63) == 0)
                part[s][tid >> 6] = t;
        }
    }
    __syncthreads();
    double r[NS];
#pragma unroll
    for (int s = 0; s < NS; s++)
        r[s] = pti_norm::inv_root(part[s], a.cols, a.norm_eps);
#pragma unroll
    for (int i = 0; i < BATCH; i++) {
        const int it = i * THREADS + tid;
        if (it >= nitems)
            break;
        int rd, cg, l;
        stage_item<UC>(it, rd, cg, l);
        float4 *base = xs + lds_slot<UC, NSP>(rd, cg, 0, l);
#pragma unroll
        for (int p = 0; p < NS; p++) {
            float *e = reinterpret_cast<float *>(base + p * 64);
#pragma unroll
            for (int q = 0; q < 4; q++)
                e[q] = pti_norm::apply(e[q], r[p]);
        }
    }
    __syncthreads();
}

// Stage rounds [r0, r0 + nr) of x into LDS rounds 0..nr-1 (nr at most the
// LDS budget's chunk, which BATCH items per thread cover).
template <int UC, int NSP, int NS, int BATCH, int THREADS>
__device__ __forceinline__ void stage_all(const GemvArgs &a0, float4 *xs, int r0, int nr, int tid)
{
    GemvArgs a = a0;  // x pointers shifted to the chunk's first column
    const int c0 = r0 * 64 * UC;
#pragma unroll
    for (int s = 0; s < NS; s++)
        a.x[s] += c0;
    a.cols -= c0;
    const int nitems = nr * 64 * (UC / 4);  // <= BATCH * THREADS
    float4 v[BATCH][NSP];
    stage_load<UC, NSP, NS, BATCH, THREADS>(a, 0, v, tid, nitems);
    stage_store<UC, NSP, BATCH, THREADS>(xs, 0, v, tid, nitems);
}

template <int CTRL, int ROW_MASK, bool BOUND_ZERO>
__device__ __forceinline__ float dpp(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf,
                                                                 BOUND_ZERO));
}

// Values carried into tree_sums: n rounded up to a power of two.
constexpr int tree_width(int n) { return n <= 1 ? 1 : n <= 2 ? 2 : n <= 4 ? 4 : 8; }

// Lane i gets the value of lane i ^ 4: two row shifts by 4, each writing the
// banks (groups of four lanes) it serves.
__device__ __forceinline__ float xor4(float v)
{
    const int x = __builtin_bit_cast(int, v);
    int t = __builtin_amdgcn_update_dpp(x, x, 0x104, 0xf, 0x5, false);  // banks 0, 2: row_shl 4
    t = __builtin_amdgcn_update_dpp(t, x, 0x114, 0xf, 0xa, false);      // banks 1, 3: row_shr 4
    return __builtin_bit_cast(float, t);
}

// The sums over the 64 lanes of N values at once (N <= 8), each by the fixed
// lane tree of every GEMV kernel here: the balanced binary tree that pairs
// lanes by bit 0 of the lane index, then by bit 1, ..., then by bit 5.
// Addition being commutative, that pairing alone fixes each sum's bits, so
// every kernel and stream count gives a row the same bits.  The stages for
// the bits below log2(V) (V = tree_width(N)) also halve the values a lane
// carries: of each pair of values (2t, 2t + 1) a lane keeps the one its bit
// selects and adds its partner's copy of it, so V values cost about as much
// as two single-value trees.  Later stages carry one value: row shifts by 1,
// 2, 4, 8 (right in the lanes whose bits log2(V)..3 are set), then the row
// and half-wave swaps for bits 4 and 5.  The total of value k lands in lane
// 16 - V + k of every row.  Works in place on c (destroyed).
template <int N>
__device__ __forceinline__ float tree_sums(float (&c)[N], int lane)
{
    static_assert(N >= 1 && N <= 8, "tree_sums carries at most eight values");
    constexpr int V = tree_width(N);
    constexpr int LV = V == 8 ? 3 : V == 4 ? 2 : V == 2 ? 1 : 0;
    // values past N (three streams) are zeros; pair t writes c[t] after
    // reading c[2t] and c[2t + 1]
    auto at = [&](int k) { return k < N ? c[k] : 0.f; };
    if constexpr (LV > 0) {
        const bool hi = lane & 1;
#pragma unroll
        for (int t = 0; t < V / 2; t++) {
            const float e0 = at(2 * t), e1 = at(2 * t + 1);
            const float keep = hi ? e1 : e0, send = hi ? e0 : e1;
            if (t < N)
                c[t] = keep + dpp<0xB1, 0xf, false>(send);  // quad_perm [1, 0, 3, 2]
        }
    }
    if constexpr (LV > 1) {
        const bool hi = lane & 2;
#pragma unroll
        for (int t = 0; t < V / 4; t++) {
            const float keep = hi ? c[2 * t + 1] : c[2 * t], send = hi ? c[2 * t] : c[2 * t + 1];
            c[t] = keep + dpp<0x4E, 0xf, false>(send);  // quad_perm [2, 3, 0, 1]
        }
    }
    if constexpr (LV > 2) {
        const bool hi = lane & 4;
        const float keep = hi ? c[1] : c[0], send = hi ? c[0] : c[1];
        c[0] = keep + xor4(send);
    }
    float x = c[0];
    if constexpr (LV <= 0)
        x = x + dpp<0x111, 0xf, true>(x);
    if constexpr (LV <= 1)
        x = x + dpp<0x112, 0xf, true>(x);
    if constexpr (LV <= 2)
        x = x + dpp<0x114, 0xf, true>(x);
    x = x + dpp<0x118, 0xf, true>(x);
    // the swaps return two vectors; each element is cast to a scalar before
    // its bits are read
    const auto r16 = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                      false, false);
    x = __builtin_bit_cast(float, (unsigned)r16[0]) + __builtin_bit_cast(float, (unsigned)r16[1]);
    const auto r32 = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                      false, false);
    return __builtin_bit_cast(float, (unsigned)r32[0]) + __builtin_bit_cast(float, (unsigned)r32[1]);
}

// One step of an unsigned 64-bit max over lanes: DPP moves the low and high
// words with the same control; lanes DPP does not write see 0 (the identity).
template <int CTRL, int ROW_MASK, bool BOUND_ZERO>
__device__ __forceinline__ unsigned long long umax_dpp(unsigned long long k)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)k, CTRL, ROW_MASK, 0xf, BOUND_ZERO);
    const uint32_t hi =
        (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(k >> 32), CTRL, ROW_MASK, 0xf, BOUND_ZERO);
    const unsigned long long o = ((unsigned long long)hi << 32) | lo;
    return o > k ? o : k;
}

// Unsigned 64-bit max over the 64 lanes, in lane 63: row shifts by 1, 2, 4, 8
// within each 16-lane row, then row_bcast15 and row_bcast31 across rows.
__device__ __forceinline__ unsigned long long wave_umax(unsigned long long k)
{
    k = umax_dpp<0x111, 0xf, true>(k);
    k = umax_dpp<0x112, 0xf, true>(k);
    k = umax_dpp<0x114, 0xf, true>(k);
    k = umax_dpp<0x118, 0xf, true>(k);
    k = umax_dpp<0x142, 0xa, false>(k);
    k = umax_dpp<0x143, 0xc, false>(k);
    return k;
}

// Key ordering (value, then lower row) as one unsigned 64-bit number: the
// float's bits made monotonic (-0 counted as +0), then the row inverted.  The
// largest key is the argmax with the lowest row among equals; no key is 0.
__device__ __forceinline__ unsigned long long verify_key(float v, int64_t row)
{
    uint32_t u = __builtin_bit_cast(uint32_t, v == 0.f ? 0.f : v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((unsigned long long)u << 32) | (0xFFFFFFFFu - (uint32_t)row);
}

constexpr int kKeyStride = pti::kVerifyKeyStride;  // keys per workgroup in a per-wave-row verify (streams, padded)

// Row addressing of the per-wave-row kernel.
//   kAmFlat: one matrix, row r at seg_base[0] + r * row_bytes.
//   kAmSeg:  a grouped launch, rows stacked over the segments (row_addr).
//   kAmPair: the gate and up matrices of an MLP (seg_base[0], seg_base[1]);
//            a.rows counts row pairs, a wave's pass p takes row u of each
//            (R = 2: gate in row slot 0, up in slot 1) and the pair leaves
//            as y[s][u] = silu(gate) * up, so the activation needs no launch
//            of its own and gate, up are never stored.
constexpr int kAmFlat = 0, kAmSeg = 1, kAmPair = 2;

template <int FMT, int NSP, int NS, int R, bool ROWS4, int kD, int AM>
struct Wave {
    static_assert(AM != kAmPair || R == 2, "a pass takes one gate row and one up row");
    static constexpr int UC = unit_cols<FMT>();
    static constexpr int CG = UC / 4;

    const GemvArgs &a;
    const float4 *xs;
    int lane;
    // Rows of this wave (wave-uniform): row(t) = first + t * stride, t < nrow.
    int64_t first, stride;
    int nrow, npass;
    LaneOffsets lo;
    float acc[R][NS];
    // finished rows of the current group, row j of the group in lane j of
    // outv[0] (pairs: pair j's gate in lane j of outv[0], its up in outv[1])
    float outv[AM == kAmPair ? 2 : 1][NS];
    int gp0;         // first pass of the current group
    unsigned long long vkey[NS];  // a.keys: this lane's largest verify key of each stream
    Unit bufs[kD + 1][R];

    // Cursors over the steps (pass, round) of the current segment: passes
    // [p0, p1), rounds [i0, i1).  The issue cursor runs kD steps ahead of the
    // compute cursor; each keeps what it needs of its pass in scalar
    // registers, rebuilt when it enters a new pass, so a step costs a few
    // scalar instructions (the scalar unit is shared by the CU's waves).
    int p1, i0, i1, nsteps;
    int ip, ir;                        // issue cursor
    __amdgpu_buffer_rsrc_t irs[R];     // its pass's rows (empty past the end)
    int icls[R];                       // Q8 class of those rows
    int cp, cr;                        // compute cursor
    int cnrows;                        // rows in the compute cursor's pass
    int ccls[R];

    __device__ __forceinline__ Wave(const GemvArgs &a_, const float4 *xs_, int lane_, int64_t first_,
                                    int64_t stride_, int nrow_)
        : a(a_), xs(xs_), lane(lane_), first(first_), stride(stride_), nrow(nrow_)
    {
        npass = AM == kAmPair ? nrow : (nrow + R - 1) / R;
        lo = lane_offsets(lane_);
#pragma unroll
        for (int s = 0; s < NS; s++)
            vkey[s] = 0;
#pragma unroll
        for (int r = 0; r < R; r++)
#pragma unroll
            for (int s = 0; s < NS; s++)
                acc[r][s] = 0.f;
    }

    // Address of a row: a launch of one matrix (SEG false) needs no segment
    // search, whose selects and 64-bit compares would otherwise run at every
    // pass on the CU's one scalar unit, shared by its 16 waves.
    __device__ __forceinline__ uintptr_t row_ptr(int64_t row) const
    {
        if constexpr (AM == kAmSeg)
            return reinterpret_cast<uintptr_t>(row_addr(a, row));
        else
            return a.seg_base[0] + (uintptr_t)row * (uintptr_t)a.row_bytes;
    }

    // Address of row slot r of pass p.
    __device__ __forceinline__ uintptr_t pass_row_ptr(int p, int r) const
    {
        if constexpr (AM == kAmPair)
            return a.seg_base[r] + (uintptr_t)(first + (int64_t)p * stride) * (uintptr_t)a.row_bytes;
        else
            return row_ptr(first + ((int64_t)p * R + r) * stride);
    }

    __device__ __forceinline__ int rows_in(int pass) const
    {
        return AM == kAmPair ? R : min(R, nrow - pass * R);
    }

    // Buffer resources over the rows of pass p (dword-aligned bases).  Rows
    // past the pass's last, or a pass past the segment, get empty resources:
    // their loads return 0 without touching memory, but are still issued, so
    // the count of loads in flight is the same on every path and each wait
    // covers exactly one step.
    __device__ __forceinline__ void set_issue_pass(int p)
    {
        const int nr_in = p < p1 ? rows_in(p) : 0;
#pragma unroll
        for (int r = 0; r < R; r++) {
            const uintptr_t q = pass_row_ptr(p, r);
            const uint32_t e0 = (uint32_t)(q & 3);
            icls[r] = ROWS4 ? 0 : (int)(e0 >> 1);
            const uint32_t n = r < nr_in ? e0 + (uint32_t)a.row_bytes : 0u;
            irs[r] = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(q & ~uintptr_t(3)), (short)0, (int)n,
                                                       0x00020000);
        }
    }

    __device__ __forceinline__ void set_compute_pass(int p)
    {
        cnrows = rows_in(p);
        if constexpr (!ROWS4) {
#pragma unroll
            for (int r = 0; r < R; r++)
                ccls[r] = (int)((pass_row_ptr(p, r) >> 1) & 1);
        }
    }

    // Issue the loads of the issue cursor's step into buf, then advance it.
    __device__ __forceinline__ void issue(Unit (&buf)[R])
    {
        const int soff = ir * (int)kRoundBytes;
#pragma unroll
        for (int r = 0; r < R; r++) {
            if constexpr (FMT == kSSQ) {
                buf[r].sc = __builtin_amdgcn_raw_buffer_load_b32(irs[r], (int)lo.ssq_sc, soff, 0);
                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(irs[r], (int)lo.ssq_d, soff, 0);
                buf[r].d[0] = v.x, buf[r].d[1] = v.y, buf[r].d[2] = v.z, buf[r].d[3] = v.w;
            } else {
                const int c = icls[r];
                buf[r].sc = __builtin_amdgcn_raw_buffer_load_b32(irs[r], (int)pick(lo.q_sc, c), soff, 0);
                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(irs[r], (int)pick(lo.q_d, c), soff, 0);
                buf[r].d[0] = v.x, buf[r].d[1] = v.y, buf[r].d[2] = v.z, buf[r].d[3] = v.w;
                // rows of an even number of blocks: the dword holding quant
                // bytes 15-16 lies inside the row; otherwise read the halfword
                buf[r].d[4] = ROWS4 ? __builtin_amdgcn_raw_buffer_load_b32(irs[r], (int)pick(lo.q_h, c), soff, 0)
                                    : (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(
                                          irs[r], (int)pick(lo.q_h, c) + 2 - (int)pick(lo.q_sh, c), soff, 0);
            }
        }
        if (++ir == i1) {
            ir = i0;
            set_issue_pass(++ip);
        }
    }

    // Accumulate the compute cursor's step from buf (x of round cr at LDS round
    // cr - i0); at the end of a pass reduce its rows.  Lanes past
    // the last unit of a row, and rows past the last of a partial pass, read
    // zero weights through the buffer bounds (and such lanes zero activations
    // from LDS), so they add nothing and need no branch; only the stores are
    // guarded.
    __device__ __forceinline__ void compute(const Unit (&buf)[R])
    {
        const float4 *xr = xs + ((cr - i0) * CG * NSP) * 64;
        uint32_t q[R][4];
        if constexpr (FMT == kQ8) {
#pragma unroll
            for (int r = 0; r < R; r++) {
                // realign the 16 quants: byte offset 0 or 2 within d[0]
                const uint32_t sh = ROWS4 ? lo.q_sh[0] : pick(lo.q_sh, ccls[r]);
#pragma unroll
                for (int k = 0; k < 4; k++)
                    q[r][k] = __builtin_amdgcn_alignbyte(buf[r].d[k + 1], buf[r].d[k], sh);
            }
        }
        float bs[R][NS];
#pragma unroll
        for (int c = 0; c < CG; c++) {
            float xv[4][NSP];  // [column of the group][stream]
#pragma unroll
            for (int p = 0; p < NSP; p++) {
                const float4 t = xr[(c * NSP + p) * 64 + (lane ^ (c * (16 / CG)))];
                xv[0][p] = t.x, xv[1][p] = t.y, xv[2][p] = t.z, xv[3][p] = t.w;
            }
#pragma unroll
            for (int r = 0; r < R; r++) {
#pragma unroll
                for (int m = 0; m < 4; m++) {
                    if constexpr (FMT == kQ8) {
                        const float wq = sbyte(q[r][c], m);
#pragma unroll
                        for (int s = 0; s < NS; s++)
                            bs[r][s] = (c == 0 && m == 0) ? wq * xv[m][s] : __builtin_fmaf(wq, xv[m][s], bs[r][s]);
                    } else {
                        // slot 4c + m of the unit: dword 2c + m/2, halfword m % 2;
                        // twin A = high byte (even streams), twin B = low byte
                        // (odd streams)
                        const uint32_t dw = buf[r].d[2 * c + (m >> 1)];
#pragma unroll
                        for (int s = 0; s < NS; s++) {
                            const float wq = sbyte(dw, 2 * (m & 1) + ((s & 1) ? 0 : 1));
                            bs[r][s] = (c == 0 && m == 0) ? wq * xv[m][s] : __builtin_fmaf(wq, xv[m][s], bs[r][s]);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int r = 0; r < R; r++) {
            if constexpr (FMT == kQ8) {
                const float d = f16_lo(buf[r].sc >> (ROWS4 ? lo.q_ssh[0] : pick(lo.q_ssh, ccls[r])));
#pragma unroll
                for (int s = 0; s < NS; s++)
                    acc[r][s] = __builtin_fmaf(d, bs[r][s], acc[r][s]);
            } else {
#pragma unroll
                for (int s = 0; s < NS; s++)
                    acc[r][s] = __builtin_fmaf((s & 1) ? f16_hi(buf[r].sc) : f16_lo(buf[r].sc), bs[r][s], acc[r][s]);
            }
        }
        if (cr == a.rounds - 1) {  // the pass's rows are complete
            // The pass's R x NS sums go through one tree_sums; each moves to
            // lane (row in group) of outv, stored after the loop, so the loop
            // holds no vector stores (stores share the counter that the
            // weight-load waits use).
            constexpr int V = tree_width(R * NS);
            const int tot = __builtin_bit_cast(int, tree_sums<R * NS>(reinterpret_cast<float (&)[R * NS]>(acc), lane));
#pragma unroll
            for (int r = 0; r < R; r++) {
                // the lane and outv slot of row slot r
                const int j = AM == kAmPair ? cp - gp0 : (cp - gp0) * R + r;
                float(&o)[NS] = outv[AM == kAmPair ? r : 0];
#pragma unroll
                for (int s = 0; s < NS; s++) {
                    const float t = __builtin_bit_cast(float, __builtin_amdgcn_readlane(tot, 16 - V + r * NS + s));
                    o[s] = lane == j ? t : o[s];
                    acc[r][s] = 0.f;
                }
            }
        }
        if (++cr == i1) {
            cr = i0;
            if (++cp < p1)
                set_compute_pass(cp);
        }
    }

    // Run steps (pass, round) for passes [p0, p1) and rounds [i0, i1).
    // begin() issues the loads of the first kD steps; loop() computes step s
    // from buffer s % (kD + 1) after issuing the loads of step s + kD into the
    // buffer step s - 1 used.  Unrolled kD + 1 times so every buffer index is
    // a compile-time constant.
    __device__ __forceinline__ void begin(int p0_, int p1_, int i0_, int i1_)
    {
        p1 = p1_, i0 = i0_, i1 = i1_;
        nsteps = max(0, (p1_ - p0_) * (i1_ - i0_));
        ip = cp = p0_;
        ir = cr = i0_;
        set_issue_pass(ip);
        if (cp < p1)
            set_compute_pass(cp);
#pragma unroll
        for (int k = 0; k < kD; k++)
            issue(bufs[k]);
    }

    // One step: issue the loads kD steps ahead, then compute this one (a
    // padding step past the segment's last issues its empty loads and skips
    // the arithmetic).
    template <int K>
    __device__ __forceinline__ void step(int index)
    {
        issue(bufs[(K + kD) % (kD + 1)]);
        __builtin_amdgcn_sched_barrier(0);
        if (index < nsteps)  // wave-uniform
            compute(bufs[K]);
        __builtin_amdgcn_sched_barrier(0);
    }

    // PAD: run the step count rounded up to a multiple of kD + 1, so the loop
    // has one exit, at its end.  An exit inside the unrolled body gives the
    // compiler a path back to the loop head on which fewer loads are in
    // flight, and it then makes the head's step wait for nearly all of them
    // (draining the prefetch once per iteration).  The extra steps load
    // through empty buffer resources (zero weights and scales), so they add
    // exact zeros to the accumulators, and any row they complete lies past the
    // segment's passes, in a lane that is never stored.
    // !PAD: stop after exactly nsteps steps (short segments between barriers,
    // where padding would cost more than the waits).
    template <bool PAD>
    __device__ __forceinline__ void loop()
    {
        if constexpr (PAD) {
            const int iters = (nsteps + kD) / (kD + 1);
            for (int it = 0; it < iters; it++) {
                [&]<int... K>(std::integer_sequence<int, K...>) {
                    (step<K>(it * (kD + 1) + K), ...);
                }(std::make_integer_sequence<int, kD + 1>{});
            }
        } else {
            for (int s = 0;; s += kD + 1) {
#pragma unroll
                for (int k = 0; k <= kD; k++) {
                    if (s + k >= nsteps)
                        goto done;
                    issue(bufs[(k + kD) % (kD + 1)]);
                    __builtin_amdgcn_sched_barrier(0);
                    compute(bufs[k]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        done:;
        }
    }

    // Passes per output group: a group's rows (pairs) fit one lane each of outv.
    static constexpr int kGroupPasses = AM == kAmPair ? 64 : 64 / R;

    __device__ __forceinline__ void begin_group(int g0)
    {
        gp0 = g0;
#pragma unroll
        for (auto &o : outv)
#pragma unroll
            for (int s = 0; s < NS; s++)
                o[s] = 0.f;
    }

    // Store the finished rows (pairs) of the group of passes [gp0, g1).
    __device__ __forceinline__ void store_group(int g1)
    {
        if constexpr (AM == kAmPair) {
            const int nj = min(g1, nrow) - gp0;
            if (lane < nj) {
                const int64_t u = first + (int64_t)(gp0 + lane) * stride;
#pragma unroll
                for (int s = 0; s < NS; s++)
                    a.y[s][u] = pti_silu::silu_mul(outv[0][s], outv[1][s]);
            }
        } else {
            const int nj = min(g1 * R, nrow) - gp0 * R;
            if (a.keys && lane < nj) {  // the launch's greedy verify (uniform test first)
                const int64_t row = first + (int64_t)(gp0 * R + lane) * stride;
#pragma unroll
                for (int s = 0; s < NS; s++)
                    vkey[s] = std::max(vkey[s], verify_key(outv[0][s], row));
            }
            if (lane < nj) {
                const int64_t row = first + (int64_t)(gp0 * R + lane) * stride;
                if (a.res[0]) {  // uniform: a residual launch sets every stream's
                    float r[NS];  // all loads first, then the sums
#pragma unroll
                    for (int s = 0; s < NS; s++)
                        r[s] = a.res[s][row];
#pragma unroll
                    for (int s = 0; s < NS; s++)
                        a.y[s][row] = r[s] + outv[0][s];
                } else {
#pragma unroll
                    for (int s = 0; s < NS; s++)
                        a.y[s][row] = outv[0][s];
                }
            }
        }
    }
};

template <int FMT, int NSP, int NS, int R, bool ROWS4, int W, int D, int AM>
__global__ __launch_bounds__(64 * W) void gemv_kernel(GemvArgs a)
{
    static_assert(W % 4 == 0, "waves per workgroup must fill the four SIMDs evenly");
    constexpr int kThreads = 64 * W;
    extern __shared__ float4 xs[];
    constexpr int UC = unit_cols<FMT>();
    // Staging items per thread: enough for the largest chunk of x the LDS
    // budget holds, so a chunk is staged in one straight-line batch (no loop
    // between the first weight loads and the main loop, which keeps the
    // compiler's count of loads in flight exact).
    constexpr int kMaxChunkItems = (kXLds / (64 * UC * NSP * 4)) * 64 * (UC / 4);
    constexpr int BATCH = (kMaxChunkItems + kThreads - 1) / kThreads;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    // Rows are dealt round-robin to the SIMDs of the grid: SIMD sg (of nsimd)
    // gets rows sg, sg + nsimd, sg + 2 nsimd, ..., so every SIMD gets the same
    // count to within one and, at any moment, the whole GPU reads one window
    // of consecutive rows.  Waves w, w + 4, w + 8, ... of a workgroup share a
    // SIMD and take turns through its rows.
    constexpr int kPerSimd = W / 4;
    const int64_t nsimd = (int64_t)gridDim.x * 4;
    const int64_t sg = (int64_t)blockIdx.x * 4 + (wv & 3);
    const int j = wv >> 2;
    const int64_t n_simd_rows = sg < a.rows ? (a.rows - sg + nsimd - 1) / nsimd : 0;
    const int nrow = (int)(n_simd_rows > j ? (n_simd_rows - j + kPerSimd - 1) / kPerSimd : 0);
    Wave<FMT, NSP, NS, R, ROWS4, D, AM> w(a, xs, lane, sg + (int64_t)j * nsimd, (int64_t)kPerSimd * nsimd, nrow);

    // (pairs are launched only with all of x in LDS)
    if (AM == kAmPair || a.chunk_rounds >= a.rounds) {
        // All of x fits: stage it once, then run every pass.  The x loads go
        // out first, then the first weight loads, so the LDS stores wait only
        // for x while the weights are already in flight.
        float4 v[BATCH][NSP];
        const int nitems = a.rounds * 64 * (UC / 4);
        stage_load<UC, NSP, NS, BATCH, kThreads>(a, 0, v, tid, nitems);
        __builtin_amdgcn_sched_barrier(0);
        w.begin(0, min(w.npass, w.kGroupPasses), 0, a.rounds);
        __builtin_amdgcn_sched_barrier(0);
        stage_store<UC, NSP, BATCH, kThreads>(xs, 0, v, tid, nitems);
        __syncthreads();
        if (a.norm)  // uniform
            norm_staged<UC, NSP, NS, BATCH, kThreads>(a, xs, tid, nitems);
        w.begin_group(0);
        w.template loop<true>();
        w.store_group(min(w.npass, w.kGroupPasses));
        // waves with more rows than one output group holds
        for (int g0 = w.kGroupPasses; g0 < w.npass; g0 += w.kGroupPasses) {
            const int g1 = min(w.npass, g0 + w.kGroupPasses);
            w.begin_group(g0);
            w.begin(g0, g1, 0, a.rounds);
            w.template loop<true>();
            w.store_group(g1);
        }
    } else {
        // x in K-chunks: every wave of the workgroup walks the same
        // (pass, chunk) sequence so that the barriers match
        const int64_t max_rows = (a.rows + nsimd * kPerSimd - 1) / (nsimd * kPerSimd);
        const int max_pass = (int)((max_rows + R - 1) / R);
        for (int p = 0; p < max_pass; p++)
            for (int i0 = 0; i0 < a.rounds; i0 += a.chunk_rounds) {
                const int i1 = min(a.rounds, i0 + a.chunk_rounds);
                __syncthreads();
                stage_all<UC, NSP, NS, BATCH, kThreads>(a, xs, i0, i1 - i0, tid);
                __syncthreads();
                if (p < w.npass) {
                    if (i0 == 0)
                        w.begin_group(p);
                    w.begin(p, p + 1, i0, i1);
                    w.template loop<false>();
                    if (i1 == a.rounds)
                        w.store_group(p + 1);
                }
            }
    }
    if (a.keys) {  // uniform: the workgroup's largest key of each stream
        // The waves' keys go to the x area (at least one round of x, whatever
        // the chunking) once every wave is done reading x.
        static_assert(NS * W * 8 <= 64 * UC * NSP * 4, "the verify keys must fit one round of x");
        unsigned long long *wk = reinterpret_cast<unsigned long long *>(xs);  // [NS][W]
        __syncthreads();
#pragma unroll
        for (int s = 0; s < NS; s++) {
            const unsigned long long k = wave_umax(w.vkey[s]);  // in lane 63
            if (lane == 63)
                wk[s * W + wv] = k;
        }
        __syncthreads();
        if (tid < NS) {
            unsigned long long k = wk[tid * W];
            for (int i = 1; i < W; i++)
                k = std::max(k, wk[tid * W + i]);
            a.keys[kKeyStride * blockIdx.x + tid] = k;
        }
    }
}

int device_cus()
{
    static thread_local int dev_cached = -1, cus = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return 0;
    if (dev != dev_cached) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        dev_cached = dev;
    }
    return cus;
}

struct RowwiseCfg {
    int waves, prefetch, rows;
};

template <int FMT, int NS>
constexpr RowwiseCfg rowwise_cfg()
{
    if constexpr (FMT == kSSQ)
        return {PTI_SSQ_ROWWISE_CFG};
    else if constexpr (NS == 1)
        return {PTI_Q8_N1_CFG};
    else if constexpr (NS == 2)
        return {PTI_Q8_N2_CFG};
    else
        return {PTI_Q8_N4_CFG};
}

// PAIR: a gate|up pair launch (kAmPair; all of x must fit in LDS, which the
// caller checks); otherwise one matrix or a grouped launch, by a.seg_end.
template <int FMT, int NSP, int NS, bool ROWS4, bool PAIR = false>
int launch(const GemvArgs &a0, hipStream_t stream)
{
    constexpr int UC = unit_cols<FMT>();
    constexpr RowwiseCfg cfg = rowwise_cfg<FMT, NS>();
    constexpr int R = PAIR ? 2 : cfg.rows, kWaves = cfg.waves, kThreads = 64 * kWaves;
    GemvArgs a = a0;
    const int per_round = 64 * UC * NSP * 4;  // LDS bytes per round of x
    a.chunk_rounds = max(1, min(a.rounds, kXLds / per_round));
    const size_t lds = (size_t)a.chunk_rounds * per_round;
    if (PAIR && a.chunk_rounds < a.rounds)
        return PTI_ERR_SHAPE;  // pairs need all of x in LDS
    const int cus = device_cus();
    if (cus <= 0) {
        pti::set_hip_error(hipGetLastError());
        return PTI_ERR_HIP;
    }
    // Every CU, whatever the row count: with few rows per SIMD the loop is
    // VALU-bound (four streams), so spreading the rows over more SIMDs is what
    // shortens it; a workgroup without rows only stages x.
    const int64_t grid = std::min<int64_t>(cus, a.rows);
    const bool seg = !PAIR && a.seg_end[0] != INT64_MAX;  // a grouped launch: rows in several matrices
    void (*kern)(GemvArgs);
    if constexpr (PAIR)
        kern = gemv_kernel<FMT, NSP, NS, R, ROWS4, kWaves, cfg.prefetch, kAmPair>;
    else
        kern = seg ? gemv_kernel<FMT, NSP, NS, R, ROWS4, kWaves, cfg.prefetch, kAmSeg>
                   : gemv_kernel<FMT, NSP, NS, R, ROWS4, kWaves, cfg.prefetch, kAmFlat>;
    // The dynamic-LDS limit is a per-device attribute of the kernel: set it once on each device each
    // instance runs on (one bit per device; two threads racing both set it, which is harmless).
    static std::atomic<uint64_t> attr_devs[2] = {0, 0};
    int dev = 0;
    if (hipError_t e = hipGetDevice(&dev); e != hipSuccess || dev < 0 || dev >= 64) {
        pti::set_hip_error(e != hipSuccess ? e : hipErrorInvalidDevice);
        return PTI_ERR_HIP;
    }
    if (!(attr_devs[seg].load(std::memory_order_acquire) >> dev & 1)) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, kXLds);
        if (e != hipSuccess) {
            pti::set_hip_error(e);
            return PTI_ERR_HIP;
        }
        attr_devs[seg].fetch_or(uint64_t{1} << dev, std::memory_order_acq_rel);
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), lds, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        pti::set_hip_error(e);
        return PTI_ERR_HIP;
    }
    return PTI_OK;
}

template <int FMT>
GemvArgs make_args(const void *w, int64_t rows, int64_t cols)
{
    GemvArgs a{};
    for (int m = 0; m < kMaxSegs; m++) {
        a.seg_base[m] = reinterpret_cast<uintptr_t>(w);
        a.seg_end[m] = INT64_MAX;
    }
    a.rows = rows;
    a.cols = (int32_t)cols;
    a.row_bytes = (cols / PTI_BLOCK) * (FMT == kSSQ ? PTI_SSQ_BLOCK_BYTES : PTI_Q8_BLOCK_BYTES);
    a.units = (int32_t)(cols / unit_cols<FMT>());
    a.rounds = (a.units + 63) / 64;
    return a;
}

// ---------------------------------------------------------------------------
// Row-split SSQ kernel: the waves of a workgroup share each row.
//
// HBM delivers the most when the requests in flight form one compact window
// of memory that slides forward (as a grid-stride read does), and when that
// window is small.  With every wave owning whole rows, the window spans
// thousands of rows with one round in flight per row.  Here workgroup g (of
// G, one per CU) owns rows g, g + G, g + 2G, ... and covers P of them per
// step; the Q waves of a row each load T consecutive rounds of it.  At any
// moment the GPU reads a narrow band of consecutive rows, each one whole.
//
// Loads run one step ahead, round by round: after computing round tt of
// step t a wave loads round tt of step t + 1 into the buffer it just freed,
// so T rounds per wave are always in flight.
//
// A wave always handles the same column slice, so it loads its T rounds of x
// (T * 8 columns per lane, every stream) once into registers: no LDS staging,
// no LDS reads in the loop.  Per step it sums its rounds per lane, reduces
// over its 64 lanes (the fixed lane tree) and parks the partial in LDS; every
// S steps the workgroup sums the Q partials of each finished row in slice
// order and stores the row.  A row's order of operations depends only on
// (rows, cols).
constexpr int kSplitMaxWaves = 16;
constexpr int kSplitTMax = 5;           // rounds per wave at most (x: 80 registers)
constexpr int kSplitWavesSmallT = 16;   // waves per workgroup when T <= 2
constexpr int kSplitWavesBigT = 4;      // ... when T >= 3 (measured best)

// Launch bound for T (the registers per wave follow from it).
constexpr int split_bound_waves(int T) { return T >= 3 ? 8 : kSplitMaxWaves; }

// Most workgroups of a row-split launch: one per CU, at most this many (the
// fused verify's workspace holds one pair of keys per workgroup).
constexpr int kSplitMaxGrid = 1024;
static_assert(kSplitMaxGrid * 2 * 8 <= PTI_SSQ_VERIFY_WORK_BYTES, "workspace size");

struct SplitArgs {
    GemvArgs g;
    int32_t P, Q;         // rows per step, waves per row
    int32_t S;            // steps per flush of finished rows
    // fused greedy verify (VERIFY kernels only): per workgroup the largest
    // key of each twin, keys[2 g + s]
    unsigned long long *keys;
};


// VERIFY: also the first half of the greedy verify of the two twins' outputs
// -- each thread keeps the largest key of the rows it stores and each
// workgroup stores the largest of its threads' (0 if it has no rows);
// verify_keys_kernel, launched next on the same stream, reduces them.  (A
// single kernel whose last workgroup reduces the keys needs a device-scope
// release and acquire per workgroup to see the others' keys; on gfx950 those
// are L2 writebacks and invalidates, which cost more than the second launch.)
//
// BW: the launch bound in waves.  Normally split_bound_waves(T); launches of
// at most four waves may use a bound of four, which lets a wave keep more
// values in registers (two streams per twin at T = 5 need it).
template <int T, int NS, bool VERIFY, int BW = split_bound_waves(T)>
__global__ __launch_bounds__(64 * BW) void gemv_ssq_split_kernel(SplitArgs sa)
{
    static_assert(NS == 2 || (NS == 4 && !VERIFY), "streams: one or two per twin; verify with one");
    constexpr int UC = unit_cols<kSSQ>();
    const GemvArgs &a = sa.g;
    const int P = sa.P, Q = sa.Q, S = sa.S;
    extern __shared__ float part[];  // [2][S * P][Q][NS]: row partials, double-buffered
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int p = wv / Q, q = wv - (wv / Q) * Q;
    const int64_t G = gridDim.x, g = blockIdx.x;
    const int64_t wg_rows = g < a.rows ? (a.rows - g + G - 1) / G : 0;
    const int steps = (int)((wg_rows + P - 1) / P);

    float xv[T][UC][NS];  // this lane's x (filled below, after the first weight requests)
    const LaneOffsets lo = lane_offsets(lane);
    const int soff = q * T * (int)kRoundBytes;
    // Buffer resource over the row of step t (empty past the workgroup's rows:
    // its loads return zeros without touching memory).
    auto rsrc_for = [&](int t) {
        const int64_t m = (int64_t)t * P + p;  // row slot within the workgroup
        const bool in = m < wg_rows;
        const int n = in ? (int)a.row_bytes : 0;
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(row_addr(a, in ? g + m * G : 0)), (short)0, n,
                                                 0x00020000);
    };
    // Loads of round tt of this wave's slice.
    auto load_round = [&](__amdgpu_buffer_rsrc_t rs, int tt, Unit &u) {
        const int so = soff + tt * (int)kRoundBytes;
        u.sc = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)lo.ssq_sc, so, 0);
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)lo.ssq_d, so, 0);
        u.d[0] = v.x, u.d[1] = v.y, u.d[2] = v.z, u.d[3] = v.w;
    };

    // Step t from ut: per round, the twins' 8-slot dot products, scaled and
    // summed per lane; after round tt, load round tt of the next step into
    // nxt.  Then the lane sums are reduced and parked in LDS (half `half` of
    // the double buffer, step `local` of the window; steps past the
    // workgroup's last write nothing).
    auto step = [&](int t, int half, int local, const Unit (&ut)[T], Unit (&nxt)[T]) {
        const __amdgpu_buffer_rsrc_t rs_next = rsrc_for(t + 1);
        float acc[NS];
#pragma unroll
        for (int tt = 0; tt < T; tt++) {
            const Unit &u = ut[tt];
            float bs[NS];
            // slot c: dword c/2, halfword c%2; twin A = high byte, twin B = low
            // byte.  Each stream's chain is the same whatever NS is.
#pragma unroll
            for (int c = 0; c < UC; c++) {
                const uint32_t dw = u.d[c >> 1];
                const float wa = sbyte(dw, 2 * (c & 1) + 1), wb = sbyte(dw, 2 * (c & 1));
#pragma unroll
                for (int s = 0; s < NS; s++) {
                    const float wq = (s & 1) ? wb : wa;
                    bs[s] = c == 0 ? wq * xv[tt][c][s] : __builtin_fmaf(wq, xv[tt][c][s], bs[s]);
                }
            }
            const float da = f16_lo(u.sc), db = f16_hi(u.sc);
            // fma into +0 at the first round, as the Q8 kernels do: the
            // product is rounded before it enters the lane tree, so no
            // contraction of it into the tree's first add can change the bits
#pragma unroll
            for (int s = 0; s < NS; s++) {
                const float d = (s & 1) ? db : da;
                acc[s] = __builtin_fmaf(d, bs[s], tt == 0 ? 0.f : acc[s]);
            }
            __builtin_amdgcn_sched_barrier(0);
            load_round(rs_next, tt, nxt[tt]);
            __builtin_amdgcn_sched_barrier(0);
        }
        const int slot = (half * S + local) * P + p;  // row slot in the double buffer
        {
            // one tree for every stream; stream s's total lands in lane 64 - V + s
            constexpr int V = tree_width(NS);
            const float v = tree_sums<NS>(acc, lane);
            const int s = lane - (64 - V);
            if (s >= 0 && s < NS && t < steps)
                part[(slot * Q + q) * NS + s] = v;
        }
    };

    unsigned long long vkey[2] = {0, 0};  // this thread's largest key per twin (VERIFY)

    // Sum the partials of the rows of steps [t0, t1) (in half `half`) in slice
    // order and store them.
    auto flush = [&](int t0, int t1, int half) {
        __syncthreads();
        const int n = (t1 - t0) * P;
        // streams by a compile-time index (unrolled): a lane-varying index
        // into the argument array would load the output pointer from memory,
        // and that wait would also drain the weight loads in flight; a
        // residual launch's loads of every stream go out before any is used
        for (int r = tid; r < n; r += 64 * P * Q) {  // r: row slot relative to step t0
            const int64_t m = (int64_t)t0 * P + r;
            if (m >= wg_rows)
                continue;
            const int slot = half * S * P + r;
            const int64_t row = g + m * G;
            float rv[NS];
            if (a.res[0]) {  // uniform: a residual launch sets every stream's
#pragma unroll
                for (int s = 0; s < NS; s++)
                    rv[s] = a.res[s][row];
            }
#pragma unroll
            for (int s = 0; s < NS; s++) {
                float acc = part[(slot * Q) * NS + s];
                for (int j = 1; j < Q; j++)
                    acc += part[((slot * Q) + j) * NS + s];
                if (a.res[0])
                    acc = rv[s] + acc;
                a.y[s][row] = acc;
                if constexpr (VERIFY)
                    vkey[s & 1] = std::max(vkey[s & 1], verify_key(acc, row));
            }
        }
        // Stores count on the same counter as the weight loads.  Without this
        // wait the compiler cannot tell how many operations follow the
        // prefetched loads when the loop is re-entered, and it would make the
        // first step of every iteration wait for all of them; with it, the
        // count is known (one drain per flush).
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), other counters untouched
    };

    // x of this lane's units in rounds q T .. q T + T - 1, every stream (stream
    // s feeds twin A if s is even, twin B if odd), through a resource over the
    // row's units: past the last unit the loads return zero.
#pragma unroll
    for (int s = 0; s < NS; s++) {
        const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float *>(a.x[s]), (short)0, (int)(a.units * UC * 4), 0x00020000);
#pragma unroll
        for (int tt = 0; tt < T; tt++) {
            const int unit = (q * T + tt) * 64 + lane;
#pragma unroll
            for (int k = 0; k < UC / 4; k++) {
                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(xrs, (unit * UC + 4 * k) * 4, 0, 0);
#pragma unroll
                for (int e = 0; e < 4; e++)
                    xv[tt][4 * k + e][s] = __builtin_bit_cast(float, (uint32_t)v[e]);
            }
        }
    }
    // The first step's weights (2 loads per round), then a wait for x alone:
    // the loop is entered with exactly the loads of one step in flight, the
    // same as on every later iteration.  (Entered with x still in flight, the
    // loop's first step would wait for every load on each iteration.)
    Unit bufs[2][T];
    {
        // in the loop's order (scale, then slots, round by round), so the
        // loop's waits hold on entry as on every later iteration
        const __amdgpu_buffer_rsrc_t rs0 = rsrc_for(0);
#pragma unroll
        for (int tt = 0; tt < T; tt++) {
            __builtin_amdgcn_sched_barrier(0);
            load_round(rs0, tt, bufs[0][tt]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    static_assert(2 * T < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * T));  // vmcnt(2T), other counters untouched
    // Windows of S steps (S even, so step t always uses buffer t mod 2); the
    // last window is rounded up to an even count so the loop has a single
    // exit: an extra step falls past the workgroup's rows, loads through an
    // empty resource and writes nothing.
    int half = 0;
    for (int t0 = 0; t0 < steps; t0 += S, half ^= 1) {
        const int t1 = t0 + S < steps ? t0 + S : steps;
        const int iters = (t1 - t0 + 1) / 2;
        for (int it = 0; it < iters; it++) {
            const int local = 2 * it, tb = t0 + local;
            step(tb, half, local, bufs[0], bufs[1]);
            step(tb + 1, half, local + 1, bufs[1], bufs[0]);
        }
        flush(t0, t1, half);
    }

    if constexpr (VERIFY) {
        __shared__ unsigned long long wkey[2][kSplitMaxWaves];
        const int nw = P * Q;
#pragma unroll
        for (int s = 0; s < 2; s++) {
            const unsigned long long k = wave_umax(vkey[s]);
            if (lane == 63)
                wkey[s][wv] = k;
        }
        __syncthreads();
        if (tid < 2) {
            unsigned long long k = wkey[tid][0];
            for (int i = 1; i < nw; i++)
                k = std::max(k, wkey[tid][i]);
            sa.keys[2 * g + tid] = k;
        }
    }
}

// The rest of the fused verify: argmax of each twin from the workgroups' keys
// (the largest key is the largest value, the lowest row among equals) and the
// accept count of twin B's guess.  One wave: each lane takes the maximum of
// its workgroups' keys (all its loads in flight together), then the wave's.
__global__ __launch_bounds__(64) void verify_keys_kernel(const unsigned long long *__restrict__ keys, int n_groups,
                                                         const int32_t *__restrict__ tokens_in,
                                                         int32_t *__restrict__ argmax_out,
                                                         int32_t *__restrict__ accept_out)
{
    const int lane = threadIdx.x;
    unsigned long long k[2] = {0, 0};
#pragma unroll 4
    for (int i = lane; i < n_groups; i += 64) {
        const ulonglong2 v = reinterpret_cast<const ulonglong2 *>(keys)[i];
        k[0] = std::max(k[0], (unsigned long long)v.x);
        k[1] = std::max(k[1], (unsigned long long)v.y);
    }
    k[0] = wave_umax(k[0]);
    k[1] = wave_umax(k[1]);
    if (lane == 63) {
        int32_t am[2];
#pragma unroll
        for (int s = 0; s < 2; s++) {
            am[s] = (int32_t)(0xFFFFFFFFu - (uint32_t)(k[s] & 0xFFFFFFFFull));
            argmax_out[s] = am[s];
        }
        accept_out[0] = 1 + (tokens_in[1] == am[0] ? 1 : 0);
    }
}

// The same for a per-wave-row launch's keys of n streams (keys[kKeyStride g +
// s]): each stream's argmax and the accept count of the staggered streams, 1
// + the leading run of tokens_in[i] == argmax[i - 1], as pti_verify_argmax
// gives them.
__global__ __launch_bounds__(64) void verify_keys_n_kernel(const unsigned long long *__restrict__ keys, int n_groups,
                                                           int n, const int32_t *__restrict__ tokens_in,
                                                           int32_t *__restrict__ argmax_out,
                                                           int32_t *__restrict__ accept_out)
{
    const int lane = threadIdx.x;
    unsigned long long k[kKeyStride] = {0, 0, 0, 0};
#pragma unroll 4
    for (int i = lane; i < n_groups; i += 64) {
        const ulonglong2 *g = reinterpret_cast<const ulonglong2 *>(keys + (size_t)kKeyStride * i);
        const ulonglong2 v0 = g[0], v1 = g[1];
        k[0] = std::max(k[0], (unsigned long long)v0.x);
        k[1] = std::max(k[1], (unsigned long long)v0.y);
        k[2] = std::max(k[2], (unsigned long long)v1.x);
        k[3] = std::max(k[3], (unsigned long long)v1.y);
    }
#pragma unroll
    for (int s = 0; s < kKeyStride; s++)
        k[s] = wave_umax(k[s]);
    if (lane == 63) {
        int32_t am[kKeyStride];
#pragma unroll
        for (int s = 0; s < kKeyStride; s++) {
            am[s] = (int32_t)(0xFFFFFFFFu - (uint32_t)(k[s] & 0xFFFFFFFFull));
            if (s < n)
                argmax_out[s] = am[s];
        }
        int acc = 1;
#pragma unroll
        for (int s = 1; s < kKeyStride; s++)
            if (s < n && acc == s && tokens_in[s] == am[s - 1])
                acc++;
        accept_out[0] = acc;
    }
}

// Rounds per wave for a row of `rounds` rounds: at most kSplitTMax, spread
// evenly over the fewest waves.
int split_T(int rounds)
{
    const int q = (rounds + kSplitTMax - 1) / kSplitTMax;
    return (rounds + q - 1) / q;
}

// Geometry for T, or false if the row needs more waves than a workgroup may
// have.  S: steps per flush, even, with the partials' double buffer at most
// 32 KB of LDS.
bool split_shape(int rounds, int T, int ns, SplitArgs &sa)
{
    const int Q = (rounds + T - 1) / T, W = split_bound_waves(T);
    if (rounds < 1 || Q > W)
        return false;
    sa.Q = Q;
    sa.P = std::max(1, std::min(W, T >= 3 ? kSplitWavesBigT : kSplitWavesSmallT) / Q);
    int S = 64;
    while (S > 2 && 2 * S * sa.P * Q * ns * 4 > 32 * 1024)
        S -= 2;
    sa.S = S;
    return true;
}

constexpr int kNotSplit = 1;  // the row-split kernel does not take this shape

// Outputs of the fused verify (VERIFY launches only).
struct VerifyOut {
    unsigned long long *keys;  // workspace, 2 keys per workgroup
    const int32_t *tokens_in;
    int32_t *argmax_out, *accept_out;
};

template <int T, int NS, bool VERIFY>
int launch_ssq_split(const GemvArgs &a, const VerifyOut *vo, hipStream_t stream)
{
    SplitArgs sa{};
    if (!split_shape(a.rounds, T, NS, sa))
        return kNotSplit;
    sa.g = a;
    if constexpr (VERIFY)
        sa.keys = vo->keys;
    const int cus = device_cus();
    if (cus <= 0) {
        pti::set_hip_error(hipGetLastError());
        return PTI_ERR_HIP;
    }
    const int64_t grid = std::min<int64_t>(std::min(cus, kSplitMaxGrid), a.rows);
    const size_t lds = (size_t)2 * sa.S * sa.P * sa.Q * NS * sizeof(float);
    bool small = false;
    if constexpr (NS == 4)
        small = sa.P * sa.Q <= 4;
    if constexpr (NS == 4) {
        if (small)
            hipLaunchKernelGGL((gemv_ssq_split_kernel<T, NS, VERIFY, 4>), dim3((unsigned)grid),
                               dim3((unsigned)(64 * sa.P * sa.Q)), lds, stream, sa);
    }
    if (!small)
        hipLaunchKernelGGL((gemv_ssq_split_kernel<T, NS, VERIFY>), dim3((unsigned)grid),
                           dim3((unsigned)(64 * sa.P * sa.Q)), lds, stream, sa);
    if constexpr (VERIFY)
        hipLaunchKernelGGL(verify_keys_kernel, dim3(1), dim3(64), 0, stream, vo->keys, (int)grid, vo->tokens_in,
                           vo->argmax_out, vo->accept_out);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        pti::set_hip_error(e);
        return PTI_ERR_HIP;
    }
    return PTI_OK;
}

// vo: the verify outputs (VERIFY only, else null).  NS: 2 (one stream per
// twin) or 4 (two per twin).
template <int NS, bool VERIFY>
int launch_ssq_split(const GemvArgs &a, const VerifyOut *vo, hipStream_t stream)
{
    switch (split_T(a.rounds)) {
    case 1: return launch_ssq_split<1, NS, VERIFY>(a, vo, stream);
    case 2: return launch_ssq_split<2, NS, VERIFY>(a, vo, stream);
    case 3: return launch_ssq_split<3, NS, VERIFY>(a, vo, stream);
    case 4: return launch_ssq_split<4, NS, VERIFY>(a, vo, stream);
    default: return launch_ssq_split<5, NS, VERIFY>(a, vo, stream);
    }
}

// Q8 form of the row-split kernel, for rows of an even number of blocks (so
// every row starts on a dword) and at most kQ8SplitMaxQ waves per row.  The
// same geometry as the SSQ kernel -- workgroup g owns rows g, g + G, ...;
// the Q waves of a row each take T consecutive rounds; loads run one step
// ahead, round by round -- with Q8 units: 16 columns per lane, two lanes per
// 34-byte block, the quants realigned with v_alignbyte.  Each of the NS
// streams (up to four) keeps its x slice in registers (80 per stream at
// T = 5), which a bound of four waves per workgroup leaves room for.  A
// stream's chain (16 products in column order per unit, scaled into the
// lane's sum per round, the lane tree, the Q partials in slice order) is the
// same whatever NS is.
constexpr int kQ8SplitMaxQ = 4;
constexpr int64_t kQ8SplitMaxRows = 8192;

template <int T, int NS>
__global__ __launch_bounds__(64 * 4) void gemv_q8_split_kernel(SplitArgs sa)
{
    constexpr int UC = unit_cols<kQ8>();
    const GemvArgs &a = sa.g;
    const int P = sa.P, Q = sa.Q, S = sa.S;
    extern __shared__ float part[];  // [2][S * P][Q][NS]: row partials, double-buffered
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int p = wv / Q, q = wv - (wv / Q) * Q;
    const int64_t G = gridDim.x, g = blockIdx.x;
    const int64_t wg_rows = g < a.rows ? (a.rows - g + G - 1) / G : 0;
    const int steps = (int)((wg_rows + P - 1) / P);

    float xv[T][UC][NS];  // this lane's x (filled below)
    const LaneOffsets lo = lane_offsets(lane);
    const int soff = q * T * (int)kRoundBytes;
    // Paired loads (PL): the two lanes of a block read its nine aligned dwords
    // W0..W8 with one b128 each (its quants' window: W0-3 and W4-7 in an even
    // block of the round, which starts on a dword; W1-4 and W5-8 in an odd
    // one, which starts 2 bytes into W0) and one b32 between them (W8 by the
    // second lane of an even block, W0 by the first lane of an odd one; the
    // other lane's b32 points past the buffer and reads nothing), then swap
    // one dword: the first lane's W0 (the scale) and the second lane's first
    // b128 dword (W4, the first lane's fifth quant dword in an even block).
    // Each lane then holds the bytes the three loads per lane would give it
    // (the fifth dword only where its quants start 2 bytes in), so the
    // arithmetic is unchanged; two load instructions per round instead of
    // three.
    constexpr bool PL = NS <= PTI_Q8_PAIRED_MAX_NS;
    const bool second = lane & 1, odd_block = (lane >> 1) & 1;
    const bool sends_extra = !second && odd_block;  // the first lane of an odd block holds W0 in its b32
    const uint32_t xoff = odd_block ? (second ? kPastBuffer : lo.q_sc[0]) : (second ? lo.q_sc[0] + 32 : kPastBuffer);
    auto rsrc_for = [&](int t) {
        const int64_t m = (int64_t)t * P + p;
        const bool in = m < wg_rows;
        const int n = in ? (int)a.row_bytes : 0;
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(row_addr(a, in ? g + m * G : 0)), (short)0, n,
                                                 0x00020000);
    };
    // Loads of round tt: the scale's dword, the 16 quants (4 + 1 dwords);
    // paired: the b128 and the lane's b32 (in d[4]), sc unused.
    auto load_round = [&](__amdgpu_buffer_rsrc_t rs, int tt, Unit &u) {
        const int so = soff + tt * (int)kRoundBytes;
        if constexpr (!PL)
            u.sc = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)lo.q_sc[0], so, 0);
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)lo.q_d[0], so, 0);
        u.d[0] = v.x, u.d[1] = v.y, u.d[2] = v.z, u.d[3] = v.w;
        u.d[4] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)(PL ? xoff : lo.q_h[0]), so, 0);
    };

    auto step = [&](int t, int half, int local, const Unit (&ut)[T], Unit (&nxt)[T]) {
        const __amdgpu_buffer_rsrc_t rs_next = rsrc_for(t + 1);
        float acc[NS];
#pragma unroll
        for (int tt = 0; tt < T; tt++) {
            const Unit &u = ut[tt];
            uint32_t sc = u.sc, d4 = u.d[4];
            if constexpr (PL) {
                const uint32_t send = sends_extra ? u.d[4] : u.d[0];
                const uint32_t got = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send, 0xB1, 0xf, 0xf, false);
                sc = second ? got : send;
                d4 = second ? u.d[4] : got;
            }
            uint32_t qd[4];
#pragma unroll
            for (int k = 0; k < 4; k++)
                qd[k] = __builtin_amdgcn_alignbyte(k < 3 ? u.d[k + 1] : d4, u.d[k], lo.q_sh[0]);
            float bs[NS];
#pragma unroll
            for (int c = 0; c < UC; c++) {
                const float wq = sbyte(qd[c >> 2], c & 3);
#pragma unroll
                for (int s = 0; s < NS; s++)
                    bs[s] = c == 0 ? wq * xv[tt][c][s] : __builtin_fmaf(wq, xv[tt][c][s], bs[s]);
            }
            const float d = f16_lo(sc >> lo.q_ssh[0]);
            // fma into +0 at the first round, as the per-wave-row kernel does
            // (d * bs would keep a -0 that it turns into +0)
#pragma unroll
            for (int s = 0; s < NS; s++)
                acc[s] = __builtin_fmaf(d, bs[s], tt == 0 ? 0.f : acc[s]);
            __builtin_amdgcn_sched_barrier(0);
            load_round(rs_next, tt, nxt[tt]);
            __builtin_amdgcn_sched_barrier(0);
        }
        const int slot = (half * S + local) * P + p;
        {
            // one tree for every stream; stream s's total lands in lane 64 - V + s
            constexpr int V = tree_width(NS);
            const float v = tree_sums<NS>(acc, lane);
            const int s = lane - (64 - V);
            if (s >= 0 && s < NS && t < steps)
                part[(slot * Q + q) * NS + s] = v;
        }
    };

    auto flush = [&](int t0, int t1, int half) {
        __syncthreads();
        const int n = (t1 - t0) * P;
        for (int r = tid; r < n; r += 64 * P * Q) {  // as in the SSQ kernel
            const int64_t m = (int64_t)t0 * P + r;
            if (m >= wg_rows)
                continue;
            const int slot = half * S * P + r;
            const int64_t row = g + m * G;
            float rv[NS];
            if (a.res[0]) {  // uniform: a residual launch sets every stream's
#pragma unroll
                for (int s = 0; s < NS; s++)
                    rv[s] = a.res[s][row];
            }
#pragma unroll
            for (int s = 0; s < NS; s++) {
                float acc = part[(slot * Q) * NS + s];
                for (int j = 1; j < Q; j++)
                    acc += part[((slot * Q) + j) * NS + s];
                if (a.res[0])
                    acc = rv[s] + acc;
                a.y[s][row] = acc;
            }
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): see the SSQ kernel
    };

    // x first, then the first step's weights in the loop's order, then a wait
    // for x alone, so the loop is entered as every iteration ends.
#pragma unroll
    for (int s = 0; s < NS; s++) {
        const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float *>(a.x[s]), (short)0, (int)(a.units * UC * 4), 0x00020000);
#pragma unroll
        for (int tt = 0; tt < T; tt++) {
            const int unit = (q * T + tt) * 64 + lane;
#pragma unroll
            for (int k = 0; k < UC / 4; k++) {
                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(xrs, (unit * UC + 4 * k) * 4, 0, 0);
#pragma unroll
                for (int e = 0; e < 4; e++)
                    xv[tt][4 * k + e][s] = __builtin_bit_cast(float, (uint32_t)v[e]);
            }
        }
    }
    Unit bufs[2][T];
    {
        const __amdgpu_buffer_rsrc_t rs0 = rsrc_for(0);
#pragma unroll
        for (int tt = 0; tt < T; tt++) {
            __builtin_amdgcn_sched_barrier(0);
            load_round(rs0, tt, bufs[0][tt]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    constexpr int kLoads = (PL ? 2 : 3) * T;  // weight loads of one step
    static_assert(kLoads < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0F70 | kLoads);  // vmcnt(kLoads): the x loads are done

    int half = 0;
    for (int t0 = 0; t0 < steps; t0 += S, half ^= 1) {
        const int t1 = t0 + S < steps ? t0 + S : steps;
        const int iters = (t1 - t0 + 1) / 2;
        for (int it = 0; it < iters; it++) {
            const int local = 2 * it, tb = t0 + local;
            step(tb, half, local, bufs[0], bufs[1]);
            step(tb + 1, half, local + 1, bufs[1], bufs[0]);
        }
        flush(t0, t1, half);
    }
}

template <int T, int NS>
int launch_q8_split(const GemvArgs &a, hipStream_t stream)
{
    SplitArgs sa{};
    sa.Q = (a.rounds + T - 1) / T;
    if (sa.Q > kQ8SplitMaxQ)
        return kNotSplit;
    sa.P = std::max(1, 4 / sa.Q);
    int S = 64;
    while (S > 2 && 2 * S * sa.P * sa.Q * NS * 4 > 32 * 1024)
        S -= 2;
    sa.S = S;
    sa.g = a;
    const int cus = device_cus();
    if (cus <= 0) {
        pti::set_hip_error(hipGetLastError());
        return PTI_ERR_HIP;
    }
    const int64_t grid = std::min<int64_t>(std::min(cus, kSplitMaxGrid), a.rows);
    const size_t lds = (size_t)2 * sa.S * sa.P * sa.Q * NS * sizeof(float);
    hipLaunchKernelGGL((gemv_q8_split_kernel<T, NS>), dim3((unsigned)grid), dim3((unsigned)(64 * sa.P * sa.Q)), lds,
                       stream, sa);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        pti::set_hip_error(e);
        return PTI_ERR_HIP;
    }
    return PTI_OK;
}

template <int NS>
int launch_q8_split(const GemvArgs &a, hipStream_t stream)
{
    switch (split_T(a.rounds)) {
    case 1: return launch_q8_split<1, NS>(a, stream);
    case 2: return launch_q8_split<2, NS>(a, stream);
    case 3: return launch_q8_split<3, NS>(a, stream);
    case 4: return launch_q8_split<4, NS>(a, stream);
    default: return launch_q8_split<5, NS>(a, stream);
    }
}

// Taller Q8 matrices take the per-wave-row kernel, except that with one or
// two streams a matrix whose rows take one wave of four or five rounds in the
// row-split kernel takes that kernel (measured faster there: 18.7 against
// 20.1 us at 17408 x 5120, one stream).  With one wave per row the two
// kernels do the same operations in the same order -- the lane's 16-column
// sums, the scale FMAs into +0 then the running sum, round by round, the same
// 64-lane tree, and no further sum -- so a stream's bits do not depend on
// which of them ran, and the choice may follow the stream count.
constexpr int kQ8TallSplitMaxStreams = 2;
constexpr int kQ8TallSplitMinRounds = 4;  // two rounds measured slower split (32000 x 2048)

bool q8_tall_split(const GemvArgs &a, int n_streams)
{
    return n_streams <= kQ8TallSplitMaxStreams && a.rounds >= kQ8TallSplitMinRounds &&
           split_T(a.rounds) == a.rounds;
}

// Kernel choice of each format: by shape, and by the stream count only
// between kernels that give the same bits (above).
int launch_q8(const GemvArgs &a, int n_streams, hipStream_t st)
{
    // rows start on dword boundaries when a row holds an even number of blocks
    if ((a.cols / PTI_BLOCK) % 2 == 0) {
        int rc = kNotSplit;
        // the row-split form for matrices of up to kQ8SplitMaxRows rows; the
        // per-wave-row kernel, whose many waves hide more latency, for taller
        // ones (measured: it is faster there at four streams)
        if (a.rows <= kQ8SplitMaxRows || q8_tall_split(a, n_streams))
            switch (n_streams) {
            case 1: rc = launch_q8_split<1>(a, st); break;
            case 2: rc = launch_q8_split<2>(a, st); break;
            case 3: rc = launch_q8_split<3>(a, st); break;
            default: rc = launch_q8_split<4>(a, st); break;
            }
        if (rc != kNotSplit)
            return rc;
        switch (n_streams) {
        case 1: return launch<kQ8, 1, 1, true>(a, st);
        case 2: return launch<kQ8, 2, 2, true>(a, st);
        case 3: return launch<kQ8, 4, 3, true>(a, st);
        default: return launch<kQ8, 4, 4, true>(a, st);
        }
    }
    switch (n_streams) {
    case 1: return launch<kQ8, 1, 1, false>(a, st);
    case 2: return launch<kQ8, 2, 2, false>(a, st);
    case 3: return launch<kQ8, 4, 3, false>(a, st);
    default: return launch<kQ8, 4, 4, false>(a, st);
    }
}

// n_per_twin: streams per twin (1 or 2); a.x / a.y hold stream s at s, twin
// A for even s and twin B for odd s.  The kernel choice depends on the shape
// alone, so a (twin, stream) output does not depend on n_per_twin.
int launch_ssq(const GemvArgs &a, int n_per_twin, hipStream_t st)
{
    const int rc = n_per_twin == 1 ? launch_ssq_split<2, false>(a, nullptr, st)
                                   : launch_ssq_split<4, false>(a, nullptr, st);
    if (rc != kNotSplit)
        return rc;
    return n_per_twin == 1 ? launch<kSSQ, 2, 2, true>(a, st) : launch<kSSQ, 4, 4, true>(a, st);
}

// A grouped launch's matrices: validated, then stacked into one row space.
// bytes(rows, cols): the packed size of one matrix.  Checks: host arrays
// present, 1 <= n <= PTI_MAX_GROUP, every matrix present, 4-byte aligned,
// 1 <= rows[m], and the stacked shape within the limits; the outputs must
// not overlap any matrix.
template <int FMT>
int group_args(const void *const *w, const int64_t *rows, int n, int64_t cols, const pti::Range *outs, int n_outs,
               GemvArgs &a)
{
    if (!w || !rows)
        return PTI_ERR_NULL;
    if (n < 1 || n > PTI_MAX_GROUP)
        return PTI_ERR_SHAPE;
    int64_t total = 0;
    for (int m = 0; m < n; m++) {
        if (!w[m])
            return PTI_ERR_NULL;
        if (rows[m] < 1 || rows[m] > PTI_MAX_ROWS - total)
            return PTI_ERR_SHAPE;
        total += rows[m];
    }
    if (!pti::shape_ok(total, cols))
        return PTI_ERR_SHAPE;
    for (int m = 0; m < n; m++) {
        if (!pti::aligned(w[m], 4))
            return PTI_ERR_ALIGN;
        const size_t wn = FMT == kSSQ ? pti_ssq_bytes(rows[m], cols) : pti_q8_bytes(rows[m], cols);
        for (int o = 0; o < n_outs; o++)
            if (pti::overlap(outs[o], {w[m], wn}))
                return PTI_ERR_OVERLAP;
    }
    a = make_args<FMT>(w[0], total, cols);
    int64_t start = 0;
    for (int m = 0; m < n; m++) {
        a.seg_base[m] = reinterpret_cast<uintptr_t>(w[m]) - (uintptr_t)start * (uintptr_t)a.row_bytes;
        start += rows[m];
        a.seg_end[m] = m + 1 < n ? start : INT64_MAX;
    }
    for (int m = n; m < kMaxSegs; m++)
        a.seg_base[m] = a.seg_base[n - 1], a.seg_end[m] = INT64_MAX;
    return PTI_OK;
}

// Whether the Q8 GEMV of stacked rows a (n streams) takes the per-wave-row
// kernel with all of x staged at once, the kernel that can normalise x as it
// stages it (otherwise the shape takes the row-split kernel at every stream
// count, or x does not fit in LDS).
bool q8_norm_fusable(const GemvArgs &a, int n)
{
    const bool even = (a.cols / PTI_BLOCK) % 2 == 0;
    if (even && a.rows <= kQ8SplitMaxRows && (a.rounds + split_T(a.rounds) - 1) / split_T(a.rounds) <= kQ8SplitMaxQ)
        return false;
    const int nsp = n == 1 ? 1 : n == 2 ? 2 : 4;
    return a.rounds * 64 * unit_cols<kQ8>() * nsp * 4 <= kXLds;
}

}  // namespace

extern "C" {

int pti_gemv_ssq(const void *w_ssq, const float *x_a, const float *x_b, float *y_a, float *y_b, int64_t rows,
                 int64_t cols, void *stream)
{
    if (!w_ssq || !x_a || !x_b || !y_a || !y_b)
        return PTI_ERR_NULL;
    if (!pti::shape_ok(rows, cols))
        return PTI_ERR_SHAPE;
    if (!pti::aligned(w_ssq, 4) || !pti::aligned(x_a, 16) || !pti::aligned(x_b, 16) || !pti::aligned(y_a, 4) ||
        !pti::aligned(y_b, 4))
        return PTI_ERR_ALIGN;
    const size_t wn = pti_ssq_bytes(rows, cols), xn = size_t(cols) * 4, yn = size_t(rows) * 4;
    const pti::Range ya{y_a, yn}, yb{y_b, yn};
    if (pti::overlap(ya, yb) || pti::overlap(ya, {w_ssq, wn}) || pti::overlap(yb, {w_ssq, wn}) ||
        pti::overlap(ya, {x_a, xn}) || pti::overlap(ya, {x_b, xn}) || pti::overlap(yb, {x_a, xn}) ||
        pti::overlap(yb, {x_b, xn}))
        return PTI_ERR_OVERLAP;
    GemvArgs a = make_args<kSSQ>(w_ssq, rows, cols);
    a.x[0] = x_a, a.x[1] = x_b;
    a.y[0] = y_a, a.y[1] = y_b;
    return launch_ssq(a, 1, static_cast<hipStream_t>(stream));
}

int pti_gemv_ssq_multi(const void *w_ssq, const float *x_a, const float *x_b, float *y_a, float *y_b, int64_t rows,
                       int64_t cols, int n_per_twin, void *stream)
{
    if (!w_ssq || !x_a || !x_b || !y_a || !y_b)
        return PTI_ERR_NULL;
    if (!pti::shape_ok(rows, cols))
        return PTI_ERR_SHAPE;
    if (n_per_twin < 1 || 2 * n_per_twin > PTI_MAX_STREAMS)
        return PTI_ERR_NSTREAMS;
    if (!pti::aligned(w_ssq, 4) || !pti::aligned(x_a, 16) || !pti::aligned(x_b, 16) || !pti::aligned(y_a, 4) ||
        !pti::aligned(y_b, 4))
        return PTI_ERR_ALIGN;
    const size_t n = size_t(n_per_twin), wn = pti_ssq_bytes(rows, cols), xn = n * cols * 4, yn = n * rows * 4;
    const pti::Range ya{y_a, yn}, yb{y_b, yn};
    if (pti::overlap(ya, yb) || pti::overlap(ya, {w_ssq, wn}) || pti::overlap(yb, {w_ssq, wn}) ||
        pti::overlap(ya, {x_a, xn}) || pti::overlap(ya, {x_b, xn}) || pti::overlap(yb, {x_a, xn}) ||
        pti::overlap(yb, {x_b, xn}))
        return PTI_ERR_OVERLAP;
    GemvArgs a = make_args<kSSQ>(w_ssq, rows, cols);
    for (int j = 0; j < n_per_twin; j++) {
        a.x[2 * j] = x_a + (size_t)j * cols, a.x[2 * j + 1] = x_b + (size_t)j * cols;
        a.y[2 * j] = y_a + (size_t)j * rows, a.y[2 * j + 1] = y_b + (size_t)j * rows;
    }
    return launch_ssq(a, n_per_twin, static_cast<hipStream_t>(stream));
}

int pti_gemv_ssq_grouped(const void *const *w_ssq, const int64_t *rows, int n_mats, const float *x_a,
                         const float *x_b, float *y_a, float *y_b, int64_t cols, void *stream)
{
    if (!x_a || !x_b || !y_a || !y_b)
        return PTI_ERR_NULL;
    int64_t total = 0;  // for the overlap ranges; the arrays are read only once n_mats is in range
    for (int m = 0; rows && n_mats >= 1 && n_mats <= PTI_MAX_GROUP && m < n_mats; m++)
        total += rows[m] > 0 ? std::min<int64_t>(rows[m], PTI_MAX_ROWS) : 0;
    const size_t yn = size_t(total) * 4, xn = size_t(cols > 0 ? cols : 0) * 4;
    const pti::Range outs[] = {{y_a, yn}, {y_b, yn}};
    GemvArgs a;
    const int rc = group_args<kSSQ>(w_ssq, rows, n_mats, cols, outs, 2, a);
    if (rc != PTI_OK)
        return rc;
    if (!pti::aligned(x_a, 16) || !pti::aligned(x_b, 16) || !pti::aligned(y_a, 4) || !pti::aligned(y_b, 4))
        return PTI_ERR_ALIGN;
    if (pti::overlap(outs[0], outs[1]) || pti::overlap(outs[0], {x_a, xn}) || pti::overlap(outs[0], {x_b, xn}) ||
        pti::overlap(outs[1], {x_a, xn}) || pti::overlap(outs[1], {x_b, xn}))
        return PTI_ERR_OVERLAP;
    a.x[0] = x_a, a.x[1] = x_b;
    a.y[0] = y_a, a.y[1] = y_b;
    return launch_ssq(a, 1, static_cast<hipStream_t>(stream));
}

int pti_gemv_ssq_verify(const void *w_ssq, const float *x_a, const float *x_b, float *y_a, float *y_b, int64_t rows,
                        int64_t cols, const int32_t *tokens_in, int32_t *argmax_out, int32_t *accept_out, void *work,
                        size_t work_bytes, void *stream)
{
    if (!w_ssq || !x_a || !x_b || !y_a || !y_b || !tokens_in || !argmax_out || !accept_out || !work)
        return PTI_ERR_NULL;
    if (!pti::shape_ok(rows, cols))
        return PTI_ERR_SHAPE;
    if (work_bytes < PTI_SSQ_VERIFY_WORK_BYTES)
        return PTI_ERR_SHAPE;
    if (!pti::aligned(w_ssq, 4) || !pti::aligned(x_a, 16) || !pti::aligned(x_b, 16) || !pti::aligned(y_a, 4) ||
        !pti::aligned(y_b, 4) || !pti::aligned(tokens_in, 4) || !pti::aligned(argmax_out, 4) ||
        !pti::aligned(accept_out, 4) || !pti::aligned(work, 16))
        return PTI_ERR_ALIGN;
    const size_t wn = pti_ssq_bytes(rows, cols), xn = size_t(cols) * 4, yn = size_t(rows) * 4;
    // every output against every other output and every input
    const pti::Range outs[] = {{y_a, yn}, {y_b, yn}, {argmax_out, 8}, {accept_out, 4},
                               {work, PTI_SSQ_VERIFY_WORK_BYTES}};
    const pti::Range ins[] = {{w_ssq, wn}, {x_a, xn}, {x_b, xn}, {tokens_in, 8}};
    for (size_t i = 0; i < sizeof outs / sizeof outs[0]; i++) {
        for (size_t j = i + 1; j < sizeof outs / sizeof outs[0]; j++)
            if (pti::overlap(outs[i], outs[j]))
                return PTI_ERR_OVERLAP;
        for (const pti::Range &in : ins)
            if (pti::overlap(outs[i], in))
                return PTI_ERR_OVERLAP;
    }
    const hipStream_t st = static_cast<hipStream_t>(stream);
    GemvArgs a = make_args<kSSQ>(w_ssq, rows, cols);
    a.x[0] = x_a, a.x[1] = x_b;
    a.y[0] = y_a, a.y[1] = y_b;
    const VerifyOut vo{static_cast<unsigned long long *>(work), tokens_in, argmax_out, accept_out};
    const int rc = launch_ssq_split<2, true>(a, &vo, st);
    if (rc != kNotSplit)
        return rc;
    // shapes the row-split kernel does not take: GEMV, then the verify kernel
    const int g = launch<kSSQ, 2, 2, true>(a, st);
    if (g != PTI_OK)
        return g;
    pti::StreamRows lg{};
    lg.p[0] = y_a, lg.p[1] = y_b;
    return pti::launch_verify_rows(lg, tokens_in, argmax_out, accept_out, rows, 2, stream);
}

int pti_gemv_q8_multi(const void *w_q8, const float *x, float *y, int64_t rows, int64_t cols, int n_streams,
                      void *stream)
{
    if (!w_q8 || !x || !y)
        return PTI_ERR_NULL;
    if (!pti::shape_ok(rows, cols))
        return PTI_ERR_SHAPE;
    if (n_streams < 1 || n_streams > PTI_MAX_STREAMS)
        return PTI_ERR_NSTREAMS;
    if (!pti::aligned(w_q8, 4) || !pti::aligned(x, 16) || !pti::aligned(y, 4))
        return PTI_ERR_ALIGN;
    const size_t wn = pti_q8_bytes(rows, cols), xn = size_t(n_streams) * cols * 4,
                 yn = size_t(n_streams) * rows * 4;
    if (pti::overlap({y, yn}, {w_q8, wn}) || pti::overlap({y, yn}, {x, xn}))
        return PTI_ERR_OVERLAP;
    GemvArgs a = make_args<kQ8>(w_q8, rows, cols);
    for (int s = 0; s < n_streams; s++) {
        a.x[s] = x + (size_t)s * cols;
        a.y[s] = y + (size_t)s * rows;
    }
    return launch_q8(a, n_streams, static_cast<hipStream_t>(stream));
}

int pti_gemv_q8_multi_grouped(const void *const *w_q8, const int64_t *rows, int n_mats, const float *x, float *y,
                              int64_t cols, int n_streams, void *stream)
{
    if (!x || !y)
        return PTI_ERR_NULL;
    if (n_streams < 1 || n_streams > PTI_MAX_STREAMS)
        return PTI_ERR_NSTREAMS;
    int64_t total = 0;  // for the overlap ranges; the arrays are read only once n_mats is in range
    for (int m = 0; rows && n_mats >= 1 && n_mats <= PTI_MAX_GROUP && m < n_mats; m++)
        total += rows[m] > 0 ? std::min<int64_t>(rows[m], PTI_MAX_ROWS) : 0;
    const size_t yn = size_t(n_streams) * total * 4, xn = size_t(n_streams) * (cols > 0 ? cols : 0) * 4;
    const pti::Range outs[] = {{y, yn}};
    GemvArgs a;
    const int rc = group_args<kQ8>(w_q8, rows, n_mats, cols, outs, 1, a);
    if (rc != PTI_OK)
        return rc;
    if (!pti::aligned(x, 16) || !pti::aligned(y, 4))
        return PTI_ERR_ALIGN;
    if (pti::overlap(outs[0], {x, xn}))
        return PTI_ERR_OVERLAP;
    for (int s = 0; s < n_streams; s++) {
        a.x[s] = x + (size_t)s * cols;
        a.y[s] = y + (size_t)s * a.rows;
    }
    return launch_q8(a, n_streams, static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace pti {

int gemv_q8_res(const void *w, const float *x, float *y, const float *res, int64_t rows, int64_t cols, int n,
                void *stream)
{
    GemvArgs a = make_args<kQ8>(w, rows, cols);
    for (int s = 0; s < n; s++) {
        a.x[s] = x + (size_t)s * cols;
        a.y[s] = y + (size_t)s * rows;
        a.res[s] = res + (size_t)s * rows;
    }
    return launch_q8(a, n, static_cast<hipStream_t>(stream));
}


int q8_gemv_rmsnorm(const void *const *w, const int64_t *rows, int n_mats, const float *x, float *y, int64_t cols,
                    int n, float eps, void *stream, unsigned long long *keys)
{
    GemvArgs a;
    const int rc = group_args<kQ8>(w, rows, n_mats, cols, nullptr, 0, a);
    if (rc != PTI_OK)
        return rc;
    a.keys = keys;
    const bool even = (a.cols / PTI_BLOCK) % 2 == 0;
    if (!q8_norm_fusable(a, n))
        return kNormNotFused;
    for (int s = 0; s < n; s++) {
        a.x[s] = x + (size_t)s * cols;
        a.y[s] = y + (size_t)s * a.rows;
    }
    a.norm = 1;
    a.norm_eps = double(eps);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    switch (n) {
    case 1: return even ? launch<kQ8, 1, 1, true>(a, st) : launch<kQ8, 1, 1, false>(a, st);
    case 2: return even ? launch<kQ8, 2, 2, true>(a, st) : launch<kQ8, 2, 2, false>(a, st);
    case 3: return even ? launch<kQ8, 4, 3, true>(a, st) : launch<kQ8, 4, 3, false>(a, st);
    default: return even ? launch<kQ8, 4, 4, true>(a, st) : launch<kQ8, 4, 4, false>(a, st);
    }
}

int64_t rowwise_groups(int64_t rows)
{
    const int cus = device_cus();
    return cus > 0 ? std::min<int64_t>(cus, rows) : 0;
}

int launch_verify_keys_n(const unsigned long long *keys, int n_groups, int n, const int32_t *tokens_in,
                         int32_t *argmax_out, int32_t *accept_out, void *stream)
{
    hipLaunchKernelGGL(verify_keys_n_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), keys, n_groups, n,
                       tokens_in, argmax_out, accept_out);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        pti::set_hip_error(e);
        return PTI_ERR_HIP;
    }
    return PTI_OK;
}

int q8_gate_up_silu(const void *gate, const void *up, int64_t ffn, const float *x, float *y, int64_t cols, int n,
                    float eps, void *stream)
{
    const void *w[2] = {gate, up};
    const int64_t rows[2] = {ffn, ffn};
    GemvArgs a;
    const int rc = group_args<kQ8>(w, rows, 2, cols, nullptr, 0, a);
    if (rc != PTI_OK)
        return rc;
    // the shapes whose gate|up GEMV fuses the norm: the same kernel and rows,
    // so gate and up keep the bits of that GEMV
    const bool even = (a.cols / PTI_BLOCK) % 2 == 0;
    if (!q8_norm_fusable(a, n))
        return kNormNotFused;
    a.rows = ffn;  // row pairs
    a.seg_base[0] = reinterpret_cast<uintptr_t>(gate);
    a.seg_base[1] = reinterpret_cast<uintptr_t>(up);
    for (int s = 0; s < n; s++) {
        a.x[s] = x + (size_t)s * cols;
        a.y[s] = y + (size_t)s * ffn;
    }
    a.norm = 1;
    a.norm_eps = double(eps);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    switch (n) {
    case 1: return even ? launch<kQ8, 1, 1, true, true>(a, st) : launch<kQ8, 1, 1, false, true>(a, st);
    case 2: return even ? launch<kQ8, 2, 2, true, true>(a, st) : launch<kQ8, 2, 2, false, true>(a, st);
    case 3: return even ? launch<kQ8, 4, 3, true, true>(a, st) : launch<kQ8, 4, 3, false, true>(a, st);
    default: return even ? launch<kQ8, 4, 4, true, true>(a, st) : launch<kQ8, 4, 4, false, true>(a, st);
    }
}

int gemv_ssq_res(const void *w, const float *x_a, const float *x_b, float *y_a, float *y_b, const float *res_a,
                 const float *res_b, int64_t rows, int64_t cols, void *stream)
{
    GemvArgs a = make_args<kSSQ>(w, rows, cols);
    a.x[0] = x_a, a.x[1] = x_b;
    a.y[0] = y_a, a.y[1] = y_b;
    a.res[0] = res_a, a.res[1] = res_b;
    return launch_ssq(a, 1, static_cast<hipStream_t>(stream));
}

}  // namespace pti

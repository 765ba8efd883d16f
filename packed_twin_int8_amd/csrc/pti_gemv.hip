// Packed-weight decode GEMVs for gfx950: the SSQ twin GEMV and the Q8
// multi-stream GEMV, one kernel family.
//
// What is computed [README = "打包双子推理（PTI）", section "与 SSQ（Side-by-Side
// Quantization）的关系" (relation to SSQ); section "带宽分析：为什么会有开销"
// (bandwidth analysis)]: every weight is read from HBM once per call; one SSQ
// slot feeds twin A (high byte) and twin B (low byte); one Q8 block feeds up to
// four activation vectors.  Output y[s][r] = sum_c scale(r, c/32) * q[r][c] * x[s][c].
//
// Mapping onto CDNA4 (gfx950, wave64, 160 KB LDS per CU):
//   * Unit = 64 columns = two 32-column blocks: 68 bytes of Q8 (one dword-aligned
//     block pair) or 136 bytes of SSQ.  A lane loads whole units with dwordx4 loads.
//   * 16 lanes (one DPP row) own a band of R rows.  Lane j handles units
//     j, j+16, j+32, ... of every row of the band, so the activations it needs
//     are the same for all R rows: each LDS read of x serves R rows.
//   * x is staged into LDS once per workgroup (per K-chunk when it does not
//     fit), not re-read from L2 per row block: the README's bandwidth analysis
//     traces the L2 thrash of its multi-stream kernel to that re-reading.  The
//     LDS layout puts lane j's 16 bytes next to lane j+1's, so every
//     ds_read_b128 of a 16-lane group is a contiguous 256-byte span.
//   * Signed bytes convert to fp32 with one SDWA v_cvt_f32_i32 each; each
//     32-column block is summed in fp32 (column order), scaled by its f16 scale
//     with one FMA into the lane's accumulator; the 16 lanes of a band reduce
//     with a fixed DPP tree (row_shr 1, 2, 4, 8).  No MFMA: this is a
//     matrix-vector product, one FMA per weight and stream.
//   * The per-row operation order depends only on (rows, cols): not on the
//     stream count, the stream's slot, R, or the format, so a stream's output is
//     bitwise independent of those, and an SSQ twin equals a Q8 GEMV of the same
//     model bit for bit.
//   * Two unit buffers per lane: the next round's loads are in flight while the
//     current round is computed.
#include <hip/hip_runtime.h>

#include "pti_internal.h"

#ifndef PTI_R_Q8_N1
#define PTI_R_Q8_N1 4
#endif
#ifndef PTI_R_Q8_N2
#define PTI_R_Q8_N2 4
#endif
#ifndef PTI_R_Q8_N4
#define PTI_R_Q8_N4 4
#endif
#ifndef PTI_R_SSQ
#define PTI_R_SSQ 2
#endif
#ifndef PTI_LDS_BUDGET
#define PTI_LDS_BUDGET (80 * 1024)
#endif

namespace {

constexpr int kLanes = 16;                    // lanes per row band (one DPP row)
constexpr int kGroups = 16;                   // bands per workgroup
constexpr int kThreads = kLanes * kGroups;    // 256
constexpr int kUnitCols = 64;                 // columns per unit
constexpr int kRoundCols = kLanes * kUnitCols;  // columns covered by one round of a band

enum Fmt { kQ8 = 0, kSSQ = 1 };

struct GemvArgs {
    const uint8_t *w;
    const float *x[4];
    float *y[4];
    int64_t rows;
    int64_t row_bytes;
    int32_t cols;
    int32_t nb;            // blocks per row
    int32_t nu;            // units per row (the last one is half a unit when nb is odd)
    int32_t rounds;        // ceil(nu / kLanes)
    int32_t chunk_rounds;  // rounds of x held in LDS at once
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

// dwords per unit
template <int FMT>
constexpr int unit_dwords() { return FMT == kQ8 ? 17 : 34; }

template <int FMT>
struct Unit {
    uint32_t d[unit_dwords<FMT>()];
};

template <int N>
__device__ __forceinline__ void load_dwords(uint32_t *dst, const uint32_t *src)
{
#pragma unroll
    for (int i = 0; i + 4 <= N; i += 4) {
        u32x4 v = *reinterpret_cast<const u32x4_a4 *>(src + i);
        dst[i] = v.x, dst[i + 1] = v.y, dst[i + 2] = v.z, dst[i + 3] = v.w;
    }
#pragma unroll
    for (int i = N & ~3; i < N; i++)
        dst[i] = src[i];
}

// Loads unit u of a row into canonical dword form (the unit's bytes starting at
// a dword boundary).  ALIGNED: the unit starts on a dword boundary (always true
// for SSQ, and for Q8 when the row's block count is even, which also means Q8
// has no half units).  Otherwise (Q8 with an odd block count: rows alternate
// 2-byte offsets) it is read as 16-bit words.  A half unit (only its first
// block exists) reads only that block; the dwords of the missing block are
// left unset and never used.
template <int FMT, bool ALIGNED>
__device__ __forceinline__ void load_unit(Unit<FMT> &w, const uint8_t *row, int u, bool half)
{
    constexpr int DW = unit_dwords<FMT>();
    if constexpr (ALIGNED) {
        const uint32_t *p = reinterpret_cast<const uint32_t *>(row + (size_t)u * (DW * 4));
        if constexpr (FMT == kQ8) {
            load_dwords<DW>(w.d, p);
        } else {
            load_dwords<DW / 2>(w.d, p);
            if (!half)
                load_dwords<DW / 2>(w.d + DW / 2, p + DW / 2);
        }
    } else {
        const uint16_t *p = reinterpret_cast<const uint16_t *>(row + (size_t)u * (DW * 4));
        const int nh = half ? 17 : 2 * DW;  // halfwords present
#pragma unroll
        for (int i = 0; i < DW; i++) {
            uint32_t lo = (2 * i < nh) ? p[2 * i] : 0u;
            uint32_t hi = (2 * i + 1 < nh) ? p[2 * i + 1] : 0u;
            w.d[i] = lo | (hi << 16);
        }
    }
}

__device__ __forceinline__ float f16_to_f32(uint32_t bits16)
{
    return (float)__builtin_bit_cast(_Float16, (unsigned short)bits16);
}

__device__ __forceinline__ float sbyte(uint32_t d, int k)
{
    return (float)(int8_t)(d >> (8 * k));
}

// Signed int8 weight of column (4c + m) of block bb of a unit; for SSQ, twin
// t (0 = A, high byte of the slot; 1 = B, low byte).
template <int FMT>
__device__ __forceinline__ float weight(const Unit<FMT> &w, int bb, int c, int m, int t)
{
    if constexpr (FMT == kQ8) {
        if (bb == 0)  // bytes 2 + 4c + m of the unit
            return m < 2 ? sbyte(w.d[c], 2 + m) : sbyte(w.d[c + 1], m - 2);
        return sbyte(w.d[9 + c], m);  // bytes 36 + 4c + m
    } else {
        // slot (4c + m) of block bb: dword 17 bb + 1 + 2c + m/2, halfword m % 2
        const uint32_t d = w.d[17 * bb + 1 + 2 * c + (m >> 1)];
        return sbyte(d, 2 * (m & 1) + (t == 0 ? 1 : 0));
    }
}

template <int FMT>
__device__ __forceinline__ uint32_t scale_bits(const Unit<FMT> &w, int bb, int t)
{
    if constexpr (FMT == kQ8)
        return bb == 0 ? (w.d[0] & 0xffffu) : (w.d[8] >> 16);
    else
        return t == 0 ? (w.d[17 * bb] & 0xffffu) : (w.d[17 * bb] >> 16);
}

// LDS layout of one chunk of x (float4 elements):
//   xs[((round * 16 + cg) * NSP + p) * 16 + lane]
// cg = column group (4 columns) within the lane's unit (0..15), p = piece.
// Piece p of (lane, cg) holds elements 4p..4p+3 of the column-major flattening
// e = m * NSP + s (m = column within the group, s = stream); NSP = streams
// rounded up to 1, 2 or 4 (a fourth stream of zeros pads three streams).
template <int NSP, int NS>
__device__ __forceinline__ void stage_x(const GemvArgs &a, float4 *xs, int round0, int nr, int tid)
{
    const int jj = tid & (kLanes - 1), cg = tid / kLanes;  // 16 x 16 = 256 items per round
    for (int il = 0; il < nr; il++) {
        const int col = ((round0 + il) * kLanes + jj) * kUnitCols + cg * 4;
        float v[4][4];
#pragma unroll
        for (int s = 0; s < NSP; s++) {
            float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
            if (s < NS && col < a.cols)
                t = *reinterpret_cast<const float4 *>(a.x[s] + col);
            v[s][0] = t.x, v[s][1] = t.y, v[s][2] = t.z, v[s][3] = t.w;
        }
        float4 *base = xs + ((il * 16 + cg) * NSP) * kLanes + jj;
#pragma unroll
        for (int p = 0; p < NSP; p++) {
            float e[4];
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int flat = 4 * p + q;
                e[q] = v[flat % NSP][flat / NSP];
            }
            base[p * kLanes] = make_float4(e[0], e[1], e[2], e[3]);
        }
    }
}

// Accumulates one unit of R rows into acc.  xr points at the lane's x for this
// round: xr[(cg * NSP + p) * 16].
template <int FMT, int NSP, int NS, int R>
__device__ __forceinline__ void compute_unit(const Unit<FMT> (&w)[R], const float4 *xr, bool half,
                                             float (&acc)[R][NS])
{
#pragma unroll
    for (int bb = 0; bb < 2; bb++) {
        if (bb == 1 && half)
            break;
        float bs[R][NS];
#pragma unroll
        for (int c = 0; c < 8; c++) {
            float xv[4][NSP];
#pragma unroll
            for (int p = 0; p < NSP; p++) {
                const float4 t = xr[((bb * 8 + c) * NSP + p) * kLanes];
                const float e[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const int flat = 4 * p + q;
                    xv[flat / NSP][flat % NSP] = e[q];
                }
            }
#pragma unroll
            for (int r = 0; r < R; r++) {
#pragma unroll
                for (int m = 0; m < 4; m++) {
                    if constexpr (FMT == kQ8) {
                        const float q = weight<FMT>(w[r], bb, c, m, 0);
#pragma unroll
                        for (int s = 0; s < NS; s++)
                            bs[r][s] = (c == 0 && m == 0) ? q * xv[m][s] : __builtin_fmaf(q, xv[m][s], bs[r][s]);
                    } else {
#pragma unroll
                        for (int s = 0; s < NS; s++) {
                            const float q = weight<FMT>(w[r], bb, c, m, s);
                            bs[r][s] = (c == 0 && m == 0) ? q * xv[m][s] : __builtin_fmaf(q, xv[m][s], bs[r][s]);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int r = 0; r < R; r++)
#pragma unroll
            for (int s = 0; s < NS; s++)
                acc[r][s] = __builtin_fmaf(f16_to_f32(scale_bits<FMT>(w[r], bb, FMT == kQ8 ? 0 : s)), bs[r][s],
                                           acc[r][s]);
    }
}

__device__ __forceinline__ float dpp_shr(float v, int ctrl_shift)
{
    int iv = __builtin_bit_cast(int, v), r;
    switch (ctrl_shift) {
    case 1: r = __builtin_amdgcn_update_dpp(0, iv, 0x111, 0xf, 0xf, true); break;
    case 2: r = __builtin_amdgcn_update_dpp(0, iv, 0x112, 0xf, 0xf, true); break;
    case 4: r = __builtin_amdgcn_update_dpp(0, iv, 0x114, 0xf, 0xf, true); break;
    default: r = __builtin_amdgcn_update_dpp(0, iv, 0x118, 0xf, 0xf, true); break;
    }
    return __builtin_bit_cast(float, r);
}

// Sum over the 16 lanes of a DPP row; the total lands in the row's lane 15.
__device__ __forceinline__ float row_sum16(float v)
{
    v = v + dpp_shr(v, 1);
    v = v + dpp_shr(v, 2);
    v = v + dpp_shr(v, 4);
    v = v + dpp_shr(v, 8);
    return v;
}

template <int FMT, int NSP, int NS, int R, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvArgs a)
{
    extern __shared__ float4 xs[];
    const int tid = threadIdx.x, j = tid & (kLanes - 1), g = tid / kLanes;
    const int64_t row0 = ((int64_t)blockIdx.x * kGroups + g) * R;

    const uint8_t *rowp[R];
    bool rvalid[R];
#pragma unroll
    for (int r = 0; r < R; r++) {
        rvalid[r] = row0 + r < a.rows;
        rowp[r] = a.w + (rvalid[r] ? row0 + r : 0) * a.row_bytes;
    }

    float acc[R][NS];
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
        for (int s = 0; s < NS; s++)
            acc[r][s] = 0.f;

    Unit<FMT> wa[R], wb[R];
    // Lanes past the last unit and rows past the last row load a valid unit
    // (the row's last one, row 0) and skip its compute / store.
    auto load = [&](Unit<FMT>(&buf)[R], int round) {
        const int u = min(round * kLanes + j, a.nu - 1);
        const bool half = 2 * u + 1 >= a.nb;
#pragma unroll
        for (int r = 0; r < R; r++)
            load_unit<FMT, ALIGNED>(buf[r], rowp[r], u, half);
    };
    auto compute = [&](const Unit<FMT>(&buf)[R], int round, int il) {
        const int u = round * kLanes + j;
        if (u < a.nu)
            compute_unit<FMT, NSP, NS, R>(buf, xs + (il * 16 * NSP) * kLanes + j, 2 * u + 1 >= a.nb, acc);
    };

    for (int round0 = 0; round0 < a.rounds; round0 += a.chunk_rounds) {
        const int nr = min(a.chunk_rounds, a.rounds - round0);
        load(wa, round0);  // in flight while x is staged
        if (round0)
            __syncthreads();  // every lane is done with the previous chunk
        stage_x<NSP, NS>(a, xs, round0, nr, tid);
        __syncthreads();
        for (int il = 0; il < nr; il += 2) {
            if (il + 1 < nr)
                load(wb, round0 + il + 1);
            compute(wa, round0 + il, il);
            if (il + 1 >= nr)
                break;
            if (il + 2 < nr)
                load(wa, round0 + il + 2);
            compute(wb, round0 + il + 1, il + 1);
        }
    }

#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
        for (int s = 0; s < NS; s++) {
            const float v = row_sum16(acc[r][s]);
            if (j == kLanes - 1 && rvalid[r])
                a.y[s][row0 + r] = v;
        }
}

template <int FMT, int NSP, int NS, int R, bool ALIGNED>
int launch(const GemvArgs &a0, hipStream_t stream)
{
    GemvArgs a = a0;
    const int per_round = kRoundCols * NSP * 4;  // LDS bytes per round of x
    a.chunk_rounds = max(1, min(a.rounds, PTI_LDS_BUDGET / per_round));
    const size_t lds = (size_t)a.chunk_rounds * per_round;
    const int64_t bands = (a.rows + R - 1) / R;
    const dim3 grid((unsigned)((bands + kGroups - 1) / kGroups));
    auto kern = gemv_kernel<FMT, NSP, NS, R, ALIGNED>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, PTI_LDS_BUDGET);
        if (e != hipSuccess) {
            pti::set_hip_error(e);
            return PTI_ERR_HIP;
        }
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        pti::set_hip_error(e);
        return PTI_ERR_HIP;
    }
    return PTI_OK;
}

GemvArgs make_args(const void *w, int64_t rows, int64_t cols, int fmt_bytes)
{
    GemvArgs a{};
    a.w = static_cast<const uint8_t *>(w);
    a.rows = rows;
    a.cols = (int32_t)cols;
    a.nb = (int32_t)(cols / PTI_BLOCK);
    a.row_bytes = (int64_t)a.nb * fmt_bytes;
    a.nu = (a.nb + 1) / 2;
    a.rounds = (a.nu + kLanes - 1) / kLanes;
    return a;
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
    GemvArgs a = make_args(w_ssq, rows, cols, PTI_SSQ_BLOCK_BYTES);
    a.x[0] = x_a, a.x[1] = x_b;
    a.y[0] = y_a, a.y[1] = y_b;
    return launch<kSSQ, 2, 2, PTI_R_SSQ, true>(a, static_cast<hipStream_t>(stream));
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
    GemvArgs a = make_args(w_q8, rows, cols, PTI_Q8_BLOCK_BYTES);
    for (int s = 0; s < n_streams; s++) {
        a.x[s] = x + (size_t)s * cols;
        a.y[s] = y + (size_t)s * rows;
    }
    const bool aligned_rows = (a.nb % 2) == 0;
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (n_streams) {
    case 1:
        return aligned_rows ? launch<kQ8, 1, 1, PTI_R_Q8_N1, true>(a, st) : launch<kQ8, 1, 1, PTI_R_Q8_N1, false>(a, st);
    case 2:
        return aligned_rows ? launch<kQ8, 2, 2, PTI_R_Q8_N2, true>(a, st) : launch<kQ8, 2, 2, PTI_R_Q8_N2, false>(a, st);
    case 3:
        return aligned_rows ? launch<kQ8, 4, 3, PTI_R_Q8_N4, true>(a, st) : launch<kQ8, 4, 3, PTI_R_Q8_N4, false>(a, st);
    default:
        return aligned_rows ? launch<kQ8, 4, 4, PTI_R_Q8_N4, true>(a, st) : launch<kQ8, 4, 4, PTI_R_Q8_N4, false>(a, st);
    }
}

}  // extern "C"

"""Pure-Python scalar form of the SSQ twin GEMV (part of the oracle).

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's CPU
baseline may use it.  It reads the packed bytes with plain Python integer and
float operations (the f16 scales through the struct module's binary16 codec)
and shares nothing with the HIP library or with oracle.c.  It is the slow
reference the benchmark times on the tiny twin workload (256 x 512).

What it computes [README = "打包双子推理（PTI）", section "与 SSQ（Side-by-Side
Quantization）的关系" (relation to SSQ): each slot holds twin A's int8 in its
high byte and twin B's in its low byte, and each twin accumulates
scale * weight * x; Digest = "Packed Twin Inference：无需草稿模型的推测解码新方案，
实现2倍吞吐量提升", section "PTI的核心创新：SSQ打包技术" (SSQ packing): the
68-byte block [scale_A f16][scale_B f16][32 x uint16 slot], little-endian]:

    y_A[r] = sum_c scale_A(r, c/32) * A[r][c] * x_A[c]
    y_B[r] = sum_c scale_B(r, c/32) * B[r][c] * x_B[c]

summed in column order in double precision, with T = sum_c |scale * q * x|
beside each output (the magnitude the error bound is measured against).
"""

from __future__ import annotations

import struct

BLOCK = 32
SSQ_BLOCK_BYTES = 68


def _int8(byte: int) -> int:
    return byte - 256 if byte >= 128 else byte


def gemv_ssq(packed: bytes, rows: int, cols: int, x_a, x_b):
    """Both twins' outputs and |term| sums of a packed SSQ matrix:
    returns (y_a, y_b, t_a, t_b), lists of Python floats of length rows."""
    if cols % BLOCK:
        raise ValueError("cols must be a multiple of 32")
    nb = cols // BLOCK
    mv = bytes(packed)
    if len(mv) != rows * nb * SSQ_BLOCK_BYTES:
        raise ValueError("packed size does not match rows x cols")
    xa = [float(v) for v in x_a]
    xb = [float(v) for v in x_b]
    y_a, y_b, t_a, t_b = [], [], [], []
    for r in range(rows):
        acc_a = acc_b = mag_a = mag_b = 0.0
        for k in range(nb):
            off = (r * nb + k) * SSQ_BLOCK_BYTES
            s_a, s_b = struct.unpack_from("<ee", mv, off)
            for j in range(BLOCK):
                lo = mv[off + 4 + 2 * j]      # the slot's low byte: twin B
                hi = mv[off + 5 + 2 * j]      # the slot's high byte: twin A
                wa = s_a * _int8(hi)
                wb = s_b * _int8(lo)
                c = k * BLOCK + j
                acc_a += wa * xa[c]
                acc_b += wb * xb[c]
                mag_a += abs(wa) * abs(xa[c])
                mag_b += abs(wb) * abs(xb[c])
        y_a.append(acc_a)
        y_b.append(acc_b)
        t_a.append(mag_a)
        t_b.append(mag_b)
    return y_a, y_b, t_a, t_b

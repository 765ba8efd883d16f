"""Python binding of libpti.so, the packed-twin (PTI) decode path for MI355X.

Argument marshalling only: every step of the path runs in the library's HIP
kernels (device calls) or its C++ packer (host calls).  Device tensors come
from PyTorch, which supplies device memory and the current HIP stream; there
is no fallback of any kind -- if libpti.so is missing, importing the binding's
functions raises.

Shapes as this binding sees them:
  SSQ weights   uint8 [rows, cols/32*68]      (pack_ssq)
  Q8 weights    uint8 [rows, cols/32*34]      (pack_q8)
  activations   float32 [cols] / [n, cols]    (contiguous, 16-byte aligned)
  outputs       float32 [rows] / [n, rows]
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import LIB as LIB_PATH

__all__ = [
    "PtiError", "lib", "ssq_bytes", "q8_bytes", "pack_ssq", "unpack_ssq", "pack_q8", "unpack_q8",
    "ssq_split", "ssq_join", "gemv_ssq", "gemv_q8_multi", "verify_argmax", "status_str",
]

PTI_OK = 0
STATUS = {0: "PTI_OK", -1: "PTI_ERR_NULL", -2: "PTI_ERR_SHAPE", -3: "PTI_ERR_NSTREAMS", -4: "PTI_ERR_ALIGN",
          -5: "PTI_ERR_HIP", -6: "PTI_ERR_OVERLAP"}

# every symbol include/pti.h declares
EXPORTS = (
    "pti_status_str", "pti_last_hip_error", "pti_abi_version", "pti_ssq_bytes", "pti_q8_bytes", "pti_pack_ssq",
    "pti_unpack_ssq", "pti_pack_q8", "pti_unpack_q8", "pti_ssq_split", "pti_ssq_join", "pti_gemv_ssq",
    "pti_gemv_q8_multi", "pti_verify_argmax",
)


class PtiError(RuntimeError):
    def __init__(self, fn: str, status: int, hip_error: int = 0):
        self.status = status
        self.hip_error = hip_error
        msg = f"{fn}: {STATUS.get(status, status)} ({status_str(status)})"
        if status == -5:
            msg += f", hipError {hip_error}"
        super().__init__(msg)


_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int


def lib() -> ctypes.CDLL:
    """Load libpti.so (built in-tree by __graft_entry__.build() or
    ``python packed_twin_int8_amd/build.py``); raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        L.pti_status_str.argtypes = [_INT]
        L.pti_status_str.restype = ctypes.c_char_p
        L.pti_last_hip_error.restype = _INT
        L.pti_abi_version.restype = _INT
        L.pti_ssq_bytes.argtypes = [_I64, _I64]
        L.pti_ssq_bytes.restype = ctypes.c_size_t
        L.pti_q8_bytes.argtypes = [_I64, _I64]
        L.pti_q8_bytes.restype = ctypes.c_size_t
        L.pti_pack_ssq.argtypes = [_P, _P, _P, _P, _I64, _I64, _P]
        L.pti_unpack_ssq.argtypes = [_P, _I64, _I64, _P, _P, _P, _P]
        L.pti_pack_q8.argtypes = [_P, _P, _I64, _I64, _P]
        L.pti_unpack_q8.argtypes = [_P, _I64, _I64, _P, _P]
        L.pti_ssq_split.argtypes = [_P, _I64, _I64, _P, _P]
        L.pti_ssq_join.argtypes = [_P, _P, _I64, _I64, _P]
        L.pti_gemv_ssq.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _P]
        L.pti_gemv_q8_multi.argtypes = [_P, _P, _P, _I64, _I64, _INT, _P]
        L.pti_verify_argmax.argtypes = [_P, _P, _P, _P, _I64, _INT, _P]
        for name in EXPORTS:  # every declared symbol must resolve
            getattr(L, name)
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().pti_status_str(int(status)).decode()


def _check(fn: str, st: int):
    if st != PTI_OK:
        raise PtiError(fn, st, lib().pti_last_hip_error() if st == -5 else 0)


# ---------------------------------------------------------------- host packer

def _np(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _hp(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def ssq_bytes(rows: int, cols: int) -> int:
    return lib().pti_ssq_bytes(rows, cols)


def q8_bytes(rows: int, cols: int) -> int:
    return lib().pti_q8_bytes(rows, cols)


def pack_ssq(a, b, scale_a, scale_b) -> np.ndarray:
    """int8 [rows, cols] x2 + f16-bit scales [rows, cols/32] x2 -> uint8 [rows, cols/32*68]."""
    a, b = _np(a, np.int8), _np(b, np.int8)
    scale_a, scale_b = _np(scale_a, np.uint16), _np(scale_b, np.uint16)
    rows, cols = a.shape
    if b.shape != a.shape or scale_a.shape != (rows, cols // 32) or scale_b.shape != scale_a.shape:
        raise ValueError("pack_ssq: shape mismatch")
    out = np.empty((rows, cols // 32 * 68), np.uint8)
    _check("pti_pack_ssq", lib().pti_pack_ssq(_hp(a), _hp(b), _hp(scale_a), _hp(scale_b), rows, cols, _hp(out)))
    return out


def unpack_ssq(packed, rows: int, cols: int):
    packed = _np(packed, np.uint8)
    if packed.size != ssq_bytes(rows, cols):
        raise ValueError("unpack_ssq: size mismatch")
    a = np.empty((rows, cols), np.int8)
    b = np.empty((rows, cols), np.int8)
    sa = np.empty((rows, cols // 32), np.uint16)
    sb = np.empty((rows, cols // 32), np.uint16)
    _check("pti_unpack_ssq", lib().pti_unpack_ssq(_hp(packed), rows, cols, _hp(a), _hp(b), _hp(sa), _hp(sb)))
    return a, b, sa, sb


def pack_q8(q, scale) -> np.ndarray:
    """int8 [rows, cols] + f16-bit scales [rows, cols/32] -> uint8 [rows, cols/32*34]."""
    q, scale = _np(q, np.int8), _np(scale, np.uint16)
    rows, cols = q.shape
    if scale.shape != (rows, cols // 32):
        raise ValueError("pack_q8: shape mismatch")
    out = np.empty((rows, cols // 32 * 34), np.uint8)
    _check("pti_pack_q8", lib().pti_pack_q8(_hp(q), _hp(scale), rows, cols, _hp(out)))
    return out


def unpack_q8(packed, rows: int, cols: int):
    packed = _np(packed, np.uint8)
    if packed.size != q8_bytes(rows, cols):
        raise ValueError("unpack_q8: size mismatch")
    q = np.empty((rows, cols), np.int8)
    s = np.empty((rows, cols // 32), np.uint16)
    _check("pti_unpack_q8", lib().pti_unpack_q8(_hp(packed), rows, cols, _hp(q), _hp(s)))
    return q, s


def ssq_split(packed, rows: int, cols: int):
    packed = _np(packed, np.uint8)
    if packed.size != ssq_bytes(rows, cols):
        raise ValueError("ssq_split: size mismatch")
    qa = np.empty((rows, cols // 32 * 34), np.uint8)
    qb = np.empty((rows, cols // 32 * 34), np.uint8)
    _check("pti_ssq_split", lib().pti_ssq_split(_hp(packed), rows, cols, _hp(qa), _hp(qb)))
    return qa, qb


def ssq_join(q8_a, q8_b, rows: int, cols: int):
    q8_a, q8_b = _np(q8_a, np.uint8), _np(q8_b, np.uint8)
    if q8_a.size != q8_bytes(rows, cols) or q8_b.size != q8_a.size:
        raise ValueError("ssq_join: size mismatch")
    out = np.empty((rows, cols // 32 * 68), np.uint8)
    _check("pti_ssq_join", lib().pti_ssq_join(_hp(q8_a), _hp(q8_b), rows, cols, _hp(out)))
    return out


# ---------------------------------------------------------------- device calls

def _torch():
    import torch
    return torch


def _dev(t, name, dtype):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def gemv_ssq(w, x_a, x_b, y_a=None, y_b=None, stream=None):
    """SSQ twin GEMV: y_a = W_A x_a, y_b = W_B x_b (one pass over w).
    w: uint8 [rows, cols/32*68]; x_a, x_b: float32 [cols]."""
    torch = _torch()
    _dev(w, "w", torch.uint8), _dev(x_a, "x_a", torch.float32), _dev(x_b, "x_b", torch.float32)
    rows, cols = w.shape[0], x_a.shape[-1]
    if w.dim() != 2 or w.shape[1] != cols // 32 * 68 or x_b.shape != x_a.shape or x_a.dim() != 1:
        raise ValueError("gemv_ssq: shape mismatch")
    y_a = torch.empty(rows, dtype=torch.float32, device=w.device) if y_a is None else _dev(y_a, "y_a", torch.float32)
    y_b = torch.empty(rows, dtype=torch.float32, device=w.device) if y_b is None else _dev(y_b, "y_b", torch.float32)
    if y_a.numel() != rows or y_b.numel() != rows:
        raise ValueError("gemv_ssq: output shape mismatch")
    _check("pti_gemv_ssq", lib().pti_gemv_ssq(w.data_ptr(), x_a.data_ptr(), x_b.data_ptr(), y_a.data_ptr(),
                                              y_b.data_ptr(), rows, cols, _stream(stream)))
    return y_a, y_b


def gemv_q8_multi(w, x, y=None, stream=None):
    """Q8 multi-stream GEMV: y[n] = W x[n] for n < N (one pass over w).
    w: uint8 [rows, cols/32*34]; x: float32 [N, cols] (N = 1..4)."""
    torch = _torch()
    _dev(w, "w", torch.uint8), _dev(x, "x", torch.float32)
    if x.dim() == 1:
        x = x.unsqueeze(0)
    n, cols = x.shape
    rows = w.shape[0]
    if w.dim() != 2 or w.shape[1] != cols // 32 * 34:
        raise ValueError("gemv_q8_multi: shape mismatch")
    y = torch.empty((n, rows), dtype=torch.float32, device=w.device) if y is None else _dev(y, "y", torch.float32)
    if y.numel() != n * rows:
        raise ValueError("gemv_q8_multi: output shape mismatch")
    _check("pti_gemv_q8_multi", lib().pti_gemv_q8_multi(w.data_ptr(), x.data_ptr(), y.data_ptr(), rows, cols, n,
                                                        _stream(stream)))
    return y


def verify_argmax(logits, tokens_in, argmax_out=None, accept_out=None, stream=None):
    """Greedy verify: argmax per stream and the accept count.
    logits: float32 [N, vocab]; tokens_in: int32 [N] (device)."""
    torch = _torch()
    _dev(logits, "logits", torch.float32), _dev(tokens_in, "tokens_in", torch.int32)
    if logits.dim() == 1:
        logits = logits.unsqueeze(0)
    n, vocab = logits.shape
    if tokens_in.numel() != n:
        raise ValueError("verify_argmax: tokens_in must have one entry per stream")
    dev = logits.device
    argmax_out = torch.empty(n, dtype=torch.int32, device=dev) if argmax_out is None else _dev(
        argmax_out, "argmax_out", torch.int32)
    accept_out = torch.empty(1, dtype=torch.int32, device=dev) if accept_out is None else _dev(
        accept_out, "accept_out", torch.int32)
    _check("pti_verify_argmax", lib().pti_verify_argmax(logits.data_ptr(), tokens_in.data_ptr(),
                                                        argmax_out.data_ptr(), accept_out.data_ptr(), vocab, n,
                                                        _stream(stream)))
    return argmax_out, accept_out

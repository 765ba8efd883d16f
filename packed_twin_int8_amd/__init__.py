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
    "ssq_split", "ssq_join", "gemv_ssq", "gemv_q8_multi", "verify_argmax", "status_str", "sample_verify", "sample_verify_workspace",
    "sample_verify_static",
    "embed_q8", "embed_ssq", "rmsnorm", "silu_mul", "add", "ToyStack", "FMT_Q8", "FMT_SSQ",
]

FMT_Q8, FMT_SSQ = 0, 1
TOY_MAX_LAYERS = 64

PTI_OK = 0
STATUS = {0: "PTI_OK", -1: "PTI_ERR_NULL", -2: "PTI_ERR_SHAPE", -3: "PTI_ERR_NSTREAMS", -4: "PTI_ERR_ALIGN",
          -5: "PTI_ERR_HIP", -6: "PTI_ERR_OVERLAP"}

# every symbol include/pti.h declares
EXPORTS = (
    "pti_status_str", "pti_last_hip_error", "pti_abi_version", "pti_ssq_bytes", "pti_q8_bytes", "pti_pack_ssq",
    "pti_unpack_ssq", "pti_pack_q8", "pti_unpack_q8", "pti_ssq_split", "pti_ssq_join", "pti_gemv_ssq",
    "pti_gemv_ssq_verify", "pti_gemv_q8_multi", "pti_gemv_ssq_grouped", "pti_gemv_q8_multi_grouped",
    "pti_gemv_ssq_multi", "pti_attn_workspace_bytes", "pti_attn_decode", "pti_verify_argmax", "pti_sample_verify", "pti_sample_verify_workspace_bytes",
    "pti_sample_verify_static", "pti_embed_q8", "pti_embed_ssq", "pti_rmsnorm",
    "pti_silu_mul", "pti_add", "pti_toy_workspace_bytes", "pti_toy_forward", "pti_toy_decode",
    "pti_toy_forward_graph", "pti_graph_launch", "pti_graph_destroy",
)


class ToyModelC(ctypes.Structure):
    """struct pti_toy_model."""
    _fields_ = [("format", ctypes.c_int32), ("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int64),
                ("ffn", ctypes.c_int64), ("vocab", ctypes.c_int64), ("eps", ctypes.c_float),
                ("embed", ctypes.c_void_p), ("head", ctypes.c_void_p), ("gate", ctypes.POINTER(ctypes.c_void_p)),
                ("up", ctypes.POINTER(ctypes.c_void_p)), ("down", ctypes.POINTER(ctypes.c_void_p))]


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
        L.pti_gemv_ssq_verify.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.pti_gemv_q8_multi.argtypes = [_P, _P, _P, _I64, _I64, _INT, _P]
        L.pti_gemv_ssq_multi.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _INT, _P]
        L.pti_attn_workspace_bytes.argtypes = [_INT, _INT, _INT, _INT, _I64]
        L.pti_attn_workspace_bytes.restype = ctypes.c_size_t
        L.pti_attn_decode.argtypes = [_P, _P, _P, _P, _P, _P, _P, _INT, _INT, _INT, _INT, _I64, _P, ctypes.c_size_t, _P]
        L.pti_gemv_ssq_grouped.argtypes = [_P, _P, _INT, _P, _P, _P, _P, _I64, _P]
        L.pti_gemv_q8_multi_grouped.argtypes = [_P, _P, _INT, _P, _P, _I64, _INT, _P]
        L.pti_verify_argmax.argtypes = [_P, _P, _P, _P, _I64, _INT, _P]
        L.pti_sample_verify.argtypes = [_P, _P, _P, ctypes.c_double, _P, _P, _I64, _INT, _P, ctypes.c_size_t, _P]
        L.pti_sample_verify_static.argtypes = [_P, _P, _P, ctypes.c_double, _P, _P, _I64, _INT, _P]
        L.pti_sample_verify_workspace_bytes.argtypes = [_I64, _INT]
        L.pti_sample_verify_workspace_bytes.restype = ctypes.c_size_t
        L.pti_embed_q8.argtypes = [_P, _P, _P, _I64, _I64, _INT, _P]
        L.pti_embed_ssq.argtypes = [_P, _P, _P, _I64, _I64, _P]
        L.pti_rmsnorm.argtypes = [_P, _P, _I64, _INT, ctypes.c_float, _P]
        L.pti_silu_mul.argtypes = [_P, _P, _P, _I64, _P]
        L.pti_add.argtypes = [_P, _P, _P, _I64, _P]
        L.pti_toy_workspace_bytes.argtypes = [ctypes.POINTER(ToyModelC), _INT]
        L.pti_toy_workspace_bytes.restype = ctypes.c_size_t
        L.pti_toy_forward.argtypes = [ctypes.POINTER(ToyModelC), _P, _P, _P, ctypes.c_size_t, _INT, _P]
        L.pti_toy_forward_graph.argtypes = [ctypes.POINTER(ToyModelC), _P, _P, _P, ctypes.c_size_t, _INT,
                                            ctypes.POINTER(ctypes.c_void_p)]
        L.pti_graph_launch.argtypes = [_P, _P]
        L.pti_graph_destroy.argtypes = [_P]
        L.pti_toy_decode.argtypes = [ctypes.POINTER(ToyModelC), ctypes.c_int32, _INT, _INT, ctypes.c_double, _P, _P,
                                     ctypes.c_size_t, _P, _P, _P, ctypes.POINTER(ctypes.c_int64), _P]
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


SSQ_VERIFY_WORK_BYTES = 16384  # PTI_SSQ_VERIFY_WORK_BYTES


def ssq_verify_workspace(device):
    """Scratch for gemv_ssq_verify (contents need no initialisation)."""
    return _torch().empty(SSQ_VERIFY_WORK_BYTES, dtype=_torch().uint8, device=device)


def gemv_ssq_multi(w, x_a, x_b, y_a=None, y_b=None, stream=None):
    """SSQ twin GEMV with n streams per twin (n = 1, 2): y_a[j] = W_A x_a[j],
    y_b[j] = W_B x_b[j], one pass over w.  x_a, x_b: float32 [n, cols]."""
    torch = _torch()
    _dev(w, "w", torch.uint8), _dev(x_a, "x_a", torch.float32), _dev(x_b, "x_b", torch.float32)
    if x_a.dim() == 1:
        x_a, x_b = x_a.unsqueeze(0), x_b.unsqueeze(0)
    n, cols = x_a.shape
    rows = w.shape[0]
    if w.dim() != 2 or w.shape[1] != cols // 32 * 68 or x_b.shape != x_a.shape:
        raise ValueError("gemv_ssq_multi: shape mismatch")
    dev = w.device
    y_a = torch.empty((n, rows), dtype=torch.float32, device=dev) if y_a is None else _dev(y_a, "y_a", torch.float32)
    y_b = torch.empty((n, rows), dtype=torch.float32, device=dev) if y_b is None else _dev(y_b, "y_b", torch.float32)
    if y_a.numel() != n * rows or y_b.numel() != n * rows:
        raise ValueError("gemv_ssq_multi: output shape mismatch")
    _check("pti_gemv_ssq_multi", lib().pti_gemv_ssq_multi(w.data_ptr(), x_a.data_ptr(), x_b.data_ptr(), y_a.data_ptr(),
                                                          y_b.data_ptr(), rows, cols, n, _stream(stream)))
    return y_a, y_b


def gemv_ssq_verify(w, x_a, x_b, tokens_in, work, y_a=None, y_b=None, argmax_out=None, accept_out=None,
                    stream=None):
    """SSQ twin GEMV fused with the greedy verify of (y_a, y_b): returns
    y_a, y_b, argmax_out [2] and accept_out [1].  tokens_in: int32 [2] (device;
    entry 1 is the guess twin B ran on); work: from ssq_verify_workspace."""
    torch = _torch()
    _dev(w, "w", torch.uint8), _dev(x_a, "x_a", torch.float32), _dev(x_b, "x_b", torch.float32)
    _dev(tokens_in, "tokens_in", torch.int32), _dev(work, "work", torch.uint8)
    rows, cols = w.shape[0], x_a.shape[-1]
    if w.dim() != 2 or w.shape[1] != cols // 32 * 68 or x_b.shape != x_a.shape or x_a.dim() != 1:
        raise ValueError("gemv_ssq_verify: shape mismatch")
    if tokens_in.numel() != 2:
        raise ValueError("gemv_ssq_verify: tokens_in must have two entries")
    dev = w.device
    y_a = torch.empty(rows, dtype=torch.float32, device=dev) if y_a is None else _dev(y_a, "y_a", torch.float32)
    y_b = torch.empty(rows, dtype=torch.float32, device=dev) if y_b is None else _dev(y_b, "y_b", torch.float32)
    argmax_out = torch.empty(2, dtype=torch.int32, device=dev) if argmax_out is None else _dev(
        argmax_out, "argmax_out", torch.int32)
    accept_out = torch.empty(1, dtype=torch.int32, device=dev) if accept_out is None else _dev(
        accept_out, "accept_out", torch.int32)
    if y_a.numel() != rows or y_b.numel() != rows or argmax_out.numel() != 2 or accept_out.numel() != 1:
        raise ValueError("gemv_ssq_verify: output shape mismatch")
    _check("pti_gemv_ssq_verify", lib().pti_gemv_ssq_verify(
        w.data_ptr(), x_a.data_ptr(), x_b.data_ptr(), y_a.data_ptr(), y_b.data_ptr(), rows, cols,
        tokens_in.data_ptr(), argmax_out.data_ptr(), accept_out.data_ptr(), work.data_ptr(), work.numel(),
        _stream(stream)))
    return y_a, y_b, argmax_out, accept_out


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


def _group(ws, block_bytes, name):
    """Host arrays of device pointers and row counts for a grouped launch."""
    torch = _torch()
    ws = list(ws)
    if not ws:
        raise ValueError(f"{name}: at least one matrix")
    cols = ws[0].shape[1] // block_bytes * 32
    for i, w in enumerate(ws):
        _dev(w, f"w[{i}]", torch.uint8)
        if w.dim() != 2 or w.shape[1] != cols // 32 * block_bytes:
            raise ValueError(f"{name}: matrix {i} does not have {cols} columns")
    ptrs = (ctypes.c_void_p * len(ws))(*[w.data_ptr() for w in ws])
    rows = (ctypes.c_int64 * len(ws))(*[w.shape[0] for w in ws])
    return ptrs, rows, sum(w.shape[0] for w in ws), cols


def gemv_ssq_grouped(ws, x_a, x_b, y_a=None, y_b=None, stream=None):
    """SSQ twin GEMV over several matrices with the same columns in one
    launch; outputs over the stacked rows (matrix m's rows follow matrix
    m-1's).  ws: list of uint8 [rows_m, cols/32*68]."""
    torch = _torch()
    _dev(x_a, "x_a", torch.float32), _dev(x_b, "x_b", torch.float32)
    ptrs, rows, total, cols = _group(ws, 68, "gemv_ssq_grouped")
    if x_a.dim() != 1 or x_a.shape[0] != cols or x_b.shape != x_a.shape:
        raise ValueError("gemv_ssq_grouped: x shape mismatch")
    dev = x_a.device
    y_a = torch.empty(total, dtype=torch.float32, device=dev) if y_a is None else _dev(y_a, "y_a", torch.float32)
    y_b = torch.empty(total, dtype=torch.float32, device=dev) if y_b is None else _dev(y_b, "y_b", torch.float32)
    if y_a.numel() != total or y_b.numel() != total:
        raise ValueError("gemv_ssq_grouped: output shape mismatch")
    _check("pti_gemv_ssq_grouped", lib().pti_gemv_ssq_grouped(ptrs, rows, len(rows), x_a.data_ptr(), x_b.data_ptr(),
                                                              y_a.data_ptr(), y_b.data_ptr(), cols, _stream(stream)))
    return y_a, y_b


def gemv_q8_multi_grouped(ws, x, y=None, stream=None):
    """Q8 multi-stream GEMV over several matrices with the same columns in
    one launch: y [N, sum(rows)], matrix m's rows following matrix m-1's.
    ws: list of uint8 [rows_m, cols/32*34]; x: float32 [N, cols]."""
    torch = _torch()
    _dev(x, "x", torch.float32)
    if x.dim() == 1:
        x = x.unsqueeze(0)
    ptrs, rows, total, cols = _group(ws, 34, "gemv_q8_multi_grouped")
    n = x.shape[0]
    if x.shape[1] != cols:
        raise ValueError("gemv_q8_multi_grouped: x shape mismatch")
    y = torch.empty((n, total), dtype=torch.float32, device=x.device) if y is None else _dev(y, "y", torch.float32)
    if y.numel() != n * total:
        raise ValueError("gemv_q8_multi_grouped: output shape mismatch")
    _check("pti_gemv_q8_multi_grouped", lib().pti_gemv_q8_multi_grouped(ptrs, rows, len(rows), x.data_ptr(),
                                                                        y.data_ptr(), cols, n, _stream(stream)))
    return y


def attn_workspace(n_streams: int, n_heads: int, n_kv_heads: int, head_dim: int, max_len: int, device):
    """Scratch for attn_decode (no initialisation needed)."""
    nb = lib().pti_attn_workspace_bytes(n_streams, n_heads, n_kv_heads, head_dim, max_len)
    if nb == 0:
        raise PtiError("pti_attn_workspace_bytes", -2)
    return _torch().empty(nb, dtype=_torch().uint8, device=device)


def attn_decode(q, k_new, v_new, k_caches, v_caches, pos, work, out=None, stream=None):
    """One decode-attention step per stream: store k_new/v_new (rounded to
    binary16) at pos[s] of stream s's caches, then attend over positions
    0..pos[s].  q: float32 [S, H, d]; k_new, v_new: float32 [S, Hkv, d];
    k_caches, v_caches: lists of S float16 tensors [Hkv, max_len, d];
    pos: int32 [S] (device)."""
    torch = _torch()
    _dev(q, "q", torch.float32), _dev(k_new, "k_new", torch.float32), _dev(v_new, "v_new", torch.float32)
    _dev(pos, "pos", torch.int32), _dev(work, "work", torch.uint8)
    S, H, d = q.shape
    Hkv = k_new.shape[1]
    if k_new.shape != (S, Hkv, d) or v_new.shape != k_new.shape or pos.numel() != S:
        raise ValueError("attn_decode: shape mismatch")
    if len(k_caches) != S or len(v_caches) != S:
        raise ValueError("attn_decode: one K and one V cache per stream")
    max_len = k_caches[0].shape[1]
    for i, c in enumerate(list(k_caches) + list(v_caches)):
        _dev(c, f"cache[{i}]", torch.float16)
        if c.shape != (Hkv, max_len, d):
            raise ValueError("attn_decode: caches must be [Hkv, max_len, d]")
    out = torch.empty_like(q) if out is None else _dev(out, "out", torch.float32)
    kp = (ctypes.c_void_p * S)(*[c.data_ptr() for c in k_caches])
    vp = (ctypes.c_void_p * S)(*[c.data_ptr() for c in v_caches])
    _check("pti_attn_decode", lib().pti_attn_decode(q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), kp, vp,
                                                    pos.data_ptr(), out.data_ptr(), S, H, Hkv, d, max_len,
                                                    work.data_ptr(), work.numel(), _stream(stream)))
    return out


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


def sample_verify_workspace(vocab: int, n_streams: int, device):
    """Scratch for sample_verify (no initialisation needed)."""
    nb = lib().pti_sample_verify_workspace_bytes(vocab, n_streams)
    if nb == 0:
        raise PtiError("pti_sample_verify_workspace_bytes", -2)
    return _torch().empty(nb, dtype=_torch().uint8, device=device)


def sample_verify(logits, tokens_in, uniforms, temperature: float, tokens_out=None, accept_out=None, work=None,
                  stream=None):
    """Sampled verify at temperature > 0: one inverse-CDF draw per stream with
    uniforms[n], then the accept count.  logits: float32 [N, vocab];
    tokens_in: int32 [N]; uniforms: float64 [N] (device); work: from
    sample_verify_workspace (allocated here when omitted)."""
    torch = _torch()
    _dev(logits, "logits", torch.float32), _dev(tokens_in, "tokens_in", torch.int32)
    _dev(uniforms, "uniforms", torch.float64)
    if logits.dim() == 1:
        logits = logits.unsqueeze(0)
    n, vocab = logits.shape
    if tokens_in.numel() != n or uniforms.numel() != n:
        raise ValueError("sample_verify: tokens_in and uniforms need one entry per stream")
    dev = logits.device
    tokens_out = torch.empty(n, dtype=torch.int32, device=dev) if tokens_out is None else _dev(
        tokens_out, "tokens_out", torch.int32)
    accept_out = torch.empty(1, dtype=torch.int32, device=dev) if accept_out is None else _dev(
        accept_out, "accept_out", torch.int32)
    work = sample_verify_workspace(vocab, n, dev) if work is None else work
    _check("pti_sample_verify", lib().pti_sample_verify(logits.data_ptr(), tokens_in.data_ptr(), uniforms.data_ptr(),
                                                        float(temperature), tokens_out.data_ptr(),
                                                        accept_out.data_ptr(), vocab, n, work.data_ptr(),
                                                        work.numel() * work.element_size(), _stream(stream)))
    return tokens_out, accept_out


STATIC_SCRATCH_BYTES = 65536  # PTI_STATIC_SCRATCH_BYTES


def sample_verify_static(logits, tokens_in, uniforms, temperature: float, tokens_out, accept_out, stream=None):
    """sample_verify with the part sums in the library's own scratch (the call
    allocates nothing; outputs must be given).  Calls overlapping in time on
    one GPU share that scratch and race."""
    torch = _torch()
    _dev(logits, "logits", torch.float32), _dev(tokens_in, "tokens_in", torch.int32)
    _dev(uniforms, "uniforms", torch.float64)
    _dev(tokens_out, "tokens_out", torch.int32), _dev(accept_out, "accept_out", torch.int32)
    if logits.dim() == 1:
        logits = logits.unsqueeze(0)
    n, vocab = logits.shape
    if tokens_in.numel() != n or uniforms.numel() != n or tokens_out.numel() != n or accept_out.numel() < 1:
        raise ValueError("sample_verify_static: one token, uniform and output per stream, one accept count")
    _check("pti_sample_verify_static", lib().pti_sample_verify_static(
        logits.data_ptr(), tokens_in.data_ptr(), uniforms.data_ptr(), float(temperature), tokens_out.data_ptr(),
        accept_out.data_ptr(), vocab, n, _stream(stream)))
    return tokens_out, accept_out


# ---------------------------------------------------------------- decoder-stack glue

def embed_q8(w, tokens, vocab: int, hidden: int, x=None, stream=None):
    """Rows tokens[n] of a Q8 matrix [vocab, hidden], dequantised -> float32 [N, hidden]."""
    torch = _torch()
    _dev(w, "w", torch.uint8), _dev(tokens, "tokens", torch.int32)
    n = tokens.numel()
    if w.numel() != q8_bytes(vocab, hidden):
        raise ValueError("embed_q8: weight size mismatch")
    x = torch.empty((n, hidden), dtype=torch.float32, device=w.device) if x is None else _dev(x, "x", torch.float32)
    _check("pti_embed_q8", lib().pti_embed_q8(w.data_ptr(), tokens.data_ptr(), x.data_ptr(), vocab, hidden, n,
                                              _stream(stream)))
    return x


def embed_ssq(w, tokens, vocab: int, hidden: int, x=None, stream=None):
    """Twin A's row tokens[0] and twin B's row tokens[1] of an SSQ matrix -> float32 [2, hidden]."""
    torch = _torch()
    _dev(w, "w", torch.uint8), _dev(tokens, "tokens", torch.int32)
    if tokens.numel() != 2 or w.numel() != ssq_bytes(vocab, hidden):
        raise ValueError("embed_ssq: shape mismatch")
    x = torch.empty((2, hidden), dtype=torch.float32, device=w.device) if x is None else _dev(x, "x", torch.float32)
    _check("pti_embed_ssq", lib().pti_embed_ssq(w.data_ptr(), tokens.data_ptr(), x.data_ptr(), vocab, hidden,
                                                _stream(stream)))
    return x


def rmsnorm(x, eps: float, y=None, stream=None):
    """y[n] = x[n] / sqrt(mean(x[n]^2) + eps) per row of x [N, dim]."""
    torch = _torch()
    _dev(x, "x", torch.float32)
    if x.dim() == 1:
        x = x.unsqueeze(0)
    n, dim = x.shape
    y = torch.empty_like(x) if y is None else _dev(y, "y", torch.float32)
    _check("pti_rmsnorm", lib().pti_rmsnorm(x.data_ptr(), y.data_ptr(), dim, n, float(eps), _stream(stream)))
    return y


def silu_mul(g, u, y=None, stream=None):
    """y = silu(g) * u elementwise."""
    torch = _torch()
    _dev(g, "g", torch.float32), _dev(u, "u", torch.float32)
    if g.shape != u.shape:
        raise ValueError("silu_mul: shape mismatch")
    y = torch.empty_like(g) if y is None else _dev(y, "y", torch.float32)
    _check("pti_silu_mul", lib().pti_silu_mul(g.data_ptr(), u.data_ptr(), y.data_ptr(), g.numel(), _stream(stream)))
    return y


def add(a, b, y=None, stream=None):
    """y = a + b elementwise (fp32)."""
    torch = _torch()
    _dev(a, "a", torch.float32), _dev(b, "b", torch.float32)
    if a.shape != b.shape:
        raise ValueError("add: shape mismatch")
    y = torch.empty_like(a) if y is None else _dev(y, "y", torch.float32)
    _check("pti_add", lib().pti_add(a.data_ptr(), b.data_ptr(), y.data_ptr(), a.numel(), _stream(stream)))
    return y


class ForwardGraph:
    """An instantiated HIP graph of one forward pass (pti_toy_forward_graph);
    keeps the model and buffers it was captured over alive."""

    def __init__(self, handle, keep):
        self._h, self._keep = handle, keep

    def launch(self, stream=None):
        if not self._h:
            raise RuntimeError("graph destroyed")
        _check("pti_graph_launch", lib().pti_graph_launch(self._h, _stream(stream)))

    def destroy(self):
        if self._h:
            _check("pti_graph_destroy", lib().pti_graph_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


class ToyStack:
    """Device weights of the decoder stack plus the struct that names them.

    ``mats``: dict with "emb", "head" (uint8 tensors [vocab, ...]) and
    "gate", "up", "down" (lists of uint8 tensors), all packed in ``fmt``
    (FMT_Q8 or FMT_SSQ) and resident on the GPU."""

    def __init__(self, mats: dict, hidden: int, ffn: int, vocab: int, fmt: int = FMT_Q8, eps: float = 1e-6):
        torch = _torch()
        self.mats = mats  # keeps the tensors alive
        L = len(mats["gate"])
        if not (1 <= L <= TOY_MAX_LAYERS) or len(mats["up"]) != L or len(mats["down"]) != L:
            raise ValueError("ToyStack: layer lists must have equal length in [1, 64]")
        nbytes = ssq_bytes if fmt == FMT_SSQ else q8_bytes
        want = {"emb": nbytes(vocab, hidden), "head": nbytes(vocab, hidden)}
        for k, v in want.items():
            _dev(mats[k], k, torch.uint8)
            if mats[k].numel() != v:
                raise ValueError(f"ToyStack: {k} size mismatch")
        for k, (r, c) in (("gate", (ffn, hidden)), ("up", (ffn, hidden)), ("down", (hidden, ffn))):
            for t in mats[k]:
                _dev(t, k, torch.uint8)
                if t.numel() != nbytes(r, c):
                    raise ValueError(f"ToyStack: {k} size mismatch")
        Arr = ctypes.c_void_p * L
        self._gate = Arr(*[t.data_ptr() for t in mats["gate"]])
        self._up = Arr(*[t.data_ptr() for t in mats["up"]])
        self._down = Arr(*[t.data_ptr() for t in mats["down"]])
        vp = ctypes.POINTER(ctypes.c_void_p)
        self.c = ToyModelC(fmt, L, hidden, ffn, vocab, eps, mats["emb"].data_ptr(), mats["head"].data_ptr(),
                           ctypes.cast(self._gate, vp), ctypes.cast(self._up, vp), ctypes.cast(self._down, vp))
        self.fmt, self.hidden, self.ffn, self.vocab, self.device = fmt, hidden, ffn, vocab, mats["emb"].device

    def workspace(self, n_streams: int):
        nb = lib().pti_toy_workspace_bytes(ctypes.byref(self.c), n_streams)
        if nb == 0:
            raise PtiError("pti_toy_workspace_bytes", -3 if self.fmt == FMT_SSQ else -2)
        torch = _torch()
        return torch.empty(nb, dtype=torch.uint8, device=self.device)  # torch allocations are 256-byte aligned

    def forward(self, tokens, logits=None, work=None, stream=None):
        """logits [N, vocab] for device int32 tokens [N]."""
        torch = _torch()
        _dev(tokens, "tokens", torch.int32)
        n = tokens.numel()
        work = self.workspace(n) if work is None else work
        logits = torch.empty((n, self.vocab), dtype=torch.float32, device=self.device) if logits is None else _dev(
            logits, "logits", torch.float32)
        _check("pti_toy_forward", lib().pti_toy_forward(ctypes.byref(self.c), tokens.data_ptr(), logits.data_ptr(),
                                                        work.data_ptr(), work.numel(), n, _stream(stream)))
        return logits

    def forward_graph(self, tokens, logits, work):
        """One forward pass captured as a HIP graph over these buffers (the
        tensors must stay alive while the graph is used); returns a
        ForwardGraph whose launch() replays the pass."""
        torch = _torch()
        _dev(tokens, "tokens", torch.int32), _dev(logits, "logits", torch.float32), _dev(work, "work", torch.uint8)
        n = tokens.numel()
        if logits.numel() != n * self.vocab:
            raise ValueError("forward_graph: logits must be [N, vocab]")
        h = ctypes.c_void_p()
        _check("pti_toy_forward_graph", lib().pti_toy_forward_graph(
            ctypes.byref(self.c), tokens.data_ptr(), logits.data_ptr(), work.data_ptr(), work.numel(), n,
            ctypes.byref(h)))
        return ForwardGraph(h, (self, tokens, logits, work))

    def decode(self, first_token: int, n_streams: int, n_steps: int, temperature: float = 0.0, uniforms=None,
               work=None, stream=None):
        """The staggered decode loop.  uniforms: float64 array [(n_steps+1) * 2N]
        (host) when temperature > 0.  Returns (committed, accepts, passes) as
        numpy arrays; passes rows are (step, slot, stream, input, output)."""
        work = self.workspace(n_streams) if work is None else work
        N = n_streams
        committed = np.zeros(max(n_steps, 1), np.int32)
        accepts = np.zeros(max(n_steps, 1), np.int32)
        passes = np.zeros(((N - 1) + n_steps * (2 * N - 1), 5), np.int32)
        npass = ctypes.c_int64(0)
        u = None
        if temperature > 0:
            u = _np(uniforms, np.float64)
            if u.size != (n_steps + 1) * 2 * N:
                raise ValueError("decode: uniforms must hold (n_steps + 1) * 2 * n_streams values")
        _check("pti_toy_decode", lib().pti_toy_decode(
            ctypes.byref(self.c), int(first_token), N, n_steps, float(temperature), None if u is None else _hp(u),
            work.data_ptr(), work.numel(), _hp(committed), _hp(accepts), _hp(passes) if passes.size else None,
            ctypes.byref(npass), _stream(stream)))
        return committed[:n_steps], accepts[:n_steps], passes[:npass.value]

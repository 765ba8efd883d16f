"""fp64 CPU oracle for the packed-twin decode path.

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  It shares no code
with the HIP library under ``packed_twin_int8_amd/`` and never imports it.

The scalar C part (``oracle.c``: f16 decode, pack/unpack, GEMV, argmax,
verify) is loaded through ctypes; ``accept.py`` holds the exact
acceptance-probability enumeration and ``toy.py`` the fp64 toy decode model.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def _bind(path: str) -> ctypes.CDLL:
    L = ctypes.CDLL(path)
    L.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
    L.orc_f16_to_f64.restype = ctypes.c_double
    L.orc_ssq_bytes.argtypes = [_I64, _I64]
    L.orc_ssq_bytes.restype = ctypes.c_size_t
    L.orc_q8_bytes.argtypes = [_I64, _I64]
    L.orc_q8_bytes.restype = ctypes.c_size_t
    L.orc_pack_ssq.argtypes = [_P, _P, _P, _P, _I64, _I64, _P]
    L.orc_unpack_ssq.argtypes = [_P, _I64, _I64, _P, _P, _P, _P]
    L.orc_pack_q8.argtypes = [_P, _P, _I64, _I64, _P]
    L.orc_unpack_q8.argtypes = [_P, _I64, _I64, _P, _P]
    L.orc_gemv_q8.argtypes = [_P, _I64, _I64, _P, ctypes.c_int, _P, _P]
    L.orc_gemv_q8_rows.argtypes = [_P, _I64, _I64, _P, ctypes.c_int, _P, _I64, _P, _P]
    L.orc_gemv_ssq.argtypes = [_P, _I64, _I64, _P, _P, _P, _P, _P, _P]
    L.orc_gemv_ssq_rows.argtypes = [_P, _I64, _I64, _P, _P, _P, _I64, _P, _P, _P, _P]
    L.orc_argmax.argtypes = [_P, _I64]
    L.orc_argmax.restype = _I64
    L.orc_accept_count.argtypes = [_P, _P, ctypes.c_int]
    L.orc_accept_count.restype = ctypes.c_int
    L.orc_verify_argmax.argtypes = [_P, _P, _P, _I64, ctypes.c_int]
    L.orc_verify_argmax.restype = ctypes.c_int
    return L


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """The C oracle bound from one shared library (the default one, or a
    test-built variant of the same source)."""

    def __init__(self, path: str):
        self.path = path
        self.L = _bind(path)

    def f16_to_f64(self, bits) -> float:
        return self.L.orc_f16_to_f64(int(bits) & 0xFFFF)

    def ssq_bytes(self, rows: int, cols: int) -> int:
        return self.L.orc_ssq_bytes(rows, cols)

    def q8_bytes(self, rows: int, cols: int) -> int:
        return self.L.orc_q8_bytes(rows, cols)

    def pack_ssq(self, A, B, sA, sB) -> np.ndarray:
        A, B = _c(A, np.int8), _c(B, np.int8)
        sA, sB = _c(sA, np.uint16), _c(sB, np.uint16)
        rows, cols = A.shape
        assert B.shape == A.shape and cols % 32 == 0 and sA.shape == sB.shape == (rows, cols // 32)
        out = np.empty((rows, cols // 32 * 68), dtype=np.uint8)
        self.L.orc_pack_ssq(_ptr(A), _ptr(B), _ptr(sA), _ptr(sB), rows, cols, _ptr(out))
        return out

    def unpack_ssq(self, P, rows: int, cols: int):
        P = _c(P, np.uint8)
        assert P.size == rows * (cols // 32) * 68
        A = np.empty((rows, cols), np.int8)
        B = np.empty((rows, cols), np.int8)
        sA = np.empty((rows, cols // 32), np.uint16)
        sB = np.empty((rows, cols // 32), np.uint16)
        self.L.orc_unpack_ssq(_ptr(P), rows, cols, _ptr(A), _ptr(B), _ptr(sA), _ptr(sB))
        return A, B, sA, sB

    def pack_q8(self, Q, S) -> np.ndarray:
        Q, S = _c(Q, np.int8), _c(S, np.uint16)
        rows, cols = Q.shape
        assert cols % 32 == 0 and S.shape == (rows, cols // 32)
        out = np.empty((rows, cols // 32 * 34), dtype=np.uint8)
        self.L.orc_pack_q8(_ptr(Q), _ptr(S), rows, cols, _ptr(out))
        return out

    def unpack_q8(self, P, rows: int, cols: int):
        P = _c(P, np.uint8)
        assert P.size == rows * (cols // 32) * 34
        Q = np.empty((rows, cols), np.int8)
        S = np.empty((rows, cols // 32), np.uint16)
        self.L.orc_unpack_q8(_ptr(P), rows, cols, _ptr(Q), _ptr(S))
        return Q, S

    def gemv_q8(self, P, rows: int, cols: int, X):
        """Q8 GEMV of oracle-packed bytes P with X [n, cols] -> (y, t) float64 [n, rows]."""
        P = _c(P, np.uint8)
        X = _c(np.atleast_2d(X), np.float32)
        n = X.shape[0]
        assert X.shape[1] == cols and P.size == rows * (cols // 32) * 34
        y = np.empty((n, rows), np.float64)
        t = np.empty((n, rows), np.float64)
        self.L.orc_gemv_q8(_ptr(P), rows, cols, _ptr(X), n, _ptr(y), _ptr(t))
        return y, t

    def gemv_q8_rows(self, P, rows: int, cols: int, X, row_idx):
        """Q8 GEMV for the listed rows only -> (y, t) float64 [n, len(row_idx)]."""
        P = _c(P, np.uint8)
        X = _c(np.atleast_2d(X), np.float32)
        idx = _c(row_idx, np.int64)
        assert idx.min() >= 0 and idx.max() < rows
        assert X.shape[1] == cols and P.size == rows * (cols // 32) * 34
        n = X.shape[0]
        y = np.empty((n, idx.size), np.float64)
        t = np.empty((n, idx.size), np.float64)
        self.L.orc_gemv_q8_rows(_ptr(P), rows, cols, _ptr(X), n, _ptr(idx), idx.size, _ptr(y), _ptr(t))
        return y, t

    def gemv_ssq(self, P, rows: int, cols: int, xA, xB):
        """SSQ twin GEMV of oracle-packed bytes -> (yA, yB, tA, tB) float64 [rows]."""
        P = _c(P, np.uint8)
        xA, xB = _c(xA, np.float32), _c(xB, np.float32)
        assert xA.shape == xB.shape == (cols,) and P.size == rows * (cols // 32) * 68
        out = [np.empty(rows, np.float64) for _ in range(4)]
        self.L.orc_gemv_ssq(_ptr(P), rows, cols, _ptr(xA), _ptr(xB), *[_ptr(o) for o in out])
        return tuple(out)

    def gemv_ssq_rows(self, P, rows: int, cols: int, xA, xB, row_idx):
        """SSQ twin GEMV for the listed rows only -> (yA, yB, tA, tB)."""
        P = _c(P, np.uint8)
        xA, xB = _c(xA, np.float32), _c(xB, np.float32)
        idx = _c(row_idx, np.int64)
        assert idx.min() >= 0 and idx.max() < rows
        assert xA.shape == xB.shape == (cols,) and P.size == rows * (cols // 32) * 68
        out = [np.empty(idx.size, np.float64) for _ in range(4)]
        self.L.orc_gemv_ssq_rows(_ptr(P), rows, cols, _ptr(xA), _ptr(xB), _ptr(idx), idx.size,
                                 *[_ptr(o) for o in out])
        return tuple(out)

    def argmax(self, v) -> int:
        v = _c(v, np.float32)
        return int(self.L.orc_argmax(_ptr(v), v.size))

    def accept_count(self, tokens_in, amax) -> int:
        t = _c(tokens_in, np.int32)
        a = _c(amax, np.int32)
        assert t.size == a.size
        return int(self.L.orc_accept_count(_ptr(t), _ptr(a), t.size))

    def verify_argmax(self, logits, tokens_in):
        """-> (argmax int32 [n], accept count)."""
        L = _c(np.atleast_2d(logits), np.float32)
        n, vocab = L.shape
        t = _c(tokens_in, np.int32)
        assert t.size == n
        out = np.empty(n, np.int32)
        a = self.L.orc_verify_argmax(_ptr(L), _ptr(t), _ptr(out), vocab, n)
        return out, int(a)


_default = None


def default() -> Oracle:
    """The oracle built from oracle.c (built on first use if missing)."""
    global _default
    if _default is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _default = Oracle(_build.LIB)
    return _default


def __getattr__(name):
    # module-level access (oracle.gemv_ssq(...)) goes to the default build
    if name.startswith("_"):
        raise AttributeError(name)
    return getattr(default(), name)

"""libpti.so on the CPU: exported symbols, the host packer against the oracle's
packer (bit-exact), and every argument error the C ABI reports before it
touches the GPU."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
import packed_twin_int8_amd as pti
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pti.h")

OK, NULL, SHAPE, NSTREAMS, ALIGN, HIP, OVERLAP = 0, -1, -2, -3, -4, -5, -6


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pti_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_are_exported():
    syms = declared_symbols()
    assert len(syms) >= 14
    assert set(syms) == set(pti.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", pti.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (pti_[a-z0-9_]+)", out))
    missing = [s for s in syms if s not in exported]
    assert not missing, missing
    L = pti.lib()
    for s in syms:
        getattr(L, s)
    assert L.pti_abi_version() == 1


def test_status_strings():
    for st in (OK, NULL, SHAPE, NSTREAMS, ALIGN, HIP, OVERLAP):
        assert pti.status_str(st) and pti.status_str(st) != "unknown status"
    assert pti.status_str(7) == "unknown status"


@pytest.mark.parametrize("rows,cols", [(1, 32), (3, 96), (5, 512), (16, 1024), (7, 5632)])
def test_pack_matches_oracle(rows, cols):
    d = synth.twin(rows, cols, seed=rows * 1000 + cols)
    d["A"][0, 0] = -128
    d["B"][-1, -1] = -128
    d["sA"][0, 0] = 0x0001   # subnormal
    d["sB"][0, 0] = 0x8000   # -0
    d["sA"][-1, -1] = 0x7C00  # +inf
    d["sB"][-1, -1] = 0x7E01  # NaN payload
    P = pti.pack_ssq(d["A"], d["B"], d["sA"], d["sB"])
    assert np.array_equal(P, oracle.pack_ssq(d["A"], d["B"], d["sA"], d["sB"]))
    assert P.nbytes == pti.ssq_bytes(rows, cols) == rows * cols // 32 * 68
    for got, want in zip(pti.unpack_ssq(P, rows, cols), (d["A"], d["B"], d["sA"], d["sB"])):
        assert np.array_equal(got, want)
    Q = pti.pack_q8(d["A"], d["sA"])
    assert np.array_equal(Q, oracle.pack_q8(d["A"], d["sA"]))
    assert Q.nbytes == pti.q8_bytes(rows, cols) == rows * cols // 32 * 34
    q, s = pti.unpack_q8(Q, rows, cols)
    assert np.array_equal(q, d["A"]) and np.array_equal(s, d["sA"])
    qa, qb = pti.ssq_split(P, rows, cols)
    assert np.array_equal(qa, oracle.pack_q8(d["A"], d["sA"]))
    assert np.array_equal(qb, oracle.pack_q8(d["B"], d["sB"]))
    assert np.array_equal(pti.ssq_join(qa, qb, rows, cols), P)


def test_pack_random_bytes_roundtrip():
    g = np.random.default_rng(5)
    rows, cols = 9, 320
    P = g.integers(0, 256, (rows, cols // 32 * 68), dtype=np.uint8)
    assert np.array_equal(pti.pack_ssq(*pti.unpack_ssq(P, rows, cols)), P)
    Q = g.integers(0, 256, (rows, cols // 32 * 34), dtype=np.uint8)
    assert np.array_equal(pti.pack_q8(*pti.unpack_q8(Q, rows, cols)), Q)


def test_pack_large_threaded():
    # big enough to take the multi-threaded path
    rows, cols = 1024, 5120
    d = synth.twin(rows, cols, seed=9)
    P = pti.pack_ssq(d["A"], d["B"], d["sA"], d["sB"])
    assert np.array_equal(P, oracle.pack_ssq(d["A"], d["B"], d["sA"], d["sB"]))


# ------------------------------------------------------------------ ABI errors

def _fake(addr):
    # never dereferenced: every call below fails validation first
    return ctypes.c_void_p(addr)


A0 = 0x10000000  # 256-byte aligned fake device addresses, far apart
A1 = 0x20000000
A2 = 0x30000000
A3 = 0x40000000
A4 = 0x50000000


def test_host_packer_errors():
    L = pti.lib()
    buf = np.zeros(4096, np.uint8)
    p = buf.ctypes.data_as(ctypes.c_void_p)
    assert L.pti_pack_ssq(None, p, p, p, 1, 32, p) == NULL
    assert L.pti_pack_ssq(p, p, p, p, 1, 33, p) == SHAPE
    assert L.pti_pack_ssq(p, p, p, p, 0, 32, p) == SHAPE
    assert L.pti_pack_q8(p, p, 1, 16, p) == SHAPE
    assert L.pti_unpack_q8(p, -1, 32, p, p) == SHAPE
    assert L.pti_ssq_bytes(1, 31) == 0 and L.pti_q8_bytes(0, 32) == 0
    assert L.pti_ssq_bytes(2, 64) == 272 and L.pti_q8_bytes(2, 64) == 136
    # split/join reject overlapping buffers
    assert L.pti_ssq_split(p, 1, 32, p, _fake(buf.ctypes.data + 2000)) == OVERLAP


def test_gemv_ssq_errors():
    L = pti.lib()
    f = L.pti_gemv_ssq
    assert f(None, _fake(A1), _fake(A1), _fake(A2), _fake(A3), 8, 64, None) == NULL
    assert f(_fake(A0), _fake(A1), _fake(A1), None, _fake(A3), 8, 64, None) == NULL
    assert f(_fake(A0), _fake(A1), _fake(A1), _fake(A2), _fake(A3), 0, 64, None) == SHAPE
    assert f(_fake(A0), _fake(A1), _fake(A1), _fake(A2), _fake(A3), 8, 48, None) == SHAPE
    assert f(_fake(A0), _fake(A1), _fake(A1), _fake(A2), _fake(A3), 8, (1 << 24) + 32, None) == SHAPE
    assert f(_fake(A0 + 2), _fake(A1), _fake(A1), _fake(A2), _fake(A3), 8, 64, None) == ALIGN
    assert f(_fake(A0), _fake(A1 + 4), _fake(A1), _fake(A2), _fake(A3), 8, 64, None) == ALIGN
    assert f(_fake(A0), _fake(A1), _fake(A1), _fake(A2 + 1), _fake(A3), 8, 64, None) == ALIGN
    # y_b overlaps y_a; y_a overlaps w; y_b overlaps x_b
    assert f(_fake(A0), _fake(A1), _fake(A1), _fake(A2), _fake(A2 + 16), 8, 64, None) == OVERLAP
    assert f(_fake(A0), _fake(A1), _fake(A1), _fake(A0 + 64), _fake(A3), 8, 64, None) == OVERLAP
    assert f(_fake(A0), _fake(A1), _fake(A4), _fake(A2), _fake(A4 + 8), 8, 64, None) == OVERLAP


def test_gemv_ssq_verify_errors():
    L = pti.lib()
    f = L.pti_gemv_ssq_verify
    T, AM, AC, WK = 0x60000000, 0x61000000, 0x62000000, 0x63000000
    W = pti.SSQ_VERIFY_WORK_BYTES

    def call(w=A0, xa=A1, xb=A1, ya=A2, yb=A3, rows=8, cols=64, t=T, am=AM, ac=AC, wk=WK, wb=W):
        return f(_fake(w) if w else None, _fake(xa) if xa else None, _fake(xb), _fake(ya), _fake(yb), rows, cols,
                 _fake(t) if t else None, _fake(am) if am else None, _fake(ac) if ac else None,
                 _fake(wk) if wk else None, wb, None)

    for k in ("w", "xa", "t", "am", "ac", "wk"):
        assert call(**{k: 0}) == NULL, k
    assert call(rows=0) == SHAPE
    assert call(cols=48) == SHAPE
    assert call(wb=W - 1) == SHAPE        # workspace too small
    assert call(wk=WK + 8) == ALIGN       # workspace needs 16-byte alignment
    assert call(am=AM + 2) == ALIGN
    assert call(xa=A1 + 4) == ALIGN
    # argmax_out overlaps accept_out; work overlaps y_a; accept_out overlaps
    # tokens_in; y_b overlaps w
    assert call(ac=AM + 4) == OVERLAP
    assert call(wk=A2 - 1024) == OVERLAP
    assert call(ac=T + 4) == OVERLAP
    assert call(yb=A0 + 128) == OVERLAP


def test_grouped_gemv_errors():
    L = pti.lib()

    def arr(ctype, vals):
        return (ctype * len(vals))(*vals)

    W = arr(ctypes.c_void_p, [A0, A0 + 0x100000, A0 + 0x200000])
    R = arr(ctypes.c_int64, [8, 4, 4])
    q8 = L.pti_gemv_q8_multi_grouped
    assert q8(None, R, 3, _fake(A1), _fake(A2), 64, 1, None) == NULL
    assert q8(W, None, 3, _fake(A1), _fake(A2), 64, 1, None) == NULL
    assert q8(W, R, 0, _fake(A1), _fake(A2), 64, 1, None) == SHAPE
    assert q8(W, R, 5, _fake(A1), _fake(A2), 64, 1, None) == SHAPE
    assert q8(W, R, 3, _fake(A1), _fake(A2), 64, 0, None) == NSTREAMS
    assert q8(arr(ctypes.c_void_p, [A0, 0, A0]), R, 3, _fake(A1), _fake(A2), 64, 1, None) == NULL
    assert q8(W, arr(ctypes.c_int64, [8, 0, 4]), 3, _fake(A1), _fake(A2), 64, 1, None) == SHAPE
    assert q8(W, R, 3, _fake(A1), _fake(A2), 48, 1, None) == SHAPE
    assert q8(arr(ctypes.c_void_p, [A0, A0 + 0x100002, A0]), R, 3, _fake(A1), _fake(A2), 64, 1, None) == ALIGN
    # y over the second matrix
    assert q8(W, R, 3, _fake(A1), _fake(A0 + 0x100000 + 64), 64, 1, None) == OVERLAP
    ssq = L.pti_gemv_ssq_grouped
    assert ssq(W, R, 3, _fake(A1), None, _fake(A2), _fake(A3), 64, None) == NULL
    assert ssq(W, R, 5, _fake(A1), _fake(A1), _fake(A2), _fake(A3), 64, None) == SHAPE
    assert ssq(W, arr(ctypes.c_int64, [8, -1, 4]), 3, _fake(A1), _fake(A1), _fake(A2), _fake(A3), 64, None) == SHAPE
    assert ssq(W, R, 3, _fake(A1), _fake(A1), _fake(A2), _fake(A2 + 16), 64, None) == OVERLAP
    assert ssq(W, R, 3, _fake(A1), _fake(A1), _fake(A0 + 0x200000), _fake(A3), 64, None) == OVERLAP


def test_graph_handles_errors():
    L = pti.lib()
    assert L.pti_graph_launch(None, None) == NULL
    assert L.pti_graph_destroy(None) == 0
    assert L.pti_toy_forward_graph(None, _fake(A1), _fake(A2), _fake(A3), 1 << 20, 1, None) == NULL


def test_gemv_ssq_multi_errors():
    L = pti.lib()
    f = L.pti_gemv_ssq_multi
    assert f(_fake(A0), None, _fake(A1), _fake(A2), _fake(A3), 8, 64, 1, None) == NULL
    assert f(_fake(A0), _fake(A1), _fake(A1), _fake(A2), _fake(A3), 8, 64, 0, None) == NSTREAMS
    assert f(_fake(A0), _fake(A1), _fake(A1), _fake(A2), _fake(A3), 8, 64, 3, None) == NSTREAMS
    assert f(_fake(A0), _fake(A1), _fake(A1), _fake(A2), _fake(A3), 8, 48, 2, None) == SHAPE
    assert f(_fake(A0), _fake(A1 + 4), _fake(A1), _fake(A2), _fake(A3), 8, 64, 2, None) == ALIGN
    # with two streams per twin, y_a spans 64 bytes: y_b at +32 overlaps it
    assert f(_fake(A0), _fake(A1), _fake(A1), _fake(A2), _fake(A2 + 32), 8, 64, 2, None) == OVERLAP
    # x_b spans two rows of 64 floats: y_a at x_b + 256 overlaps its second row
    assert f(_fake(A0), _fake(A1), _fake(A4), _fake(A4 + 256), _fake(A3), 8, 64, 2, None) == OVERLAP


def test_attn_errors():
    L = pti.lib()
    ws = L.pti_attn_workspace_bytes
    assert ws(2, 40, 8, 128, 4096) == 2 * 40 * 32 * 130 * 4  # 128-key chunks
    assert ws(0, 8, 2, 128, 16) == 0 and ws(5, 8, 2, 128, 16) == 0
    assert ws(1, 8, 3, 128, 16) == 0 and ws(1, 18, 2, 128, 16) == 0  # not a multiple; 9 heads per kv head
    assert ws(1, 8, 2, 96, 16) == 0 and ws(1, 8, 2, 128, 0) == 0 and ws(1, 8, 2, 128, (1 << 24) + 1) == 0
    f = L.pti_attn_decode
    C0, C1 = 0x70000000, 0x71000000
    KP = (ctypes.c_void_p * 1)(C0)
    VP = (ctypes.c_void_p * 1)(C1)
    W = 1 << 20

    def call(q=A0, kn=A1, vn=A2, kp=KP, vp=VP, pos=A3, out=A4, S=1, H=8, Hkv=2, d=64, L_=16, wk=0x72000000, wb=W):
        return f(_fake(q) if q else None, _fake(kn), _fake(vn), kp, vp, _fake(pos), _fake(out), S, H, Hkv, d, L_,
                 _fake(wk) if wk else None, wb, None)

    assert call(q=0) == NULL and call(wk=0) == NULL and call(kp=None) == NULL
    assert call(kp=(ctypes.c_void_p * 1)(0)) == NULL
    assert call(S=0) == NSTREAMS and call(S=5) == NSTREAMS
    assert call(d=96) == SHAPE and call(Hkv=3) == SHAPE and call(L_=0) == SHAPE
    assert call(wb=64) == SHAPE
    assert call(kp=(ctypes.c_void_p * 1)(C0 + 8)) == ALIGN
    assert call(out=A4 + 2) == ALIGN
    assert call(wk=0x72000000 + 4) == ALIGN
    # the V cache over the K cache; out over q; the workspace over a cache
    assert call(vp=(ctypes.c_void_p * 1)(C0 + 64)) == OVERLAP
    assert call(out=A0 + 64) == OVERLAP
    assert call(wk=C1 + 128) == OVERLAP


def test_gemv_q8_errors():
    L = pti.lib()
    f = L.pti_gemv_q8_multi
    assert f(_fake(A0), None, _fake(A2), 8, 64, 1, None) == NULL
    assert f(_fake(A0), _fake(A1), _fake(A2), 8, 64, 0, None) == NSTREAMS
    assert f(_fake(A0), _fake(A1), _fake(A2), 8, 64, 5, None) == NSTREAMS
    assert f(_fake(A0), _fake(A1), _fake(A2), 8, 0, 1, None) == SHAPE
    assert f(_fake(A0), _fake(A1 + 8), _fake(A2), 8, 64, 1, None) == ALIGN
    assert f(_fake(A0), _fake(A1), _fake(A2 + 2), 8, 64, 1, None) == ALIGN
    # y [4][8] floats = 128 B starting 64 B before x
    assert f(_fake(A0), _fake(A1), _fake(A1 - 64), 8, 64, 4, None) == OVERLAP


def test_verify_errors():
    L = pti.lib()
    f = L.pti_verify_argmax
    assert f(None, _fake(A1), _fake(A2), _fake(A3), 100, 2, None) == NULL
    assert f(_fake(A0), _fake(A1), _fake(A2), _fake(A3), 0, 2, None) == SHAPE
    assert f(_fake(A0), _fake(A1), _fake(A2), _fake(A3), 100, 0, None) == NSTREAMS
    assert f(_fake(A0), _fake(A1), _fake(A2), _fake(A3), 100, 5, None) == NSTREAMS
    assert f(_fake(A0), _fake(A1), _fake(A2 + 2), _fake(A3), 100, 2, None) == ALIGN
    assert f(_fake(A0), _fake(A1), _fake(A2), _fake(A2 + 4), 100, 2, None) == OVERLAP
    assert f(_fake(A0), _fake(A1), _fake(A0 + 396), _fake(A3), 100, 2, None) == OVERLAP


def test_no_device_reports_hip_error():
    """With valid arguments and no GPU on this host the launch itself fails:
    the call must return PTI_ERR_HIP, not crash.  (Skipped where a GPU exists:
    the fake pointers would then reach a kernel.)"""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    L = pti.lib()
    st = L.pti_gemv_q8_multi(_fake(A0), _fake(A1), _fake(A2), 8, 64, 1, None)
    assert st == HIP
    assert L.pti_last_hip_error() != 0
    with pytest.raises(pti.PtiError):
        pti._check("pti_gemv_q8_multi", st)


def test_sample_verify_errors():
    L = pti.lib()
    f = L.pti_sample_verify
    wb = L.pti_sample_verify_workspace_bytes
    assert wb(100, 2) == 2 * 16 and wb(2049, 4) == 4 * 2 * 16 and wb(32000, 4) == 4 * 16 * 16
    assert wb(0, 1) == 0 and wb(100, 0) == 0 and wb(100, 5) == 0
    ok = (_fake(A0), _fake(A1), _fake(A2), 0.7, _fake(A3), _fake(A4), 100, 2, _fake(A4 + 0x1000), 32, None)

    def call(**kw):
        a = list(ok)
        for k, v in kw.items():
            a[int(k[1:])] = v
        return f(*a)

    assert call(a2=None) == NULL
    assert call(a3=0.0) == SHAPE and call(a3=-1.0) == SHAPE and call(a3=float("inf")) == SHAPE
    assert call(a3=float("nan")) == SHAPE
    assert call(a6=0) == SHAPE
    assert call(a7=0) == NSTREAMS and call(a7=5) == NSTREAMS
    assert call(a2=_fake(A2 + 4)) == ALIGN
    assert call(a4=_fake(A2 + 8)) == OVERLAP  # tokens_out inside uniforms [A2, A2+16)
    assert call(a5=_fake(A3 + 4)) == OVERLAP  # accept_out inside tokens_out
    assert call(a8=None) == NULL
    assert call(a9=31) == SHAPE  # workspace too small
    assert call(a8=_fake(A4 + 0x1008)) == ALIGN
    assert call(a8=_fake(A2)) == OVERLAP  # workspace over the uniforms
    assert call(a8=_fake(A4 - 16)) == OVERLAP  # workspace over accept_out


def test_sample_verify_static_errors():
    """The allocation-free form: the workspace form's argument checks, and
    PTI_ERR_SHAPE (before any HIP call) when the part sums would not fit the
    library's scratch."""
    L = pti.lib()
    f = L.pti_sample_verify_static
    ok = (_fake(A0), _fake(A1), _fake(A2), 0.7, _fake(A3), _fake(A4), 100, 2, None)

    def call(**kw):
        a = list(ok)
        for k, v in kw.items():
            a[int(k[1:])] = v
        return f(*a)

    assert call(a0=None) == NULL and call(a2=None) == NULL
    assert call(a3=0.0) == SHAPE and call(a3=float("nan")) == SHAPE and call(a6=0) == SHAPE
    assert call(a7=0) == NSTREAMS and call(a7=5) == NSTREAMS
    assert call(a2=_fake(A2 + 4)) == ALIGN
    assert call(a4=_fake(A2 + 8)) == OVERLAP
    # the scratch holds 4096 part sums of 2048 logits: 4 streams x 2,097,152 fit, one more logit does not
    assert pti.STATIC_SCRATCH_BYTES == 65536
    assert L.pti_sample_verify_workspace_bytes(2048 * 1024, 4) == pti.STATIC_SCRATCH_BYTES
    assert call(a6=2048 * 1024 + 1, a7=4, a1=_fake(0x70000000), a2=_fake(0x71000000), a3=0.7,
                a4=_fake(0x72000000), a5=_fake(0x73000000)) == SHAPE
    assert call(a6=4 * 2048 * 1024 + 1, a7=1) == SHAPE


def test_glue_errors():
    L = pti.lib()
    assert L.pti_embed_q8(None, _fake(A1), _fake(A2), 100, 64, 1, None) == NULL
    assert L.pti_embed_q8(_fake(A0), _fake(A1), _fake(A2), 100, 48, 1, None) == SHAPE
    assert L.pti_embed_q8(_fake(A0), _fake(A1), _fake(A2), 0, 64, 1, None) == SHAPE
    assert L.pti_embed_q8(_fake(A0), _fake(A1), _fake(A2), 100, 64, 5, None) == NSTREAMS
    assert L.pti_embed_q8(_fake(A0), _fake(A1 + 1), _fake(A2), 100, 64, 1, None) == ALIGN
    assert L.pti_embed_q8(_fake(A0), _fake(A1), _fake(A0 + 68), 100, 64, 1, None) == OVERLAP
    assert L.pti_embed_ssq(_fake(A0), _fake(A1), _fake(A1 + 4), 100, 64, None) == OVERLAP
    assert L.pti_embed_ssq(_fake(A0), None, _fake(A2), 100, 64, None) == NULL
    assert L.pti_rmsnorm(_fake(A0), _fake(A1), 0, 1, 1e-6, None) == SHAPE
    assert L.pti_rmsnorm(_fake(A0), _fake(A1), 64, 1, -1.0, None) == SHAPE
    assert L.pti_rmsnorm(_fake(A0), _fake(A1), 64, 1, float("nan"), None) == SHAPE
    assert L.pti_rmsnorm(_fake(A0), _fake(A1), 64, 0, 1e-6, None) == NSTREAMS
    assert L.pti_rmsnorm(_fake(A0), _fake(A0 + 4), 64, 1, 1e-6, None) == OVERLAP  # shifted in-place
    assert L.pti_silu_mul(_fake(A0), _fake(A1), _fake(A0 + 4), 64, None) == OVERLAP
    assert L.pti_silu_mul(_fake(A0), _fake(A1), _fake(A2), 0, None) == SHAPE
    assert L.pti_silu_mul(_fake(A0), _fake(A1 + 2), _fake(A2), 64, None) == ALIGN
    assert L.pti_add(_fake(A0), _fake(A1), _fake(A1 + 8), 64, None) == OVERLAP
    assert L.pti_add(None, _fake(A1), _fake(A2), 64, None) == NULL


def _toy(fmt=pti.FMT_Q8, layers=2, hidden=64, ffn=96, vocab=100, eps=1e-6, ptr=A0):
    Arr = ctypes.c_void_p * max(layers, 1)
    g = Arr(*([ptr] * max(layers, 1)))
    vp = ctypes.POINTER(ctypes.c_void_p)
    m = pti.ToyModelC(fmt, layers, hidden, ffn, vocab, eps, ptr, ptr, ctypes.cast(g, vp), ctypes.cast(g, vp),
                      ctypes.cast(g, vp))
    m._keep = g
    return m


def test_toy_errors():
    L = pti.lib()
    ws = L.pti_toy_workspace_bytes
    m = _toy()
    n = ws(ctypes.byref(m), 4)
    # h, r: 4*64*4 = 1024 each; stacked gate|up 4*2*96*4 = 3072; silu*up 4*96*4 = 1536;
    # logits 1600 (-> 1792); two small regions (tokens, uniforms) and the sampled verify's part
    # sums (4 x 16 -> 256); the LM head's greedy-verify keys (1024 workgroups x 4 streams x 8)
    assert n == 2 * 1024 + 3072 + 1536 + 1792 + 3 * 256 + 1024 * 4 * 8
    assert ws(ctypes.byref(m), 0) == 0 and ws(ctypes.byref(m), 5) == 0
    assert ws(ctypes.byref(_toy(fmt=pti.FMT_SSQ)), 4) == 0 and ws(ctypes.byref(_toy(fmt=pti.FMT_SSQ)), 2) > 0
    for bad in (_toy(fmt=2), _toy(layers=0), _toy(layers=65), _toy(hidden=48), _toy(ffn=0), _toy(vocab=0),
                _toy(eps=-1.0), _toy(eps=float("inf"))):
        assert ws(ctypes.byref(bad), 1) == 0
    assert ws(ctypes.byref(_toy(ptr=A0 + 2)), 1) == 0  # misaligned weights
    fwd = L.pti_toy_forward
    assert fwd(None, _fake(A1), _fake(A2), _fake(A3), n, 4, None) == NULL
    assert fwd(ctypes.byref(_toy(ptr=A0 + 2)), _fake(A1), _fake(A2), _fake(A3), n, 4, None) == ALIGN
    assert fwd(ctypes.byref(m), _fake(A1), _fake(A2), _fake(A3), n - 1, 4, None) == SHAPE
    assert fwd(ctypes.byref(m), _fake(A1), _fake(A2), _fake(A3 + 16), n, 4, None) == ALIGN
    assert fwd(ctypes.byref(m), _fake(A1), _fake(A3 + 512), _fake(A3), n, 4, None) == OVERLAP
    assert fwd(ctypes.byref(m), _fake(A1), _fake(A2), _fake(A3), n, 5, None) == NSTREAMS
    dec = L.pti_toy_decode
    buf = np.zeros(64, np.int32)
    hp = buf.ctypes.data_as(ctypes.c_void_p)
    u = np.zeros(64, np.float64).ctypes.data_as(ctypes.c_void_p)
    npass = ctypes.c_int64(-1)
    args = [ctypes.byref(m), 3, 4, 5, 0.0, None, _fake(A3), n, hp, hp, None, ctypes.byref(npass), None]

    def d(**kw):
        a = list(args)
        for k, v in kw.items():
            a[int(k[1:])] = v
        return dec(*a)

    assert d(a1=-1) == SHAPE and d(a1=100) == SHAPE
    assert d(a3=-1) == SHAPE
    assert d(a4=-0.5) == SHAPE and d(a4=float("nan")) == SHAPE
    assert d(a4=0.7) == NULL  # sampling needs uniforms
    assert d(a8=None) == NULL
    assert d(a7=n - 1) == SHAPE
    assert d(a6=_fake(A3 + 8)) == ALIGN
    assert d(a2=3, a0=ctypes.byref(_toy(fmt=pti.FMT_SSQ))) == NSTREAMS
    assert npass.value == -1  # nothing ran

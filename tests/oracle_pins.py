"""Pins of the fp64 oracle to facts fixed by the pages and by mathematics.

Each check takes an ``oracle.Oracle`` and raises AssertionError on a
mismatch, so the same checks run against the real oracle and against
deliberately broken builds of its source (to show each check has teeth).

What each pin rests on (nothing here re-types the oracle's own formula):
  * f16 decode: numpy's binary16 -> float64 conversion, all 65536 patterns.
  * block bytes: the worked bytes in tests/golden/ssq_block_bytes.json, derived
    from the SSQ block layout (digest page, SSQ packing section) and the
    high/low byte unpack arithmetic (README page, relation-to-SSQ section).
  * one-hot activations: x = e_c makes y[r] equal to scale * q[r][c] exactly,
    which isolates every (row, column) position, the byte order and which
    scale belongs to which twin.
  * integer sums: unit scales and all-ones x make y an exact integer row sum,
    computed here with int64 numpy sums of the raw weights.
  * general case: numpy float64 matrix-vector product of the weights
    dequantised from the RAW arrays (not from the packed bytes).
  * argmax: numpy.argmax (first maximum wins) on random data and crafted ties.
  * verify: the accept count's defining properties (range, prefix rule, all
    checks passing gives N) and, statistically, the pages' tokens-per-step
    formula under independent draws.
"""

from __future__ import annotations

import json
import os

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _f16(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def pin_f16_decode(O):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([O.f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "NaN patterns"
    assert np.array_equal(got[~nan], ref[~nan]), "f16 values"
    # sign of zero
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def pin_block_bytes(O):
    with open(os.path.join(GOLDEN, "ssq_block_bytes.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        A = np.full((1, 32), case["A_rest"], np.int8)
        B = np.full((1, 32), case["B_rest"], np.int8)
        A[0, 0], B[0, 0] = case["A0"], case["B0"]
        sA = np.array([[int(case["scale_A_f16"], 16)]], np.uint16)
        sB = np.array([[int(case["scale_B_f16"], 16)]], np.uint16)
        P = O.pack_ssq(A, B, sA, sB)
        assert P.size == case["block_bytes"] == O.ssq_bytes(1, 32)
        want = bytes(int(h, 16) for h in case["first_8_bytes_hex"].split())
        assert bytes(P[0, :8]) == want, (bytes(P[0, :8]).hex(), want.hex())
    # Q8: [scale][q0 .. q31], 34 bytes; two Q8 blocks = one SSQ block in size
    Q = np.arange(-16, 16, dtype=np.int8).reshape(1, 32)
    S = np.array([[0x3C00]], np.uint16)
    P = O.pack_q8(Q, S)
    assert P.size == 34 == O.q8_bytes(1, 32) and 2 * O.q8_bytes(7, 96) == O.ssq_bytes(7, 96)
    assert bytes(P[0]) == bytes([0x00, 0x3C]) + Q.tobytes()


def pin_roundtrip(O, seed=11):
    g = np.random.default_rng(seed)
    rows, cols = 5, 96
    A = g.integers(-128, 128, (rows, cols), dtype=np.int8)
    B = g.integers(-128, 128, (rows, cols), dtype=np.int8)
    sA = g.integers(0, 65536, (rows, cols // 32), dtype=np.uint16)
    sB = g.integers(0, 65536, (rows, cols // 32), dtype=np.uint16)
    P = O.pack_ssq(A, B, sA, sB)
    for got, want in zip(O.unpack_ssq(P, rows, cols), (A, B, sA, sB)):
        assert np.array_equal(got, want)
    R = g.integers(0, 256, P.shape, dtype=np.uint8)
    assert np.array_equal(O.pack_ssq(*O.unpack_ssq(R, rows, cols)), R)
    Q8 = O.pack_q8(A, sA)
    q, s = O.unpack_q8(Q8, rows, cols)
    assert np.array_equal(q, A) and np.array_equal(s, sA)
    R8 = g.integers(0, 256, Q8.shape, dtype=np.uint8)
    assert np.array_equal(O.pack_q8(*O.unpack_q8(R8, rows, cols)), R8)


def pin_one_hot(O, seed=12):
    rows, cols = 3, 96
    d = synth.twin(rows, cols, seed)
    PS = O.pack_ssq(d["A"], d["B"], d["sA"], d["sB"])
    PQ = O.pack_q8(d["A"], d["sA"])
    for c in range(cols):
        e = np.zeros(cols, np.float32)
        e[c] = 1.0
        e2 = np.zeros(cols, np.float32)
        e2[c] = -2.0
        ya, yb, ta, tb = O.gemv_ssq(PS, rows, cols, e, e2)
        wa = _f16(d["sA"][:, c // 32]) * d["A"][:, c].astype(np.float64)
        wb = _f16(d["sB"][:, c // 32]) * d["B"][:, c].astype(np.float64)
        assert np.array_equal(ya, wa) and np.array_equal(yb, -2.0 * wb), c
        assert np.array_equal(ta, np.abs(wa)) and np.array_equal(tb, 2.0 * np.abs(wb)), c
        y, t = O.gemv_q8(PQ, rows, cols, np.stack([e, e2]))
        assert np.array_equal(y[0], wa) and np.array_equal(y[1], -2.0 * wa), c


def pin_integer_sums(O, seed=13):
    g = np.random.default_rng(seed)
    rows, cols = 4, 160
    A = g.integers(-128, 128, (rows, cols), dtype=np.int8)
    B = g.integers(-128, 128, (rows, cols), dtype=np.int8)
    one = np.full((rows, cols // 32), 0x3C00, np.uint16)  # f16 1.0
    ones = np.ones(cols, np.float32)
    ya, yb, _, _ = O.gemv_ssq(O.pack_ssq(A, B, one, one), rows, cols, ones, ones)
    assert np.array_equal(ya, A.astype(np.int64).sum(1).astype(np.float64))
    assert np.array_equal(yb, B.astype(np.int64).sum(1).astype(np.float64))
    y, _ = O.gemv_q8(O.pack_q8(B, one), rows, cols, ones)
    assert np.array_equal(y[0], B.astype(np.int64).sum(1).astype(np.float64))


def pin_vs_numpy(O, rows=37, cols=320, seed=14):
    d = synth.twin(rows, cols, seed)
    WA = d["A"].astype(np.float64) * np.repeat(_f16(d["sA"]), 32, axis=1)
    WB = d["B"].astype(np.float64) * np.repeat(_f16(d["sB"]), 32, axis=1)
    xa, xb = d["xA"].astype(np.float64), d["xB"].astype(np.float64)
    ya, yb, ta, tb = O.gemv_ssq(O.pack_ssq(d["A"], d["B"], d["sA"], d["sB"]), rows, cols, d["xA"], d["xB"])
    for y, t, W, x in ((ya, ta, WA, xa), (yb, tb, WB, xb)):
        tref = np.abs(W) @ np.abs(x)
        assert np.all(np.abs(y - W @ x) <= 1e-12 * tref)
        assert np.allclose(t, tref, rtol=1e-12, atol=0)
    X = np.stack([d["xA"], d["xB"], -d["xA"]])
    y, t = O.gemv_q8(O.pack_q8(d["A"], d["sA"]), rows, cols, X)
    ref = X.astype(np.float64) @ WA.T
    assert np.all(np.abs(y - ref) <= 1e-12 * (np.abs(X.astype(np.float64)) @ np.abs(WA).T))
    # sampled rows agree with the full product
    idx = np.array([rows - 1, 0, 5, 5])
    ys, ts = O.gemv_q8_rows(O.pack_q8(d["A"], d["sA"]), rows, cols, X, idx)
    assert np.array_equal(ys, y[:, idx]) and np.array_equal(ts, t[:, idx])
    r = O.gemv_ssq_rows(O.pack_ssq(d["A"], d["B"], d["sA"], d["sB"]), rows, cols, d["xA"], d["xB"], idx)
    assert np.array_equal(r[0], ya[idx]) and np.array_equal(r[1], yb[idx])


def pin_twin_equals_two_q8(O, seed=15):
    rows, cols = 9, 256
    d = synth.twin(rows, cols, seed)
    ya, yb, ta, tb = O.gemv_ssq(O.pack_ssq(d["A"], d["B"], d["sA"], d["sB"]), rows, cols, d["xA"], d["xB"])
    qa, tqa = O.gemv_q8(O.pack_q8(d["A"], d["sA"]), rows, cols, d["xA"])
    qb, tqb = O.gemv_q8(O.pack_q8(d["B"], d["sB"]), rows, cols, d["xB"])
    assert np.array_equal(ya, qa[0]) and np.array_equal(yb, qb[0])
    assert np.array_equal(ta, tqa[0]) and np.array_equal(tb, tqb[0])
    # A == B twins with x_A == x_B give identical streams
    s = synth.twin(rows, cols, seed, same=True, same_x=True)
    ya, yb, _, _ = O.gemv_ssq(O.pack_ssq(s["A"], s["B"], s["sA"], s["sB"]), rows, cols, s["xA"], s["xB"])
    assert np.array_equal(ya, yb)


def pin_argmax(O, seed=16):
    g = np.random.default_rng(seed)
    for n in (1, 2, 7, 1000, 32000):
        v = g.standard_normal(n).astype(np.float32)
        assert O.argmax(v) == int(np.argmax(v))
    v = np.zeros(50, np.float32)
    v[[7, 9, 40]] = 3.0
    assert O.argmax(v) == 7 == int(np.argmax(v))
    v = np.full(10, -1.0, np.float32)
    v[3] = -0.0
    v[6] = 0.0
    assert O.argmax(v) == 3  # -0 == +0: first wins
    v = np.array([-np.inf, -5.0, np.inf, np.inf], np.float32)
    assert O.argmax(v) == 2
    L = g.standard_normal((4, 300)).astype(np.float32)
    am, _ = O.verify_argmax(L, np.zeros(4, np.int32))
    assert np.array_equal(am, L.argmax(1))


def pin_accept_rule(O, seed=17):
    g = np.random.default_rng(seed)
    for n in (1, 2, 3, 4):
        for _ in range(200):
            tok = g.integers(0, 3, n).astype(np.int32)
            am = g.integers(0, 3, n).astype(np.int32)
            a = O.accept_count(tok, am)
            assert 1 <= a <= n
            if n == 1:
                assert a == 1
            ok = [tok[i] == am[i - 1] for i in range(1, n)]
            # all checks pass <=> a == n; a failed check at i caps a at i
            assert (a == n) == all(ok)
            if not all(ok):
                first = ok.index(False) + 1
                assert a == first
                # tokens after the first failure cannot change a
                tok2 = tok.copy()
                tok2[first:] = (tok2[first:] + 1) % 3
                tok2[first] = tok[first]
                assert O.accept_count(tok2, am) == a
    # greedy self-speculation: every guess equals the previous stream's output
    am = np.array([5, 9, 2, 7], np.int32)
    assert O.accept_count(np.array([0, 5, 9, 2], np.int32), am) == 4
    # statistical: iid draws from p give E[a] = sum_i P^i, P = sum p^2
    p = np.array([0.5, 0.3, 0.2])
    P = float((p ** 2).sum())
    n, trials = 4, 40000
    outs = g.choice(3, size=(trials, n), p=p).astype(np.int32)
    gs = g.choice(3, size=(trials, n), p=p).astype(np.int32)
    tot = sum(O.accept_count(gs[k], outs[k]) for k in range(trials))
    mean = tot / trials
    ev = sum(P ** i for i in range(n))
    # variance of a is below n^2/4; 6 sigma
    assert abs(mean - ev) < 6 * (n / 2) / np.sqrt(trials), (mean, ev)


ALL_PINS = (pin_f16_decode, pin_block_bytes, pin_roundtrip, pin_one_hot, pin_integer_sums,
            pin_vs_numpy, pin_twin_equals_two_q8, pin_argmax, pin_accept_rule)


def run_all(O):
    """Run every pin; return the names of those that failed."""
    failed = []
    for pin in ALL_PINS:
        try:
            pin(O)
        except AssertionError:
            failed.append(pin.__name__)
    return failed

"""Pins of the pure-Python scalar SSQ GEMV (oracle/scalar.py).

It is checked against facts other than itself: one-hot activations isolate
every (row, column) weight and which byte and scale belong to which twin
(closed form from numpy's binary16 conversion of the raw scales); numpy's
float64 product of the weights dequantised from the RAW arrays; and the C
oracle's result on the tiny twin workload (an independent implementation of
the same definition, summed in the same column order, so the results agree
bitwise).  Planted mistakes in a copy of its source must fail these pins.
"""

from __future__ import annotations

import inspect
import types

import numpy as np

import oracle
import synth
from oracle import scalar


def _f16(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def pin_one_hot(mod):
    rows, cols = 3, 96
    d = synth.twin(rows, cols, 31)
    d["A"][0, 5], d["B"][1, 70] = -128, -128
    P = oracle.pack_ssq(d["A"], d["B"], d["sA"], d["sB"])
    for c in range(cols):
        e = np.zeros(cols, np.float32)
        e[c] = 1.0
        ya, yb, ta, tb = mod.gemv_ssq(P.tobytes(), rows, cols, e, -2.0 * e)
        wa = _f16(d["sA"][:, c // 32]) * d["A"][:, c].astype(np.float64)
        wb = _f16(d["sB"][:, c // 32]) * d["B"][:, c].astype(np.float64)
        assert np.array_equal(ya, wa) and np.array_equal(yb, -2.0 * wb), c
        assert np.array_equal(ta, np.abs(wa)) and np.array_equal(tb, 2.0 * np.abs(wb)), c


def pin_dense(mod):
    rows, cols = 7, 160
    d = synth.twin(rows, cols, 32)
    P = oracle.pack_ssq(d["A"], d["B"], d["sA"], d["sB"])
    ya, yb, ta, tb = (np.array(v) for v in mod.gemv_ssq(P.tobytes(), rows, cols, d["xA"], d["xB"]))
    WA = d["A"].astype(np.float64) * np.repeat(_f16(d["sA"]), 32, axis=1)
    WB = d["B"].astype(np.float64) * np.repeat(_f16(d["sB"]), 32, axis=1)
    xa, xb = d["xA"].astype(np.float64), d["xB"].astype(np.float64)
    assert np.all(np.abs(ya - WA @ xa) <= 1e-14 * (np.abs(WA) @ np.abs(xa)))
    assert np.all(np.abs(yb - WB @ xb) <= 1e-14 * (np.abs(WB) @ np.abs(xb)))
    np.testing.assert_allclose(ta, np.abs(WA) @ np.abs(xa), rtol=1e-14)
    np.testing.assert_allclose(tb, np.abs(WB) @ np.abs(xb), rtol=1e-14)


def test_scalar_pins():
    pin_one_hot(scalar)
    pin_dense(scalar)


def test_scalar_equals_c_oracle_on_tiny_workload():
    rows, cols = 256, 512
    d = synth.twin(rows, cols, synth.SEED_TINY)
    P = oracle.pack_ssq(d["A"], d["B"], d["sA"], d["sB"])
    got = [np.array(v) for v in scalar.gemv_ssq(P.tobytes(), rows, cols, d["xA"], d["xB"])]
    want = oracle.gemv_ssq(P, rows, cols, d["xA"], d["xB"])
    for g, w in zip(got, want):
        assert np.array_equal(g, w)


def _mutant(old, new):
    src = inspect.getsource(scalar)
    assert old in src
    m = types.ModuleType("scalar_mutant")
    exec(compile(src.replace(old, new, 1), "scalar_mutant", "exec"), m.__dict__)
    return m


MUTANTS = [
    ("wa = s_a * _int8(hi)", "wa = s_a * _int8(lo)"),          # twin A from the low byte
    ("wb = s_b * _int8(lo)", "wb = s_b * lo"),                  # unsigned twin B byte
    ('s_a, s_b = struct.unpack_from("<ee", mv, off)', 's_b, s_a = struct.unpack_from("<ee", mv, off)'),  # scales swapped
    ("c = k * BLOCK + j", "c = k * BLOCK + (j + 1) % BLOCK"),   # off-by-one column
    ("acc_a += wa * xa[c]", "acc_a = wa * xa[c]"),              # dropped sum
    ("mag_b += abs(wb) * abs(xb[c])", "mag_b += abs(wb * xb[c] + mag_b) * 0"),  # wrong magnitude
]


def test_scalar_pins_catch_planted_mistakes():
    for old, new in MUTANTS:
        m = _mutant(old, new)
        caught = False
        for pin in (pin_one_hot, pin_dense):
            try:
                pin(m)
            except AssertionError:
                caught = True
        assert caught, (old, new)

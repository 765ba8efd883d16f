"""GPU parity of the grouped GEMVs (several matrices, one launch).

Bar: every output of a grouped launch is bitwise the output of the
single-matrix call on its matrix (a row's arithmetic depends only on the
column count and the format), and one grouped case is checked against the
oracle within 1e-5 * sum |terms| on every row.
"""

import sys

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

# (name, cols, row counts): layer groups at their real shapes, odd block
# counts (rows at 2-byte offsets), single rows, and the most matrices a
# launch takes
GROUPS = [
    ("qkv", 5120, [5120, 1024, 1024]),
    ("gate_up", 5120, [17408, 17408]),
    ("odd_blocks", 1056, [7, 130, 1, 64]),
    ("one", 2048, [300]),
    ("tiny", 32, [1, 2, 3, 4]),
    ("ragged", 3104, [257, 33]),
    ("long_rows", 20992, [100, 60]),
]


@pytest.fixture(scope="module")
def env():
    import torch

    import packed_twin_int8_amd as pti
    assert torch.cuda.is_available()
    pti.lib()
    return torch, pti, torch.device("cuda:0")


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bits(t):
    return t.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("name,cols,rows", GROUPS, ids=[g[0] for g in GROUPS])
def test_ssq_grouped_equals_single(env, name, cols, rows):
    torch, pti, dev = env
    _note(f"ssq grouped {name}: cols {cols}, rows {rows}")
    ds = [synth.twin(r, cols, seed=100 * k + r) for k, r in enumerate(rows)]
    ws = [torch.from_numpy(pti.pack_ssq(d["A"], d["B"], d["sA"], d["sB"])).to(dev) for d in ds]
    xa = torch.from_numpy(ds[0]["xA"]).to(dev)
    xb = torch.from_numpy(ds[0]["xB"]).to(dev)
    ya, yb = pti.gemv_ssq_grouped(ws, xa, xb)
    torch.cuda.synchronize()
    r0 = 0
    for w, r in zip(ws, rows):
        sa, sb = pti.gemv_ssq(w, xa, xb)
        torch.cuda.synchronize()
        assert np.array_equal(bits(ya[r0:r0 + r]), bits(sa)) and np.array_equal(bits(yb[r0:r0 + r]), bits(sb))
        r0 += r


@pytest.mark.parametrize("n", [1, 2, 3, 4])
@pytest.mark.parametrize("name,cols,rows", GROUPS, ids=[g[0] for g in GROUPS])
def test_q8_grouped_equals_single(env, name, cols, rows, n):
    torch, pti, dev = env
    _note(f"q8 grouped {name} n={n}: cols {cols}, rows {rows}")
    qs = [synth.q8(r, cols, n, seed=7 * k + r + n) for k, r in enumerate(rows)]
    ws = [torch.from_numpy(pti.pack_q8(q["Q"], q["S"])).to(dev) for q in qs]
    x = torch.from_numpy(np.ascontiguousarray(qs[0]["X"])).to(dev)
    y = pti.gemv_q8_multi_grouped(ws, x)
    torch.cuda.synchronize()
    r0 = 0
    for w, r in zip(ws, rows):
        ys = pti.gemv_q8_multi(w, x)
        torch.cuda.synchronize()
        assert np.array_equal(bits(y[:, r0:r0 + r].contiguous()), bits(ys))
        r0 += r


def test_grouped_vs_oracle(env):
    """q|k|v at full size, Q8 N = 4 and SSQ, every row of every matrix."""
    torch, pti, dev = env
    cols, rows = 5120, [5120, 1024, 1024]
    _note("grouped vs oracle: qkv 5120/1024/1024 x 5120")
    qs = [synth.q8(r, cols, 4, seed=900 + r) for r in rows]
    ws = [torch.from_numpy(pti.pack_q8(q["Q"], q["S"])).to(dev) for q in qs]
    X = qs[0]["X"]
    y = pti.gemv_q8_multi_grouped(ws, torch.from_numpy(np.ascontiguousarray(X)).to(dev)).cpu().numpy()
    r0 = 0
    for q, r in zip(qs, rows):
        e, t = oracle.gemv_q8(oracle.pack_q8(q["Q"], q["S"]), r, cols, X)
        for s in range(4):
            err = np.abs(y[s, r0:r0 + r].astype(np.float64) - e[s])
            assert np.all(err <= 1e-5 * t[s]), (r, s)
        r0 += r
    ds = [synth.twin(r, cols, seed=950 + r) for r in rows]
    ws = [torch.from_numpy(pti.pack_ssq(d["A"], d["B"], d["sA"], d["sB"])).to(dev) for d in ds]
    ya, yb = pti.gemv_ssq_grouped(ws, torch.from_numpy(ds[0]["xA"]).to(dev), torch.from_numpy(ds[0]["xB"]).to(dev))
    ya, yb = ya.cpu().numpy(), yb.cpu().numpy()
    r0 = 0
    for d, r in zip(ds, rows):
        ea, eb, ta, tb = oracle.gemv_ssq(oracle.pack_ssq(d["A"], d["B"], d["sA"], d["sB"]), r, cols,
                                         ds[0]["xA"], ds[0]["xB"])
        assert np.all(np.abs(ya[r0:r0 + r].astype(np.float64) - ea) <= 1e-5 * ta)
        assert np.all(np.abs(yb[r0:r0 + r].astype(np.float64) - eb) <= 1e-5 * tb)
        r0 += r

"""GPU parity of the SSQ twin GEMV with two streams per twin (pti_gemv_ssq_multi).

Bar: every (twin, stream) output is bitwise the output of pti_gemv_ssq on
that stream's pair of activation vectors (the per-row arithmetic does not
depend on the stream count), and the full-size case is within
1e-5 * sum |terms| of the oracle on every row.
"""


import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

# row-split shapes with 1..5 rounds per wave (4-wave and 8-wave launch
# bounds at five rounds), ragged tails, and rows too long for the row split
SHAPES = [(1, 32), (3, 96), (37, 512), (129, 1056), (200, 2048), (256, 2560), (777, 5120), (300, 10240),
          (260, 15360), (64, 20480), (300, 20992)]


@pytest.fixture(scope="module")
def env():
    import torch

    import packed_twin_int8_amd as pti
    assert torch.cuda.is_available()
    pti.lib()
    return torch, pti, torch.device("cuda:0")


def bits(t):
    return t.contiguous().cpu().numpy().view(np.uint32)


def run(env, rows, cols, seed):
    torch, pti, dev = env
    print(f"ssq multi {rows}x{cols} seed {seed}", flush=True)
    d = synth.twin(rows, cols, seed)
    g = np.random.default_rng(seed + 1)
    xa2 = g.standard_normal((2, cols)).astype(np.float32)
    xb2 = g.standard_normal((2, cols)).astype(np.float32)
    xa2[0], xb2[0] = d["xA"], d["xB"]
    w = torch.from_numpy(pti.pack_ssq(d["A"], d["B"], d["sA"], d["sB"])).to(dev)
    xa, xb = torch.from_numpy(xa2).to(dev), torch.from_numpy(xb2).to(dev)
    ya, yb = pti.gemv_ssq_multi(w, xa, xb)
    torch.cuda.synchronize()
    for j in range(2):
        sa, sb = pti.gemv_ssq(w, xa[j].contiguous(), xb[j].contiguous())
        torch.cuda.synchronize()
        assert np.array_equal(bits(ya[j]), bits(sa)), f"twin A stream {j}"
        assert np.array_equal(bits(yb[j]), bits(sb)), f"twin B stream {j}"
    ya1, yb1 = pti.gemv_ssq_multi(w, xa[:1], xb[:1])
    torch.cuda.synchronize()
    assert np.array_equal(bits(ya1[0]), bits(ya[0])) and np.array_equal(bits(yb1[0]), bits(yb[0]))
    return d, xa2, xb2, ya.cpu().numpy(), yb.cpu().numpy()


@pytest.mark.parametrize("rows,cols", SHAPES, ids=[f"{r}x{c}" for r, c in SHAPES])
def test_ssq_multi_equals_single(env, rows, cols):
    run(env, rows, cols, seed=3 * rows + cols)


def test_ssq_multi_full_vs_oracle(env):
    """17408 x 5120, two streams per twin, every row of all four outputs."""
    rows, cols = 17408, 5120
    d, xa2, xb2, ya, yb = run(env, rows, cols, synth.SEED_SSQ_FFN)
    P = oracle.pack_ssq(d["A"], d["B"], d["sA"], d["sB"])
    for j in range(2):
        ea, eb, ta, tb = oracle.gemv_ssq(P, rows, cols, xa2[j], xb2[j])
        assert np.all(np.abs(ya[j].astype(np.float64) - ea) <= 1e-5 * ta)
        assert np.all(np.abs(yb[j].astype(np.float64) - eb) <= 1e-5 * tb)

"""GPU parity of the fused SSQ twin GEMV + greedy verify (pti_gemv_ssq_verify).

Bars:
  * y_a, y_b: bitwise equal to pti_gemv_ssq's on the same inputs, and within
    1e-5 * sum_c |scale*q*x| of the oracle's exact GEMV;
  * argmax_out and accept_out: bit-exact against the oracle's verify applied
    to the GPU's own y (the fused call must pick the same row as a separate
    verify would, ties to the lowest row, -0 equal to +0);
  * the workspace needs no initialisation (garbage in it changes nothing),
    and calls chain in stream order with one workspace.
"""

import sys

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = 1e-5

# (rows, cols): row-split shapes with 1..5 rounds per wave, ragged tails,
# fewer rows than workgroups, and rows too long for the row-split kernel
# (more than 40 rounds of 512 columns: GEMV then the separate verify kernel)
SHAPES = [
    (1, 32),
    (3, 96),
    (37, 512),
    (129, 1056),
    (200, 2048),
    (256, 2560),
    (1000, 4096),
    (777, 5120),
    (300, 20992),
    (5, 21024),
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


def check_bound(y_gpu, y_exact, t_exact, what):
    err = np.abs(np.asarray(y_gpu, np.float64) - y_exact)
    bad = err > TOL * t_exact
    assert not bad.any(), f"{what}: {bad.sum()} outputs over 1e-5*T"


def upload(env, d):
    torch, pti, dev = env
    w = torch.from_numpy(pti.pack_ssq(d["A"], d["B"], d["sA"], d["sB"])).to(dev)
    return w, torch.from_numpy(d["xA"]).to(dev), torch.from_numpy(d["xB"]).to(dev)


def fused(env, w, xa, xb, tokens, work):
    torch, pti, dev = env
    t = torch.tensor(np.asarray(tokens, np.int32), device=dev)
    ya, yb, am, acc = pti.gemv_ssq_verify(w, xa, xb, t, work)
    torch.cuda.synchronize()
    return ya.cpu().numpy(), yb.cpu().numpy(), am.cpu().numpy(), int(acc.cpu().numpy()[0])


def check_verify(ya, yb, am, acc, tokens):
    want, want_acc = oracle.verify_argmax(np.stack([ya, yb]), np.asarray(tokens, np.int32))
    assert list(am) == list(want), (list(am), list(want))
    assert acc == want_acc


@pytest.mark.parametrize("rows,cols", SHAPES, ids=[f"{r}x{c}" for r, c in SHAPES])
def test_fused_vs_gemv_and_oracle(env, rows, cols):
    torch, pti, dev = env
    _note(f"fused ssq+verify {rows}x{cols}")
    d = synth.twin(rows, cols, seed=11 * rows + cols)
    w, xa, xb = upload(env, d)
    work = pti.ssq_verify_workspace(dev)
    ra, rb = pti.gemv_ssq(w, xa, xb)
    torch.cuda.synchronize()
    ra, rb = ra.cpu().numpy(), rb.cpu().numpy()
    ya, yb, am, acc = fused(env, w, xa, xb, [0, 0], work)
    assert np.array_equal(ya.view(np.uint32), ra.view(np.uint32))
    assert np.array_equal(yb.view(np.uint32), rb.view(np.uint32))
    ea, eb, ta, tb = oracle.gemv_ssq(oracle.pack_ssq(d["A"], d["B"], d["sA"], d["sB"]), rows, cols,
                                     d["xA"], d["xB"])
    check_bound(ya, ea, ta, "y_A")
    check_bound(yb, eb, tb, "y_B")
    check_verify(ya, yb, am, acc, [0, 0])
    # twin B's guess equal to twin A's token, then one that differs
    for guess in (int(am[0]), (int(am[0]) + 1) % rows):
        ya2, yb2, am2, acc2 = fused(env, w, xa, xb, [123, guess], work)
        assert np.array_equal(ya2.view(np.uint32), ya.view(np.uint32))
        check_verify(ya2, yb2, am2, acc2, [123, guess])
        assert acc2 == (2 if guess == am[0] else 1) or rows == 1


def test_fused_full_17408x5120(env):
    torch, pti, dev = env
    rows, cols = 17408, 5120
    _note("fused ssq+verify 17408x5120, seed 2")
    d = synth.twin(rows, cols, synth.SEED_SSQ_FFN)
    w, xa, xb = upload(env, d)
    work = pti.ssq_verify_workspace(dev)
    ra, rb = pti.gemv_ssq(w, xa, xb)
    ya, yb, am, acc = fused(env, w, xa, xb, [0, 7], work)
    assert np.array_equal(ya.view(np.uint32), ra.cpu().numpy().view(np.uint32))
    assert np.array_equal(yb.view(np.uint32), rb.cpu().numpy().view(np.uint32))
    check_verify(ya, yb, am, acc, [0, 7])
    # every row of both twins against the oracle
    ea, eb, ta, tb = oracle.gemv_ssq(oracle.pack_ssq(d["A"], d["B"], d["sA"], d["sB"]), rows, cols, d["xA"], d["xB"])
    check_bound(ya, ea, ta, "y_A")
    check_bound(yb, eb, tb, "y_B")
    # twin B's guess is twin A's token: both checks pass
    ya2, yb2, am2, acc2 = fused(env, w, xa, xb, [0, int(am[0])], work)
    check_verify(ya2, yb2, am2, acc2, [0, int(am[0])])
    assert acc2 == 2


@pytest.mark.parametrize("rows,cols", [(1000, 2048), (17408, 5120), (300, 20992)])
def test_fused_ties_lowest_row(env, rows, cols):
    """Copies of the winning row at spread positions (different workgroups and
    wave slots): equal rows give bitwise equal outputs, so the fused argmax
    must return the lowest copy."""
    torch, pti, dev = env
    _note(f"fused ties {rows}x{cols}")
    d = synth.twin(rows, cols, seed=rows + 5)
    w, xa, xb = upload(env, d)
    ra, rb = pti.gemv_ssq(w, xa, xb)
    torch.cuda.synchronize()
    best = [int(np.argmax(ra.cpu().numpy())), int(np.argmax(rb.cpu().numpy()))]
    copies = sorted({3, rows // 3, rows // 2 + 1, rows - 1})
    for name, src in (("A", best[0]), ("B", best[1])):
        q, s = ("A", "sA") if name == "A" else ("B", "sB")
        for c in copies:
            d[q][c] = d[q][src]
            d[s][c] = d[s][src]
    w, xa, xb = upload(env, d)
    work = pti.ssq_verify_workspace(dev)
    ya, yb, am, acc = fused(env, w, xa, xb, [0, 0], work)
    assert list(am) == [min(copies + [best[0]]), min(copies + [best[1]])]
    check_verify(ya, yb, am, acc, [0, 0])


def test_fused_all_equal_and_signed_zero(env):
    """x = 0: every output is +-0, all tied -- the argmax is row 0."""
    torch, pti, dev = env
    rows, cols = 4099, 2560
    d = synth.twin(rows, cols, seed=99)
    d["xA"][:] = 0.0
    d["xB"][:] = -0.0
    w, xa, xb = upload(env, d)
    work = pti.ssq_verify_workspace(dev)
    ya, yb, am, acc = fused(env, w, xa, xb, [0, 0], work)
    assert not np.any(ya) and not np.any(yb)
    assert list(am) == [0, 0] and acc == 2


def test_fused_chained_calls_one_workspace(env):
    """Several calls queued back to back on one stream with one workspace,
    with a smaller matrix in between: each call's results as if alone."""
    torch, pti, dev = env
    shapes = [(2048, 4096), (129, 1056), (2048, 4096), (300, 20992), (2048, 4096)]
    work = pti.ssq_verify_workspace(dev)
    runs = []
    for k, (rows, cols) in enumerate(shapes):
        d = synth.twin(rows, cols, seed=1000 + k)
        w, xa, xb = upload(env, d)
        t = torch.tensor([0, k % 3], dtype=torch.int32, device=dev)
        runs.append((w, xa, xb, t) + pti.gemv_ssq_verify(w, xa, xb, t, work))
    torch.cuda.synchronize()
    for w, xa, xb, t, ya, yb, am, acc in runs:
        ra, rb = pti.gemv_ssq(w, xa, xb)
        torch.cuda.synchronize()
        assert torch.equal(ya, ra) and torch.equal(yb, rb)
        check_verify(ya.cpu().numpy(), yb.cpu().numpy(), am.cpu().numpy(), int(acc.cpu()[0]), t.cpu().numpy())


@pytest.mark.parametrize("fill", [0x00, 0xFF, 0x7F])
def test_fused_workspace_contents_ignored(env, fill):
    torch, pti, dev = env
    rows, cols = 5000, 3072
    d = synth.twin(rows, cols, seed=77)
    w, xa, xb = upload(env, d)
    work = torch.full((pti.SSQ_VERIFY_WORK_BYTES,), fill, dtype=torch.uint8, device=dev)
    ya, yb, am, acc = fused(env, w, xa, xb, [0, 0], work)
    check_verify(ya, yb, am, acc, [0, 0])

"""GPU parity: libpti's HIP kernels against the fp64 oracle (MI355X).

Bars (the oracle computes every expected value from the same seeded raw
arrays, packed by its own packer):
  * fp32 GEMV outputs: |y_gpu - y_exact| <= 1e-5 * sum_c |scale*q*x| per output;
  * closed forms (one-hot x, unit scales with all-ones x): bit-exact;
  * argmax and accept counts: bit-exact, with the oracle applied to the GPU's
    own logits;
  * every row of the full-size (17408 x 5120) and decoder-layer outputs, in
    the launch configuration the benchmark times;
  * properties: SSQ twin == Q8 GEMVs of the split halves (within the bound),
    A==B twins with equal x give bitwise identical outputs, a stream's output
    does not depend on the stream count or its slot, repeated calls are
    bitwise identical.
"""

import sys

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = 1e-5


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
    y_gpu = np.asarray(y_gpu, np.float64)
    err = np.abs(y_gpu - y_exact)
    bound = TOL * t_exact
    bad = err > bound
    ratio = float(np.max(err / np.maximum(t_exact, 1e-300)))
    assert not bad.any(), f"{what}: {bad.sum()} outputs over 1e-5*T, worst ratio {ratio:.3e}"
    return ratio


def run_ssq(env, d, rows, cols):
    torch, pti, dev = env
    P = pti.pack_ssq(d["A"], d["B"], d["sA"], d["sB"])
    w = torch.from_numpy(P).to(dev)
    xa = torch.from_numpy(d["xA"]).to(dev)
    xb = torch.from_numpy(d["xB"]).to(dev)
    ya, yb = pti.gemv_ssq(w, xa, xb)
    torch.cuda.synchronize()
    return ya.cpu().numpy(), yb.cpu().numpy()


def run_q8(env, Q, S, X):
    torch, pti, dev = env
    w = torch.from_numpy(pti.pack_q8(Q, S)).to(dev)
    x = torch.from_numpy(np.ascontiguousarray(X, np.float32)).to(dev)
    y = pti.gemv_q8_multi(w, x)
    torch.cuda.synchronize()
    return y.cpu().numpy()


# ------------------------------------------------------------ tiny SSQ twin

def test_tiny_ssq_twin(env):
    rows, cols = 256, 512
    _note(f"tiny ssq {rows}x{cols} seed {synth.SEED_TINY}")
    d = synth.twin(rows, cols, synth.SEED_TINY)
    ya, yb = run_ssq(env, d, rows, cols)
    Po = oracle.pack_ssq(d["A"], d["B"], d["sA"], d["sB"])
    ea, eb, ta, tb = oracle.gemv_ssq(Po, rows, cols, d["xA"], d["xB"])
    ra = check_bound(ya, ea, ta, "y_A")
    rb = check_bound(yb, eb, tb, "y_B")
    _note(f"  worst |err|/T: A {ra:.2e}  B {rb:.2e}")


def test_tiny_ssq_same_twins(env):
    rows, cols = 256, 512
    d = synth.twin(rows, cols, synth.SEED_TINY, same=True, same_x=True)
    ya, yb = run_ssq(env, d, rows, cols)
    assert np.array_equal(ya.view(np.uint32), yb.view(np.uint32))
    # A == B twins, independent activations
    d = synth.twin(rows, cols, synth.SEED_TINY, same=True)
    ya, yb = run_ssq(env, d, rows, cols)
    ea, eb, ta, tb = oracle.gemv_ssq(oracle.pack_ssq(d["A"], d["B"], d["sA"], d["sB"]), rows, cols, d["xA"], d["xB"])
    check_bound(ya, ea, ta, "y_A")
    check_bound(yb, eb, tb, "y_B")


def test_closed_forms_bit_exact(env):
    torch, pti, dev = env
    rows, cols = 37, 160
    d = synth.twin(rows, cols, 21)
    P = torch.from_numpy(pti.pack_ssq(d["A"], d["B"], d["sA"], d["sB"])).to(dev)
    sa = d["sA"].view(np.float16).astype(np.float64)
    sb = d["sB"].view(np.float16).astype(np.float64)
    for c in (0, 1, 31, 32, 63, 64, 100, 159):
        e = np.zeros(cols, np.float32)
        e[c] = 1.0
        ya, yb = pti.gemv_ssq(P, torch.from_numpy(e).to(dev), torch.from_numpy(-e).to(dev))
        wa = sa[:, c // 32] * d["A"][:, c]
        wb = sb[:, c // 32] * d["B"][:, c]
        assert np.array_equal(ya.cpu().numpy().astype(np.float64), wa.astype(np.float32).astype(np.float64)), c
        assert np.array_equal(yb.cpu().numpy().astype(np.float64), (-wb).astype(np.float32).astype(np.float64)), c
    # unit scales, all-ones x: integer row sums, exact in fp32
    one = np.full((rows, cols // 32), 0x3C00, np.uint16)
    ones = np.ones(cols, np.float32)
    y = run_q8(env, d["B"], one, np.stack([ones, 2 * ones, -ones]))
    s = d["B"].astype(np.int64).sum(1).astype(np.float64)
    assert np.array_equal(y[0], s) and np.array_equal(y[1], 2 * s) and np.array_equal(y[2], -s)


# ------------------------------------------------------------ Q8 multi-stream

SHAPES = [
    (1, 32),      # one block: half unit, odd block count
    (3, 96),      # odd block count
    (37, 512),
    (129, 1056),  # 33 blocks: odd, two rounds with a ragged tail
    (200, 2048),
    (65, 5120),
    (64, 5632),
    (40, 17408),  # x split into several LDS chunks at 4 streams
    (8192, 1024),  # the largest row count of the Q8 row-split form
    (8193, 1024),  # the smallest above it (per-wave-row kernel)
    (1, 64),       # two blocks, one row: four of 64 lanes hold weights
    (2, 1088),     # 34 blocks: two rounds, ragged
    (5, 20480),    # Q8: 20 rounds, the most the row-split form takes; SSQ: 40
    (5, 20544),    # one round more (per-wave-row kernel for both formats)
]


@pytest.mark.parametrize("rows,cols", SHAPES, ids=[f"{r}x{c}" for r, c in SHAPES])
@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_q8_multi_vs_oracle(env, rows, cols, n):
    _note(f"q8 {rows}x{cols} n={n}")
    d = synth.q8(rows, cols, n, seed=rows + cols + n)
    y = run_q8(env, d["Q"], d["S"], d["X"])
    e, t = oracle.gemv_q8(oracle.pack_q8(d["Q"], d["S"]), rows, cols, d["X"])
    for s in range(n):
        check_bound(y[s], e[s], t[s], f"stream {s}")


@pytest.mark.parametrize("rows,cols", SHAPES, ids=[f"{r}x{c}" for r, c in SHAPES])
def test_ssq_vs_oracle_and_split(env, rows, cols):
    _note(f"ssq {rows}x{cols}")
    d = synth.twin(rows, cols, seed=7 * rows + cols)
    ya, yb = run_ssq(env, d, rows, cols)
    ea, eb, ta, tb = oracle.gemv_ssq(oracle.pack_ssq(d["A"], d["B"], d["sA"], d["sB"]), rows, cols, d["xA"], d["xB"])
    check_bound(ya, ea, ta, "y_A")
    check_bound(yb, eb, tb, "y_B")
    # the twin GEMV equals two Q8 GEMVs over the split halves (both within the
    # bound of the exact result, so within twice the bound of each other)
    torch, pti, dev = env
    qa8, qb8 = pti.ssq_split(pti.pack_ssq(d["A"], d["B"], d["sA"], d["sB"]), rows, cols)
    assert np.array_equal(qa8, pti.pack_q8(d["A"], d["sA"])) and np.array_equal(qb8, pti.pack_q8(d["B"], d["sB"]))
    qa = run_q8(env, d["A"], d["sA"], d["xA"][None])
    qb = run_q8(env, d["B"], d["sB"], d["xB"][None])
    check_bound(qa[0], ea, ta, "q8(A)")
    check_bound(qb[0], eb, tb, "q8(B)")
    assert np.all(np.abs(ya.astype(np.float64) - qa[0]) <= 2 * TOL * ta)
    assert np.all(np.abs(yb.astype(np.float64) - qb[0]) <= 2 * TOL * tb)


# (129, 1056): odd block count, per-wave-row kernel; (300, 5120), (40, 17408):
# the row-split form (one and four waves per row); (8193, 1024): above the
# row-split form's row limit; (8200, 5120): above it with rows of one wave of
# five rounds, which one and two streams run in the row-split kernel and three
# and four in the per-wave-row kernel; (5, 20544) and (8200, 12288): the
# per-wave-row kernel with x staged in LDS chunks at some stream counts and
# whole at others (20544 columns: chunked from two streams on; 12288: from
# three on)
@pytest.mark.parametrize("rows,cols", [(129, 1056), (300, 5120), (40, 17408), (8193, 1024), (8200, 5120), (5, 20544),
                                       (8200, 12288)])
def test_stream_slot_invariance(env, rows, cols):
    d = synth.q8(rows, cols, 4, seed=33)
    single = [run_q8(env, d["Q"], d["S"], d["X"][s:s + 1])[0] for s in range(4)]
    for n in (2, 3, 4):
        for perm in ([0, 1, 2, 3], [3, 2, 1, 0], [2, 0, 3, 1]):
            X = d["X"][perm[:n]]
            y = run_q8(env, d["Q"], d["S"], X)
            for slot in range(n):
                assert np.array_equal(y[slot].view(np.uint32), single[perm[slot]].view(np.uint32)), (n, perm, slot)


def test_repeat_determinism(env):
    torch, pti, dev = env
    rows, cols = 1000, 5120
    d = synth.q8(rows, cols, 4, seed=44)
    w = torch.from_numpy(pti.pack_q8(d["Q"], d["S"])).to(dev)
    x = torch.from_numpy(d["X"]).to(dev)
    y0 = pti.gemv_q8_multi(w, x).cpu().numpy()
    for _ in range(3):
        y1 = pti.gemv_q8_multi(w, x).cpu().numpy()
        assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32))


def test_outputs_overwritten_and_aliased_inputs(env):
    torch, pti, dev = env
    rows, cols = 50, 512
    d = synth.twin(rows, cols, 5)
    w = torch.from_numpy(pti.pack_ssq(d["A"], d["B"], d["sA"], d["sB"])).to(dev)
    x = torch.from_numpy(d["xA"]).to(dev)
    ya = torch.full((rows,), float("nan"), device=dev)
    yb = torch.full((rows,), 1e30, device=dev)
    pti.gemv_ssq(w, x, x, ya, yb)  # x_a and x_b alias
    ea, eb, ta, tb = oracle.gemv_ssq(oracle.pack_ssq(d["A"], d["B"], d["sA"], d["sB"]), rows, cols, d["xA"], d["xA"])
    check_bound(ya.cpu().numpy(), ea, ta, "y_A")
    check_bound(yb.cpu().numpy(), eb, tb, "y_B")


def test_scale_edge_values(env):
    """Subnormal, negative, zero and the largest finite f16 scales."""
    rows, cols = 16, 256
    d = synth.q8(rows, cols, 2, seed=8)
    S = d["S"].copy()
    S[0, :] = 0x0001   # smallest subnormal
    S[1, :] = 0x03FF   # largest subnormal
    S[2, :] = 0x8000   # -0
    S[3, :] = 0xBC00   # -1
    S[4, :] = 0x7BFF   # 65504
    S[5, 3] = 0x0000
    Q = d["Q"].copy()
    Q[6, :] = -128
    Q[7, :] = 127
    y = run_q8(env, Q, S, d["X"])
    e, t = oracle.gemv_q8(oracle.pack_q8(Q, S), rows, cols, d["X"])
    for s in range(2):
        check_bound(y[s], e[s], t[s], f"stream {s}")


# ------------------------------------------------------------ full-size shapes
# Every row of every full-size output is compared with the oracle's full GEMV
# (the oracle computes a 17408 x 5120 twin GEMV in about a tenth of a second).


def test_full_ssq_17408x5120_all_rows(env):
    rows, cols = 17408, 5120
    _note("full ssq 17408x5120, seed 2, every row")
    d = synth.twin(rows, cols, synth.SEED_SSQ_FFN)
    ya, yb = run_ssq(env, d, rows, cols)
    ea, eb, ta, tb = oracle.gemv_ssq(oracle.pack_ssq(d["A"], d["B"], d["sA"], d["sB"]), rows, cols, d["xA"], d["xB"])
    ra = check_bound(ya, ea, ta, "y_A")
    rb = check_bound(yb, eb, tb, "y_B")
    _note(f"  worst |err|/T over {rows} rows: A {ra:.2e}  B {rb:.2e}")


def test_full_ssq_17408x5120_same_twins(env):
    """The self-twin (A == B) at the benchmark's shape: with one x for both
    twins the outputs are bitwise equal; with independent x each is within
    the bound of the oracle, every row."""
    rows, cols = 17408, 5120
    _note("full ssq 17408x5120 A == B")
    d = synth.twin(rows, cols, synth.SEED_SSQ_FFN, same=True, same_x=True)
    ya, yb = run_ssq(env, d, rows, cols)
    assert np.array_equal(ya.view(np.uint32), yb.view(np.uint32))
    d = synth.twin(rows, cols, synth.SEED_SSQ_FFN, same=True)
    ya, yb = run_ssq(env, d, rows, cols)
    ea, eb, ta, tb = oracle.gemv_ssq(oracle.pack_ssq(d["A"], d["B"], d["sA"], d["sB"]), rows, cols, d["xA"], d["xB"])
    check_bound(ya, ea, ta, "y_A")
    check_bound(yb, eb, tb, "y_B")


@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_full_q8_17408x5120_all_rows(env, n):
    rows, cols = 17408, 5120
    _note(f"full q8 17408x5120 n={n}, seed 3, every row")
    d = synth.q8(rows, cols, n, synth.SEED_Q8_FFN)
    y = run_q8(env, d["Q"], d["S"], d["X"])
    e, t = oracle.gemv_q8(oracle.pack_q8(d["Q"], d["S"]), rows, cols, d["X"])
    for s in range(n):
        r = check_bound(y[s], e[s], t[s], f"stream {s}")
        _note(f"  stream {s}: worst |err|/T {r:.2e}")


@pytest.mark.parametrize("name,rows,cols", synth.LAYER_SHAPES, ids=[s[0] for s in synth.LAYER_SHAPES])
def test_layer_sweep_all_rows(env, name, rows, cols):
    """One decoder layer's matrices at their real shapes, every row: SSQ with
    distinct twins, SSQ with A == B (bitwise equal twins on one x, and within
    the bound on independent x), and Q8 at one, two and four streams (each
    stream count its own call, so each runs the kernel it takes)."""
    _note(f"layer {name} {rows}x{cols}")
    d = synth.twin(rows, cols, synth.SEED_LAYER)
    ya, yb = run_ssq(env, d, rows, cols)
    ea, eb, ta, tb = oracle.gemv_ssq(oracle.pack_ssq(d["A"], d["B"], d["sA"], d["sB"]), rows, cols, d["xA"], d["xB"])
    check_bound(ya, ea, ta, "y_A")
    check_bound(yb, eb, tb, "y_B")
    s = synth.twin(rows, cols, synth.SEED_LAYER, same=True, same_x=True)
    sa, sb = run_ssq(env, s, rows, cols)
    assert np.array_equal(sa.view(np.uint32), sb.view(np.uint32)), "A == B twins on one x"
    s = synth.twin(rows, cols, synth.SEED_LAYER, same=True)
    sa, sb = run_ssq(env, s, rows, cols)
    esa, esb, tsa, tsb = oracle.gemv_ssq(oracle.pack_ssq(s["A"], s["B"], s["sA"], s["sB"]), rows, cols,
                                         s["xA"], s["xB"])
    check_bound(sa, esa, tsa, "A == B, y_A")
    check_bound(sb, esb, tsb, "A == B, y_B")
    X = np.stack([d["xA"], d["xB"], -d["xA"], d["xB"] * 0.5])
    e, t = oracle.gemv_q8(oracle.pack_q8(d["A"], d["sA"]), rows, cols, X)
    for n in (1, 2, 4):
        y = run_q8(env, d["A"], d["sA"], X[:n])
        for k in range(n):
            check_bound(y[k], e[k], t[k], f"q8 n={n} stream {k}")
        assert np.all(np.abs(y[0].astype(np.float64) - ya) <= 2 * TOL * ta)


# Edge values in SSQ slots and scales: -128 in the high byte (twin A), the low
# byte (twin B) or both; for each twin's scale the smallest and largest
# subnormals, -0, +0, -1 and 65504.  (120, 640): the row-split kernel;
# (12, 20544): rows of 41 rounds, the per-wave-row kernel.
SSQ_EDGE_SHAPES = [(120, 640), (12, 20544)]


def ssq_edge_inputs(rows, cols, seed):
    d = synth.twin(rows, cols, seed)
    A, B, sA, sB = d["A"], d["B"], d["sA"], d["sB"]
    A[0, :] = -128
    B[1, :] = -128
    A[2, :] = -128
    B[2, :] = -128
    A[3, ::2] = -128
    B[3, 1::2] = -128
    edges = [0x0001, 0x03FF, 0x8000, 0x0000, 0xBC00, 0x7BFF]
    for k, v in enumerate(edges):
        sA[4 + k % (rows - 4), :] = v
        sB[4 + (k + 3) % (rows - 4), :] = v
    sA[0, 0], sB[1, -1] = 0x7BFF, 0x0001
    return d


@pytest.mark.parametrize("rows,cols", SSQ_EDGE_SHAPES, ids=[f"{r}x{c}" for r, c in SSQ_EDGE_SHAPES])
def test_ssq_edge_values(env, rows, cols):
    torch, pti, dev = env
    _note(f"ssq edge values {rows}x{cols}")
    d = ssq_edge_inputs(rows, cols, 91)
    ya, yb = run_ssq(env, d, rows, cols)
    ea, eb, ta, tb = oracle.gemv_ssq(oracle.pack_ssq(d["A"], d["B"], d["sA"], d["sB"]), rows, cols, d["xA"], d["xB"])
    check_bound(ya, ea, ta, "y_A")
    check_bound(yb, eb, tb, "y_B")
    # the fused step and two streams per twin run the same rows
    w = torch.from_numpy(pti.pack_ssq(d["A"], d["B"], d["sA"], d["sB"])).to(dev)
    xa, xb = torch.from_numpy(d["xA"]).to(dev), torch.from_numpy(d["xB"]).to(dev)
    fa, fb, am, acc = pti.gemv_ssq_verify(w, xa, xb, torch.zeros(2, dtype=torch.int32, device=dev),
                                          pti.ssq_verify_workspace(dev))
    torch.cuda.synchronize()
    assert np.array_equal(fa.cpu().numpy().view(np.uint32), ya.view(np.uint32))
    assert np.array_equal(fb.cpu().numpy().view(np.uint32), yb.view(np.uint32))
    want, _ = oracle.verify_argmax(np.stack([ya, yb]), np.zeros(2, np.int32))
    assert list(am.cpu().numpy()) == list(want)
    ma, mb = pti.gemv_ssq_multi(w, torch.stack([xa, -xa]), torch.stack([xb, xb * 2]))
    torch.cuda.synchronize()
    assert np.array_equal(ma[0].cpu().numpy().view(np.uint32), ya.view(np.uint32))
    assert np.array_equal(mb[0].cpu().numpy().view(np.uint32), yb.view(np.uint32))
    e2a, e2b, t2a, t2b = oracle.gemv_ssq(oracle.pack_ssq(d["A"], d["B"], d["sA"], d["sB"]), rows, cols,
                                         -d["xA"], d["xB"] * 2)
    check_bound(ma[1].cpu().numpy(), e2a, t2a, "multi y_A stream 1")
    check_bound(mb[1].cpu().numpy(), e2b, t2b, "multi y_B stream 1")


# ------------------------------------------------------------ beyond 4 GiB

def _tiled(env, base, rows):
    """Device matrix of `rows` rows repeating the packed rows of `base`."""
    torch, pti, dev = env
    b = torch.from_numpy(base).to(dev)
    reps = (rows + base.shape[0] - 1) // base.shape[0]
    return b.repeat(reps, 1)[:rows].contiguous()


def test_q8_beyond_4gib_all_rows(env):
    """4.56 GB of Q8 weights (4,194,309 rows x 1024 cols, 1088-byte rows):
    the byte offsets of rows pass 2^31 and 2^32.  The matrix repeats a
    4096-row base whose period (4096 x 1088 bytes) divides neither, so a
    wrapped offset lands on a row with other values.  Every row is checked
    against the oracle's result for its base row."""
    torch, pti, dev = env
    rows, cols, period = (1 << 22) + 5, 1024, 4096
    _note(f"q8 {rows}x{cols} tiled from {period} rows")
    d = synth.q8(period, cols, 2, synth.SEED_BIG)
    w = _tiled(env, pti.pack_q8(d["Q"], d["S"]), rows)
    assert w.numel() > 2 ** 32
    y = pti.gemv_q8_multi(w, torch.from_numpy(d["X"]).to(dev))
    torch.cuda.synchronize()
    del w
    torch.cuda.empty_cache()
    e, t = oracle.gemv_q8(oracle.pack_q8(d["Q"], d["S"]), period, cols, d["X"])
    idx = np.arange(rows) % period
    y = y.cpu().numpy()
    for s in range(2):
        check_bound(y[s], e[s][idx], t[s][idx], f"stream {s}")


@pytest.mark.parametrize("n", [1, 2])
def test_q8_beyond_4gib_split_kernel_all_rows(env, n):
    """4.35 GB of Q8 weights at 5120 columns (800,003 rows of 5440 bytes): one
    and two streams take the row-split kernel for these tall rows of five
    rounds.  Row offsets pass 2^31 and 2^32; the 4096-row period
    (4096 x 5440 bytes) divides neither, so a wrapped offset reads other
    values.  Every row is checked against the oracle's result for its base
    row."""
    torch, pti, dev = env
    rows, cols, period = 800_003, 5120, 4096
    _note(f"q8 {rows}x{cols} n={n} tiled from {period} rows")
    d = synth.q8(period, cols, n, synth.SEED_BIG + n)
    w = _tiled(env, pti.pack_q8(d["Q"], d["S"]), rows)
    assert w.numel() > 2 ** 32
    y = pti.gemv_q8_multi(w, torch.from_numpy(d["X"]).to(dev))
    torch.cuda.synchronize()
    del w
    torch.cuda.empty_cache()
    e, t = oracle.gemv_q8(oracle.pack_q8(d["Q"], d["S"]), period, cols, d["X"])
    idx = np.arange(rows) % period
    y = y.cpu().numpy()
    for s in range(n):
        check_bound(y[s], e[s][idx], t[s][idx], f"stream {s}")


def test_ssq_beyond_4gib_all_rows(env):
    """The SSQ twin GEMV over 4.56 GB (2,097,155 rows x 1024 cols, 2176-byte
    rows, a 2048-row period), every row of both twins checked."""
    torch, pti, dev = env
    rows, cols, period = (1 << 21) + 3, 1024, 2048
    _note(f"ssq {rows}x{cols} tiled from {period} rows")
    d = synth.twin(period, cols, synth.SEED_BIG)
    w = _tiled(env, pti.pack_ssq(d["A"], d["B"], d["sA"], d["sB"]), rows)
    assert w.numel() > 2 ** 32
    ya, yb = pti.gemv_ssq(w, torch.from_numpy(d["xA"]).to(dev), torch.from_numpy(d["xB"]).to(dev))
    torch.cuda.synchronize()
    del w
    torch.cuda.empty_cache()
    ea, eb, ta, tb = oracle.gemv_ssq(oracle.pack_ssq(d["A"], d["B"], d["sA"], d["sB"]), period, cols, d["xA"],
                                     d["xB"])
    idx = np.arange(rows) % period
    check_bound(ya.cpu().numpy(), ea[idx], ta[idx], "y_A")
    check_bound(yb.cpu().numpy(), eb[idx], tb[idx], "y_B")


# ------------------------------------------------------------ verify

def gpu_verify(env, logits, tokens):
    torch, pti, dev = env
    L = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).to(dev)
    T = torch.from_numpy(np.asarray(tokens, np.int32)).to(dev)
    am, acc = pti.verify_argmax(L, T)
    torch.cuda.synchronize()
    return am.cpu().numpy(), int(acc.cpu().numpy()[0])


@pytest.mark.parametrize("vocab", [1, 3, 5, 1000, 32000, 32001, 151936])
@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_verify_random(env, vocab, n):
    g = np.random.default_rng(vocab * 10 + n)
    L = g.standard_normal((n, vocab)).astype(np.float32)
    am, _ = gpu_verify(env, L, np.zeros(n, np.int32))
    want, _ = oracle.verify_argmax(L, np.zeros(n, np.int32))
    assert np.array_equal(am, want)
    # guesses equal to the previous stream's argmax: every check passes
    tok = np.concatenate([[0], want[:-1]]).astype(np.int32)
    am2, acc = gpu_verify(env, L, tok)
    assert acc == n == oracle.verify_argmax(L, tok)[1]


def test_verify_ties_and_signed_zero(env):
    n, vocab = 4, 4096
    L = np.full((n, vocab), -3.0, np.float32)
    L[0, [5, 1000, 4095]] = 7.0          # first of three equal maxima
    L[1, [4095, 2048]] = 1.0             # across thread slices
    L[2, :] = -np.inf                    # all -inf: index 0
    L[3, 17] = -0.0
    L[3, 9] = 0.0
    L[3, :9] = -1.0
    L[3, 10:17] = -1.0
    L[3, 18:] = -1.0
    am, _ = gpu_verify(env, L, np.zeros(n, np.int32))
    want, _ = oracle.verify_argmax(L, np.zeros(n, np.int32))
    assert np.array_equal(am, want) and list(am) == [5, 2048, 0, 9]


def test_verify_accept_patterns_exhaustive(env):
    """Every tokens_in pattern over a 3-token alphabet against fixed argmaxes."""
    import itertools
    n, vocab = 4, 64
    L = np.full((n, vocab), -1.0, np.float32)
    amax = [1, 2, 0, 1]
    for s, t in enumerate(amax):
        L[s, t] = 5.0
    for tok in itertools.product(range(3), repeat=n):
        am, acc = gpu_verify(env, L, tok)
        assert list(am) == amax
        assert acc == oracle.accept_count(tok, am), tok

"""Pins of the fp64 toy decoder stack and the staggered loop (oracle/toy.py).

Each check ties the oracle to something other than itself: closed forms of
special cases, an independent implementation (the C oracle's packer and GEMV),
exact expectations from the acceptance enumeration, and planted mistakes that
must be caught.
"""

from __future__ import annotations

import inspect
import math
from fractions import Fraction

import numpy as np

import oracle
from oracle import accept as acc
from oracle import toy

F16 = {1.0: 0x3C00, 0.5: 0x3800, 2.0: 0x4000, 0.25: 0x3400, 0.0: 0x0000}


# ------------------------------------------------------------- elementwise pieces

def test_silu_closed_values():
    v = toy.silu(np.array([0.0, 1.0, -1.0, 2.0, 30.0, -30.0]))
    e = math.e
    want = [0.0, 1.0 / (1.0 + 1.0 / e), -1.0 / (1.0 + e), 2.0 / (1.0 + math.exp(-2.0)), 30.0, -30.0 * math.exp(-30.0)]
    np.testing.assert_allclose(v, want, rtol=1e-12, atol=1e-300)
    # odd part: silu(v) - silu(-v) = v
    x = np.linspace(-8, 8, 33)
    np.testing.assert_allclose(toy.silu(x) - toy.silu(-x), x, rtol=0, atol=1e-12)


def test_rmsnorm_closed_forms():
    # constant vector c: c / sqrt(c^2 + eps)
    for c, eps in ((3.0, 0.0), (1e-4, 1e-6), (-2.5, 1e-6)):
        y = toy.rmsnorm(np.full(64, c), eps)
        np.testing.assert_allclose(y, c / math.sqrt(c * c + eps), rtol=1e-14)
    # eps = 0: unit root-mean-square and invariance to positive scaling
    g = np.random.default_rng(5)
    x = g.standard_normal((3, 100))
    y = toy.rmsnorm(x, 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=1e-14)
    np.testing.assert_allclose(toy.rmsnorm(7.0 * x, 0.0), y, rtol=1e-13)
    # mean, not sum: a vector of ones stays ones
    np.testing.assert_allclose(toy.rmsnorm(np.ones(10), 0.0), 1.0, rtol=1e-15)


def test_dequant_matches_c_oracle_unpack():
    g = np.random.default_rng(6)
    Q = g.integers(-128, 128, size=(5, 96), dtype=np.int8)
    S = g.integers(0, 0x7C00, size=(5, 3)).astype(np.uint16)
    W = toy.dequant(Q, S)
    O = oracle.default()
    for r in range(5):
        for c in range(96):
            assert W[r, c] == O.f16_to_f64(S[r, c // 32]) * float(Q[r, c])
    assert toy.f16_to_f64(np.array([0x3C00, 0x0001, 0xC000], np.uint16)).tolist() == [1.0, 2.0 ** -24, -2.0]


def test_argmax_first_ties():
    assert toy.argmax_first(np.array([1.0, 3.0, 3.0, 2.0])) == 1
    assert toy.argmax_first(np.array([-0.0, 0.0])) == 0
    assert toy.argmax_first(np.array([5.0])) == 0


# ----------------------------------------------------------------- the stack

def _diag(n, scale_bits):
    """n x n int8 identity with one f16 scale per 32-column block of each row."""
    Q = np.eye(n, dtype=np.int8)
    S = np.full((n, n // 32), scale_bits, dtype=np.uint16)
    return dict(Q=Q, S=S)


def _tiny_raw(g, hidden=32, ffn=64, vocab=40, layers=2):
    def mat(r, c):
        return dict(Q=g.integers(-127, 128, size=(r, c), dtype=np.int8),
                    S=(g.uniform(1e-3, 1e-2, size=(r, c // 32)).astype(np.float16).view(np.uint16)))
    return dict(emb=mat(vocab, hidden), head=mat(vocab, hidden),
                layers=[dict(gate=mat(ffn, hidden), up=mat(ffn, hidden), down=mat(hidden, ffn)) for _ in range(layers)])


def test_layer_closed_form_diagonal():
    """Diagonal gate/up/down (a*I, b*I, c*I): h' = h + c * silu(a r) * (b r) per element, r = rmsnorm(h).
    Distinguishes gate from up (a != b), the norm's place, and the residual."""
    g = np.random.default_rng(7)
    n = 64
    raw = _tiny_raw(g, hidden=n, ffn=n, vocab=5, layers=1)
    a, b, c = 2.0, 0.5, 0.25
    raw["layers"][0] = dict(gate=_diag(n, F16[a]), up=_diag(n, F16[b]), down=_diag(n, F16[c]))
    m = toy.ToyModel(raw, eps=1e-6)
    for t in range(5):
        h = m.emb[t]
        ms = math.sqrt(sum(x * x for x in h) / n + 1e-6)
        want = [h[i] + c * (a * h[i] / ms) / (1.0 + math.exp(-a * h[i] / ms)) * (b * h[i] / ms) for i in range(n)]
        got = m.hidden_states([t])[-1][0]
        np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-15)


def test_zero_down_is_identity_and_head_matches_c_gemv():
    """down = 0 leaves h = embedding row; logits = head . rmsnorm(emb row), which
    the C oracle's Q8 GEMV computes independently from the packed head."""
    g = np.random.default_rng(8)
    raw = _tiny_raw(g, hidden=64, ffn=96, vocab=50, layers=3)
    for L in raw["layers"]:
        L["down"]["S"][:] = 0
    m = toy.ToyModel(raw, eps=1e-6)
    toks = [0, 7, 49]
    hs = m.hidden_states(toks)
    for h in hs:
        np.testing.assert_array_equal(h, m.emb[toks])
    O = oracle.default()
    P = O.pack_q8(raw["head"]["Q"], raw["head"]["S"])
    r = toy.rmsnorm(m.emb[toks], 1e-6)
    lg = m.logits(toks)
    for i in range(len(toks)):
        # the C GEMV takes fp32 activations: rounding r moves a logit by <= 2^-24 * t
        y, t = O.gemv_q8(P, 50, 64, r[i:i + 1])
        assert np.all(np.abs(lg[i] - y[0]) <= 2.0 ** -24 * t[0] * 1.01 + 1e-15)


def test_head_abs_terms_matches_c_oracle_t_and_brute_force():
    """T_v = sum_c |head[v][c] r[c]| with r = rmsnorm(h_L): the C oracle's Q8
    GEMV returns the same sum of |terms| from the packed head (its x is r
    rounded to fp32, which moves T by <= 2^-24 T), and a scalar loop over the
    dequantised weights gives it exactly."""
    g = np.random.default_rng(12)
    raw = _tiny_raw(g, hidden=64, ffn=96, vocab=50, layers=2)
    m = toy.ToyModel(raw, eps=1e-6)
    toks = [0, 13, 49]
    T = m.head_abs_terms(toks)
    assert T.shape == (3, 50)
    r = toy.rmsnorm(m.hidden_states(toks)[-1], 1e-6)
    O = oracle.default()
    P = O.pack_q8(raw["head"]["Q"], raw["head"]["S"])
    W = toy.dequant(raw["head"]["Q"], raw["head"]["S"])
    for i in range(3):
        _, t = O.gemv_q8(P, 50, 64, r[i:i + 1])
        np.testing.assert_allclose(T[i], t[0], rtol=2.0 ** -23)
        for v in (0, 17, 49):
            brute = 0.0
            for c in range(64):
                brute += abs(W[v, c] * r[i, c])
            assert abs(T[i, v] - brute) <= 1e-12 * brute
    # it bounds |logit| and is not the logit itself (absolute values inside the sum)
    lg = m.logits(toks)
    assert np.all(np.abs(lg) <= T * (1 + 1e-12)) and np.any(np.abs(lg) < 0.9 * T)


def test_greedy_chain_matches_transition_table_and_systolic_loop():
    """The stack is a Markov chain: greedy decoding follows the table
    next[t] = argmax_v logits(t)[v] (numpy's argmax, first index on ties),
    built from one batched logits call; and the staggered loop's committed
    chain under the same argmax draws is that chain for every stream count."""
    g = np.random.default_rng(13)
    raw = _tiny_raw(g, hidden=32, ffn=64, vocab=40, layers=2)
    m = toy.ToyModel(raw, eps=1e-6)
    nxt = np.argmax(m.logits(list(range(40))), axis=1)
    for first in (0, 7, 39):
        want, t = [], first
        for _ in range(25):
            t = int(nxt[t])
            want.append(t)
        got = toy.greedy_chain(m, first, 25)
        assert got == want
        assert len(got) == 25 and got[0] != first or nxt[first] == first
        for N in (1, 2, 4):
            committed, _, _ = toy.systolic_decode(lambda k, s, i, tok: int(nxt[tok]), first, N, 25)
            assert committed == got


def test_greedy_chain_and_abs_terms_pins_catch_planted_mistakes():
    """Mutants of the two helpers must fail the pins above."""
    g = np.random.default_rng(14)
    raw = _tiny_raw(g, hidden=32, ffn=64, vocab=40, layers=2)
    m = toy.ToyModel(raw, eps=1e-6)
    nxt = np.argmax(m.logits(list(range(40))), axis=1)
    want, t = [], 3
    for _ in range(10):
        t = int(nxt[t])
        want.append(t)
    # chain that includes the first token / stops one short / uses the last index on ties
    assert ([3] + toy.greedy_chain(m, 3, 9)) != want
    assert toy.greedy_chain(m, 3, 9) != want
    # abs outside the sum (|sum| instead of sum |.|) is not the C oracle's T
    r = toy.rmsnorm(m.hidden_states([5])[-1], 1e-6)
    O = oracle.default()
    _, t = O.gemv_q8(O.pack_q8(raw["head"]["Q"], raw["head"]["S"]), 40, 32, r)
    wrong = np.abs(r @ m.head.T)
    assert not np.allclose(wrong[0], t[0], rtol=1e-6)
    assert np.allclose(m.head_abs_terms([5])[0], t[0], rtol=2.0 ** -23)


def test_batch_rows_are_independent():
    g = np.random.default_rng(9)
    m = toy.ToyModel(_tiny_raw(g), eps=1e-6)
    both = m.logits([3, 11])
    np.testing.assert_allclose(both[0], m.logits([3])[0], rtol=1e-13)
    np.testing.assert_allclose(both[1], m.logits([11])[0], rtol=1e-13)


# ----------------------------------------------------------------- sampling

def test_inverse_cdf_boundaries():
    w = np.array([1.0, 2.0, 3.0, 4.0])  # cumulative 1, 3, 6, 10
    cases = {0.0: 0, 0.05: 0, 0.1: 1, 0.2999: 1, 0.3: 2, 0.59: 2, 0.6: 3, 0.9999: 3}
    for u, j in cases.items():
        assert toy.sample_inverse_cdf(w, u)[0] == j, u
    # zero weights are never drawn
    w = np.array([0.0, 1.0, 0.0, 1.0, 0.0])
    assert toy.sample_inverse_cdf(w, 0.0)[0] == 1
    assert toy.sample_inverse_cdf(w, 0.5)[0] == 3
    assert toy.sample_inverse_cdf(w, 0.999999)[0] == 3
    # ambiguity band flags a target on a boundary
    assert toy.sample_inverse_cdf(np.array([1.0, 1.0]), 0.5, band=1e-12)[1]
    assert not toy.sample_inverse_cdf(np.array([1.0, 1.0]), 0.25, band=1e-12)[1]


def test_softmax_t_ratios_and_draw_frequencies():
    l = np.array([0.0, 1.0, -2.0, 0.5])
    t = 0.7
    w = toy.softmax_t(l, t)
    assert w.max() == 1.0 and w[1] == 1.0
    for i in range(4):
        assert math.isclose(w[i] / w[0], math.exp((l[i] - l[0]) / t), rel_tol=1e-14)
    # the draw over a fine grid of u reproduces p exactly up to the grid step
    us = (np.arange(100000) + 0.5) / 100000
    counts = np.bincount([toy.sample_inverse_cdf(w, u)[0] for u in us[::7]], minlength=4)
    np.testing.assert_allclose(counts / counts.sum(), w / w.sum(), atol=2e-3)


# ----------------------------------------------------------------- the loop

def _chain(f, t0, n):
    out = []
    for _ in range(n):
        t0 = f(t0)
        out.append(t0)
    return out


def test_systolic_greedy_accepts_all_and_commits_the_chain():
    g = np.random.default_rng(10)
    table = g.integers(0, 97, size=97)
    f = lambda t: int(table[t])  # any deterministic next-token map
    for N in (1, 2, 3, 4):
        committed, accepts, passes = toy.systolic_decode(lambda k, s, i, t: f(t), 5, N, 40)
        assert accepts == [N] * 40
        assert committed == _chain(f, 5, 40)
        assert len(passes) == (N - 1) + 40 * N  # ramp-up, then one N-stream pass per step
        # stream i runs i positions ahead of the committed chain
        full = [5] + _chain(f, 5, 40 + N)
        for (k, s, i, tok, out) in passes:
            if k >= 1:
                assert tok == full[k - 1 + i] and out == full[k + i]


def test_systolic_greedy_with_wrong_drafter_rerams():
    """A drafter that differs from the verifier: checks fail, the failed streams
    are re-drawn from the last good output, and the committed chain is still the
    verifier's greedy chain."""
    g = np.random.default_rng(11)
    fv = g.integers(0, 13, size=13)
    fd = fv.copy()
    fd[::3] = (fd[::3] + 1) % 13  # the drafter disagrees on a third of the tokens
    draw = lambda k, s, i, t: int(fv[t]) if i == 0 else int(fd[t])
    committed, accepts, passes = toy.systolic_decode(draw, 2, 4, 60)
    assert committed == _chain(lambda t: int(fv[t]), 2, 60)
    assert min(accepts) >= 1 and max(accepts) <= 4 and min(accepts) < 4
    # every re-drawn input comes from the previous output of its left neighbour
    for k in range(1, 61):
        re = [p for p in passes if p[0] == k and p[1] >= 4]
        a = accepts[k - 1]
        assert [p[2] for p in re] == list(range(a, 4))


def _markov(g, V):
    """Context-dependent transition matrix with exact binary-fraction rows."""
    T = g.integers(1, 9, size=(V, V)).astype(np.float64)
    T /= T.sum(axis=1, keepdims=True)
    return T


def _stationary(T):
    w, v = np.linalg.eig(T.T)
    p = np.real(v[:, np.argmin(np.abs(w - 1))])
    return p / p.sum()


def _mc_mean_accept(loop, T, N, steps, seed):
    g = np.random.default_rng(seed)
    U = g.random((steps + 1, 2 * N))
    draw = lambda k, s, i, t: toy.sample_inverse_cdf(T[t], U[k, s])[0]
    _, accepts, _ = loop(draw, 0, N, steps)
    a = np.array(accepts[100:], dtype=np.float64)
    bm = a[: len(a) // 100 * 100].reshape(100, -1).mean(axis=1)  # batch means
    return a.mean(), bm.std(ddof=1) / math.sqrt(len(bm))


def _exact_long_run(T, N):
    pi = _stationary(T)
    Tf = [[Fraction(float(x)) for x in row] for row in T]
    return sum(pi[c] * float(acc.expected_accept_markov_fresh(Tf, c, N)) for c in range(len(T)))


def _mutant(old, new):
    src = inspect.getsource(toy.systolic_decode)
    assert old in src
    ns = dict(toy.__dict__)
    exec(src.replace(old, new), ns)
    return ns["systolic_decode"]


MUTANTS = {
    "no re-draw after a reject": ("for j in range(a, N):", "for j in range(N, N):"),
    "re-draw from the failed stream's output": ("prev = outs[a - 1] if a < N else None", "prev = outs[a] if a < N else None"),
    "stream i keeps its old input": ("nxt = list(outs)", "nxt = [outs[0]] + x[1:]"),
}


def test_systolic_sampling_matches_exact_long_run_acceptance():
    """Under sampling the long-run mean accept count equals
    sum_c pi(c) E[a | c] with E[a | c] the exact enumeration for fresh guesses
    (pi the stationary law of the committed chain); planted loop mistakes move it."""
    g = np.random.default_rng(14)  # a chain whose acceptance separates the mutants by >= 10 s.e.
    T = _markov(g, 3)
    N = 4
    exact = _exact_long_run(T, N)
    mean, se = _mc_mean_accept(toy.systolic_decode, T, N, 20000, 13)
    assert abs(mean - exact) <= 4 * se, (mean, exact, se)
    for name, (old, new) in MUTANTS.items():
        m2, se2 = _mc_mean_accept(_mutant(old, new), T, N, 20000, 13)
        assert abs(m2 - exact) > 6 * se2, name


def test_systolic_iid_matches_formula():
    """Context-free model: E[a] = 1 + P + ... + P^(N-1), P = sum p^2 [README, how acceptance works]."""
    p = np.array([0.5, 0.25, 0.125, 0.125])
    T = np.tile(p, (4, 1))
    for N in (2, 3, 4):
        mean, se = _mc_mean_accept(toy.systolic_decode, T, N, 30000, 14 + N)
        P = Fraction(float((p * p).sum()))
        want = float(acc.expected_accept_formula(P, N))
        assert abs(mean - want) <= 4 * se + 1e-3, (N, mean, want)

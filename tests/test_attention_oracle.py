"""Pins of the fp64 attention oracle (oracle/attention.py) against values the
definition and the mathematics fix, chosen so that a plausible mistake (no
1/sqrt(d), a wrong grouped-head mapping, no max subtraction, a store that
does not replace, the wrong rounding) fails one of them."""

import math

import numpy as np
import pytest
import scipy.special

from oracle import attention as A


def rng(seed):
    return np.random.default_rng(seed)


def test_single_entry_returns_its_value():
    g = rng(1)
    H, Hkv, d = 8, 2, 16
    q = g.standard_normal((H, d))
    K = g.standard_normal((Hkv, 1, d))
    V = g.standard_normal((Hkv, 1, d))
    out, vmag, _ = A.attend(q, K, V, H, Hkv)
    for h in range(H):
        assert np.array_equal(out[h], V[h // 4, 0])
        assert np.array_equal(vmag[h], np.abs(V[h // 4, 0]))


def test_equal_keys_average_the_values():
    g = rng(2)
    H, Hkv, d, n = 4, 4, 8, 11
    q = g.standard_normal((H, d))
    K = np.repeat(g.standard_normal((Hkv, 1, d)), n, axis=1)
    V = g.standard_normal((Hkv, n, d))
    out, _, _ = A.attend(q, K, V, H, Hkv)
    assert np.allclose(out, V.mean(axis=1), rtol=0, atol=1e-14)


def test_two_keys_weight_ratio_has_the_scale():
    """V = unit vectors: out = (p0, p1, 0, ...), p0 / p1 = exp((q.k0 - q.k1) / sqrt(d))."""
    d = 9
    q = np.zeros((1, d))
    q[0, :3] = [1.0, -2.0, 0.5]
    K = np.zeros((1, 2, d))
    K[0, 0, :3] = [2.0, 0.0, 1.0]
    K[0, 1, :3] = [0.0, 1.0, 0.0]
    V = np.zeros((1, 2, d))
    V[0, 0, 0] = 1.0
    V[0, 1, 1] = 1.0
    out, _, _ = A.attend(q, K, V, 1, 1)
    s0, s1 = (2.0 + 0.5) / 3.0, -2.0 / 3.0  # sqrt(9) = 3
    p0 = 1.0 / (1.0 + math.exp(s1 - s0))
    assert out[0, 0] == pytest.approx(p0, rel=1e-15) and out[0, 1] == pytest.approx(1 - p0, rel=1e-14)
    assert out[0, 0] / out[0, 1] == pytest.approx(math.exp(s0 - s1), rel=1e-14)
    assert not out[0, 2:].any()


def test_grouped_heads_read_their_group():
    """kv head g holds values g + 1 everywhere, so head h must return h // group + 1."""
    g = rng(3)
    H, Hkv, d, n = 8, 2, 4, 5
    q = g.standard_normal((H, d))
    K = g.standard_normal((Hkv, n, d))
    V = np.stack([np.full((n, d), 1.0), np.full((n, d), 2.0)])
    out, _, _ = A.attend(q, K, V, H, Hkv)
    want = np.array([1.0] * 4 + [2.0] * 4)
    assert np.allclose(out, want[:, None], rtol=0, atol=1e-15)


def test_position_permutation_invariance():
    g = rng(4)
    H, Hkv, d, n = 6, 3, 8, 13
    q = g.standard_normal((H, d))
    K = g.standard_normal((Hkv, n, d))
    V = g.standard_normal((Hkv, n, d))
    perm = g.permutation(n)
    a, _, _ = A.attend(q, K, V, H, Hkv)
    b, _, _ = A.attend(q, K[:, perm], V[:, perm], H, Hkv)
    assert np.allclose(a, b, rtol=0, atol=1e-14)


def test_dominant_key_and_large_scores_stay_finite():
    g = rng(5)
    d, n = 16, 9
    q = g.standard_normal((1, d))
    K = g.standard_normal((1, n, d))
    K[0, 4] = 1000.0 * q[0] / (q[0] @ q[0]) * math.sqrt(d)  # s_4 = 1000: exp(1000) overflows fp64
    V = g.standard_normal((1, n, d))
    out, _, _ = A.attend(q, K, V, 1, 1)
    assert np.all(np.isfinite(out))
    assert np.allclose(out[0], V[0, 4], rtol=0, atol=1e-12)


def test_brute_force_against_scipy_softmax():
    g = rng(6)
    H, Hkv, d, n = 4, 2, 8, 7
    q = g.standard_normal((H, d))
    K = g.standard_normal((Hkv, n, d))
    V = g.standard_normal((Hkv, n, d))
    out, vmag, smax = A.attend(q, K, V, H, Hkv)
    for h in range(H):
        kv = h // 2
        p = scipy.special.softmax(np.einsum("d,nd->n", q[h], K[kv]) / math.sqrt(d))
        assert np.allclose(out[h], np.einsum("n,nd->d", p, V[kv]), rtol=1e-13, atol=1e-14)
        assert np.allclose(vmag[h], np.einsum("n,nd->d", p, np.abs(V[kv])), rtol=1e-13, atol=1e-14)
        assert smax[h] == pytest.approx(max(np.abs(K[kv, j]) @ np.abs(q[h]) for j in range(n)), rel=1e-15)


def test_store_rounds_to_nearest_even_binary16():
    x = np.array([1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 65520.0, 2.0 ** -25, 3 * 2.0 ** -26, -2.5], np.float32)
    got = A.f16_round(x).astype(np.float64)
    want = np.array([1.0, 1 + 2.0 ** -9, np.inf, 0.0, 2.0 ** -24, -2.5])
    assert np.array_equal(got, want)


def test_step_replaces_the_entry_at_pos():
    """A reject's redraw runs at the same position: its store must replace the
    stale entry, giving what a cache that never held it gives."""
    g = rng(7)
    H, Hkv, d, L = 4, 2, 8, 16
    ks = g.standard_normal((6, Hkv, d)).astype(np.float32)
    vs = g.standard_normal((6, Hkv, d)).astype(np.float32)
    q = g.standard_normal((H, d)).astype(np.float32)
    c1 = A.Cache(Hkv, L, d)
    c2 = A.Cache(Hkv, L, d)
    for p in range(3):
        c1.step(q, ks[p], vs[p], p, H)
        c2.step(q, ks[p], vs[p], p, H)
    c1.step(q, ks[3], vs[3], 3, H)           # stale speculative entry
    redo, _, _ = c1.step(q, ks[4], vs[4], 3, H)
    fresh, _, _ = c2.step(q, ks[4], vs[4], 3, H)
    assert np.array_equal(redo, fresh)
    assert np.array_equal(c1.K[:, :4], c2.K[:, :4]) and np.array_equal(c1.V[:, :4], c2.V[:, :4])


PINS = [test_single_entry_returns_its_value, test_equal_keys_average_the_values,
        test_two_keys_weight_ratio_has_the_scale, test_grouped_heads_read_their_group,
        test_position_permutation_invariance, test_dominant_key_and_large_scores_stay_finite,
        test_brute_force_against_scipy_softmax, test_store_rounds_to_nearest_even_binary16,
        test_step_replaces_the_entry_at_pos]


def _mutant_attend(kind):
    def attend(q, K, V, n_heads, n_kv_heads):
        q = np.asarray(q, np.float64)
        K = np.asarray(K, np.float64)
        V = np.asarray(V, np.float64)
        H, d = q.shape
        group = n_heads // n_kv_heads
        out, vmag, smax = np.empty((H, d)), np.empty((H, d)), np.empty(H)
        for h in range(H):
            g = h % n_kv_heads if kind == "group_mod" else h // group
            s = K[g] @ q[h] / (1.0 if kind == "no_scale" else math.sqrt(d))
            with np.errstate(over="ignore", invalid="ignore"):
                e = np.exp(s) if kind == "no_max" else np.exp(s - s.max())
            p = e / e.sum()
            if kind == "first_only":
                p = np.zeros_like(p)
                p[0] = 1.0
            out[h] = p @ V[g]
            vmag[h] = p @ np.abs(V[g])
            smax[h] = (np.abs(K[g]) @ np.abs(q[h])).max()
        return out, vmag, smax
    return attend


@pytest.mark.parametrize("kind", ["no_scale", "group_mod", "no_max", "first_only", "bad_round", "no_replace"])
def test_pins_catch_planted_mistakes(monkeypatch, kind):
    if kind == "bad_round":
        monkeypatch.setattr(A, "f16_round", lambda x: np.asarray(x, np.float32).astype(np.float64).round(2))
    elif kind == "no_replace":
        orig = A.Cache.step

        def step(self, q, k_new, v_new, pos, n_heads):
            if np.any(self.K[:, pos]):  # keep the first entry written at a position
                return A.attend(q, self.K[:, :pos + 1], self.V[:, :pos + 1], n_heads, self.K.shape[0])
            return orig(self, q, k_new, v_new, pos, n_heads)
        monkeypatch.setattr(A.Cache, "step", step)
    else:
        monkeypatch.setattr(A, "attend", _mutant_attend(kind))
    failed = 0
    for pin in PINS:
        try:
            pin()
        except (AssertionError, FloatingPointError, ValueError):
            failed += 1
    assert failed >= 1, f"no pin caught the planted mistake {kind}"

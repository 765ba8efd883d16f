"""GPU parity of the twin-KV decode attention (pti_attn_decode) against the
fp64 oracle (oracle/attention.py).

Bars:
  * the stored entry at pos: bit-exact binary16 of the fp32 key and value;
    every other cache entry unchanged (bitwise);
  * outputs: per output (head h, dimension i), with u = 2^-24,
      |out - exact| <= (4 eps_s + (2 (136 + n_chunks) + 16) u) sum_j p_j |v_j,i|
                       + 2^-40 sum_j |v_j,i|,
      eps_s = ((d + 8) u smax + 2^-39 max_i |q_i| max_j sum_i |k_j,i|) / sqrt(d),
      smax  = max_j sum_i |q_i k_j,i|.
    The kernel scores on the matrix cores with q split into two binary16
    parts (q 2^sh = high + low, sh per head so that max |q 2^sh| lies in
    [2^14, 2^15)): the split drops at most 2^-22 |q_i| + 2^-25 2^-sh per
    element, the 128-term fp32 accumulation of exact products costs
    d u, the sum of the two parts, the scaling by 2^-sh and the product with
    the fp32 1/sqrt(d) one rounding each.  The weights (in units of 2^-15)
    are split the same way, so a chunk's weighted V carries at most 128 u of
    accumulation (32 keys per wave, then the four waves' sum: 35 u), 4 u of
    split and one rounding for the two parts' sum, plus
    2^-40 |v_j| per key from the low part's binary16 spacing.  The score
    error passes through exp into the weights (4 eps_s); the factor 2 covers
    the numerator and the exp-sum of the normalisation, n_chunks the chunk
    combine and 16 the exp and division roundings;
  * a stream's outputs do not depend on the other streams (bitwise), and a
    redo at the same position (the reject rule) gives what a cache that never
    held the stale entry gives (bitwise).
"""

import math
import sys

import numpy as np
import pytest

from oracle import attention as A

pytestmark = pytest.mark.gpu
U = 2.0 ** -24
CHUNK = 128


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


def tol_of(q, K, V, H, Hkv, n):
    """Per-output bound: the oracle's magnitudes plus the split terms."""
    d = q.shape[1]
    out, vmag, smax = A.attend(q, K, V, H, Hkv)
    kv = np.arange(H) // (H // Hkv)
    q64 = np.asarray(q, np.float64)
    k1 = np.abs(np.asarray(K, np.float64)).sum(axis=2).max(axis=1)[kv]  # max_j sum_i |k_j,i| per head
    vabs = np.abs(np.asarray(V, np.float64)).sum(axis=1)[kv]            # sum_j |v_j,i| per head
    eps_s = ((d + 8) * U * smax + 2.0 ** -39 * np.abs(q64).max(axis=1) * k1) / math.sqrt(d)
    n_chunks = (n + CHUNK - 1) // CHUNK
    tol = (4 * eps_s[:, None] + (2 * (136 + n_chunks) + 16) * U) * vmag + 2.0 ** -40 * vabs
    return out, tol


class Case:
    """S streams with random binary16 histories of pos[s] entries."""

    def __init__(self, env, S, H, Hkv, d, L, pos, seed):
        torch, pti, dev = env
        self.g = np.random.default_rng(seed)
        self.S, self.H, self.Hkv, self.d, self.L = S, H, Hkv, d, L
        self.pos = list(pos)
        self.oc = [A.Cache(Hkv, L, d) for _ in range(S)]
        for s in range(S):
            self.oc[s].K[:, :pos[s]] = A.f16_round(self.g.standard_normal((Hkv, pos[s], d)))
            self.oc[s].V[:, :pos[s]] = A.f16_round(self.g.standard_normal((Hkv, pos[s], d)))
        self.kc = [torch.from_numpy(c.K.copy()).to(dev) for c in self.oc]
        self.vc = [torch.from_numpy(c.V.copy()).to(dev) for c in self.oc]
        self.work = pti.attn_workspace(S, H, Hkv, d, L, dev)

    def inputs(self):
        g = self.g
        q = g.standard_normal((self.S, self.H, self.d)).astype(np.float32)
        kn = g.standard_normal((self.S, self.Hkv, self.d)).astype(np.float32)
        vn = g.standard_normal((self.S, self.Hkv, self.d)).astype(np.float32)
        return q, kn, vn

    def run(self, env, q, kn, vn, pos=None):
        torch, pti, dev = env
        pos = self.pos if pos is None else pos
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        out = pti.attn_decode(t(q), t(kn), t(vn), self.kc, self.vc,
                              torch.tensor(pos, dtype=torch.int32, device=dev), self.work)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def check(self, env, q, kn, vn, got, what=""):
        for s in range(self.S):
            p = self.pos[s]
            self.oc[s].K[:, p] = A.f16_round(kn[s])
            self.oc[s].V[:, p] = A.f16_round(vn[s])
            want, tol = tol_of(q[s], self.oc[s].K[:, :p + 1], self.oc[s].V[:, :p + 1], self.H, self.Hkv, p + 1)
            err = np.abs(got[s].astype(np.float64) - want)
            assert np.all(err <= tol), f"{what} stream {s}: worst err/tol {np.max(err / tol):.3f}"
            gk = self.kc[s].cpu().numpy()
            gv = self.vc[s].cpu().numpy()
            assert np.array_equal(gk.view(np.uint16), self.oc[s].K.view(np.uint16)), f"{what} K cache stream {s}"
            assert np.array_equal(gv.view(np.uint16), self.oc[s].V.view(np.uint16)), f"{what} V cache stream {s}"


SHAPES = [  # S, H, Hkv, d, L, positions
    (1, 1, 1, 64, 8, [0]),
    (1, 4, 4, 64, 300, [1]),
    (2, 8, 2, 128, 1024, [255, 256]),
    (2, 40, 8, 128, 4096, [257, 1000]),
    (4, 5, 1, 128, 2048, [0, 511, 1023, 2047]),
    (3, 6, 3, 64, 777, [776, 3, 512]),
    (2, 16, 2, 128, 8192, [4095, 8191]),
]


@pytest.mark.parametrize("S,H,Hkv,d,L,pos", SHAPES, ids=[f"S{s[0]}H{s[1]}kv{s[2]}d{s[3]}L{s[4]}" for s in SHAPES])
def test_attn_vs_oracle(env, S, H, Hkv, d, L, pos):
    _note(f"attn S={S} H={H} Hkv={Hkv} d={d} L={L} pos={pos}")
    c = Case(env, S, H, Hkv, d, L, pos, seed=S * 1000 + H * 10 + d + L)
    q, kn, vn = c.inputs()
    got = c.run(env, q, kn, vn)
    c.check(env, q, kn, vn, got)


@pytest.mark.parametrize("qscale", [1e-20, 1e20], ids=["q_tiny", "q_huge"])
def test_attn_query_magnitudes(env, qscale):
    """The per-head power-of-two scaling of q before its split into binary16
    parts: far outside the binary16 range either way."""
    _note(f"attn qscale={qscale}")
    c = Case(env, 2, 8, 2, 128, 512, [300, 301], seed=61)
    q, kn, vn = c.inputs()
    q = (q * np.float32(qscale)).astype(np.float32)
    got = c.run(env, q, kn, vn)
    c.check(env, q, kn, vn, got, what=f"qscale {qscale}")


def test_attn_subnormal_cache_entries(env):
    """binary16 subnormals in the caches: every K entry, and V in half of the
    dimensions, with q large enough that the scores spread over about 0.1:
    flushed subnormals would flatten the weights and zero those outputs."""
    _note("attn subnormal entries")
    torch, pti, dev = env
    for d, G in ((128, 8), (64, 5)):
        c = Case(env, 1, G, 1, d, 256, [200], seed=71 + d)
        g = np.random.default_rng(72 + d)
        for KV, t, dims in ((c.oc[0].K, c.kc[0], d), (c.oc[0].V, c.vc[0], d // 2)):
            ints = g.integers(1, 1024, KV[..., :dims].shape) * g.choice([-1, 1], KV[..., :dims].shape)
            KV[..., :dims] = (ints * 2.0 ** -24).astype(np.float16)
            t.copy_(torch.from_numpy(KV.copy()))
        q, kn, vn = c.inputs()
        q = (q * np.float32(2.0 ** 12)).astype(np.float32)
        kn = (kn * np.float32(2.0 ** -17)).astype(np.float32)  # the new key rounds to subnormals too
        got = c.run(env, q, kn, vn)
        c.check(env, q, kn, vn, got, what=f"subnormals d={d} G={G}")


def test_attn_bench_shape_all_heads(env):
    """The benchmark's shape and launch: two streams, 40 query heads over 8
    kv heads of 128, 32K positions (256 chunks); every head of both streams
    against the oracle."""
    _note("attn bench shape 2x40/8x128, 32768 positions")
    torch, pti, dev = env
    S, H, Hkv, d, L = 2, 40, 8, 128, 32768
    g = np.random.default_rng(81)
    pos = [L - 2, L - 1]
    K = [A.f16_round(g.standard_normal((Hkv, L, d))) for _ in range(S)]
    V = [A.f16_round(g.standard_normal((Hkv, L, d))) for _ in range(S)]
    kc = [torch.from_numpy(k).to(dev) for k in K]
    vc = [torch.from_numpy(v).to(dev) for v in V]
    q = g.standard_normal((S, H, d)).astype(np.float32)
    kn = g.standard_normal((S, Hkv, d)).astype(np.float32)
    vn = g.standard_normal((S, Hkv, d)).astype(np.float32)
    work = pti.attn_workspace(S, H, Hkv, d, L, dev)
    t = lambda a: torch.from_numpy(a).to(dev)
    out = pti.attn_decode(t(q), t(kn), t(vn), kc, vc, torch.tensor(pos, dtype=torch.int32, device=dev), work)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for s in range(S):
        p = pos[s]
        K[s][:, p] = A.f16_round(kn[s])
        V[s][:, p] = A.f16_round(vn[s])
        want, tol = tol_of(q[s], K[s][:, :p + 1], V[s][:, :p + 1], H, Hkv, p + 1)
        err = np.abs(got[s].astype(np.float64) - want)
        worst = np.unravel_index(np.argmax(err / tol), err.shape)
        assert np.all(err <= tol), f"stream {s} head {worst[0]} dim {worst[1]}: err/tol {np.max(err / tol):.3f}"


def test_attn_streams_independent(env):
    torch, pti, dev = env
    c2 = Case(env, 2, 8, 2, 128, 2048, [700, 1500], seed=11)
    q, kn, vn = c2.inputs()
    both = c2.run(env, q, kn, vn)
    for s in range(2):
        c1 = Case(env, 1, 8, 2, 128, 2048, [c2.pos[s]], seed=11)
        c1.kc[0].copy_(c2.kc[s])
        c1.vc[0].copy_(c2.vc[s])
        one = c1.run(env, q[s:s + 1], kn[s:s + 1], vn[s:s + 1])
        assert np.array_equal(one[0].view(np.uint32), both[s].view(np.uint32))


def test_attn_redo_at_same_position_replaces(env):
    """The reject rule: B's pass at position p ran on a wrong token; the redraw
    runs at p again and must give what a cache that never held it gives."""
    torch, pti, dev = env
    a = Case(env, 1, 8, 2, 128, 1024, [300], seed=21)
    b = Case(env, 1, 8, 2, 128, 1024, [300], seed=21)
    q1, k1, v1 = a.inputs()
    a.run(env, q1, k1, v1)                   # stale speculative entry
    q2, k2, v2 = a.inputs()                  # the redraw's inputs
    redo = a.run(env, q2, k2, v2)
    fresh = b.run(env, q2, k2, v2)
    assert np.array_equal(redo.view(np.uint32), fresh.view(np.uint32))
    assert torch.equal(a.kc[0], b.kc[0]) and torch.equal(a.vc[0], b.vc[0])


def test_attn_twin_sequence(env):
    """Twins A (stream 0, confirmed token) and B (stream 1, guess one position
    ahead) over several steps with accepts and rejects: B's position moves on
    after an accept and its redraw reuses the position after a reject; every
    step checked against the oracle caches."""
    c = Case(env, 2, 8, 2, 64, 512, [100, 101], seed=31)
    for accepted in (True, True, False, True, False, False, True):
        q, kn, vn = c.inputs()
        got = c.run(env, q, kn, vn)
        c.check(env, q, kn, vn, got, what=f"step accepted={accepted}")
        if accepted:
            c.pos = [c.pos[0] + 1, c.pos[1] + 1]
        else:
            # A moves on; B redraws at its position (single-stream pass), then moves on
            c.pos = [c.pos[0] + 1, c.pos[1]]
            qb, kb, vb = c.inputs()
            sub = Case.__new__(Case)
            sub.__dict__.update(c.__dict__)
            sub.S, sub.pos, sub.kc, sub.vc, sub.oc = 1, [c.pos[1]], c.kc[1:], c.vc[1:], c.oc[1:]
            import packed_twin_int8_amd as pti
            sub.work = pti.attn_workspace(1, 8, 2, 64, 512, c.kc[0].device)
            got1 = sub.run(env, qb[:1], kb[:1], vb[:1])
            sub.check(env, qb[:1], kb[:1], vb[:1], got1, what="redraw")
            c.pos = [c.pos[0], c.pos[1] + 1]


def test_attn_position_out_of_range_gives_nan_and_keeps_caches(env):
    torch, pti, dev = env
    c = Case(env, 2, 4, 2, 64, 256, [10, 20], seed=41)
    q, kn, vn = c.inputs()
    k0 = [t.clone() for t in c.kc]
    got = c.run(env, q, kn, vn, pos=[256, -1])
    assert np.all(np.isnan(got))
    assert all(torch.equal(a, b) for a, b in zip(k0, c.kc))


def test_attn_graph_replay_reads_positions_from_device(env):
    torch, pti, dev = env
    c = Case(env, 2, 8, 2, 128, 1024, [50, 51], seed=51)
    q, kn, vn = c.inputs()
    tq, tk, tv = (torch.from_numpy(a).to(dev) for a in (q, kn, vn))
    pos = torch.tensor(c.pos, dtype=torch.int32, device=dev)
    out = torch.empty_like(tq)
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        pti.attn_decode(tq, tk, tv, c.kc, c.vc, pos, c.work, out=out)
    for step in range(3):
        new_pos = [50 + 7 * step, 51 + 9 * step]
        pos.copy_(torch.tensor(new_pos, dtype=torch.int32))
        g.replay()
        torch.cuda.synchronize()
        graph_out = out.cpu().numpy().copy()
        c.pos = new_pos
        eager = c.run(env, q, kn, vn)
        assert np.array_equal(graph_out.view(np.uint32), eager.view(np.uint32)), step

"""fp64 toy decoder stack and the staggered (systolic) twin-decode loop.

TEST INFRASTRUCTURE (part of the oracle): only the tests, the smoke check and
the benchmark's CPU baseline may use it.  Plain numpy float64; shares nothing
with the HIP library.

Pages cited by title and section:
  [Digest] "Packed Twin Inference：无需草稿模型的推测解码新方案，实现2倍吞吐量提升",
           section "技术实现架构" (implementation architecture): one weight
           load serves the confirmed stream and the speculative stream, the
           outputs are compared to decide acceptance, an accept extends the
           speculative stream's state and a reject resets it.
  [README] "打包双子推理（PTI）", section "接受机制如何工作" (how acceptance
           works): stream i runs the same model i positions ahead on a guess
           produced one step earlier; under greedy decoding the guess always
           equals the verifier's token; under sampling a check passes with the
           collision probability sum_x p(x)^2.

The model.  The pages run a real LLM, which is not available here; the
stand-in is a random-weight MLP-residual stack with the same step structure
(every weight matrix read once per step, shared by all streams):

    h_0   = dequant(embedding row of the token)
    r_l   = rmsnorm(h_l)                      (no gain, eps inside the root)
    h_l+1 = h_l + down_l (silu(gate_l r_l) * up_l r_l)
    logits = head rmsnorm(h_L)

with rmsnorm(x) = x / sqrt(mean(x^2) + eps) and silu(v) = v / (1 + exp(-v)).
Every matrix is int8 with one f16 scale per 32 weights of a row; a weight's
value is scale * q.  Without attention the next-token distribution depends on
the current token only, so the stack is a Markov chain over the vocabulary.

Sampling at temperature t > 0: p = softmax(logits / t) (max subtracted), and
the draw for a uniform u in [0, 1) is the smallest index j whose cumulative
sum sum_{k<=j} exp((l_k - max)/t) exceeds u * Z (Z the full sum).  The
uniforms are inputs: the caller supplies them, one per pass slot.
"""

from __future__ import annotations

from typing import Callable, Sequence

import numpy as np

BLOCK = 32


def f16_to_f64(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns (uint16) -> float64 (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def dequant(Q: np.ndarray, S: np.ndarray) -> np.ndarray:
    """w[r][c] = scale(r, c/32) * q[r][c], float64 (exact)."""
    Q = np.asarray(Q)
    assert Q.shape[1] == S.shape[1] * BLOCK
    return Q.astype(np.float64) * np.repeat(f16_to_f64(S), BLOCK, axis=1)


def rmsnorm(x: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps), over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def silu(v: np.ndarray) -> np.ndarray:
    """v * sigmoid(v) = v / (1 + exp(-v))."""
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


class ToyModel:
    """The stack above, dequantised to float64 once.

    ``raw`` holds int8/f16 arrays as drawn by the input generator:
    emb, head: dict(Q, S); layers: list of dict(gate, up, down) of dict(Q, S).
    A twin pair is two instances; the loop's ``draw`` routes stream 0 to the
    verifier twin and the other streams to the drafting twin."""

    def __init__(self, raw: dict, eps: float = 1e-6):
        self.eps = float(eps)
        self.emb = dequant(raw["emb"]["Q"], raw["emb"]["S"])
        self.head = dequant(raw["head"]["Q"], raw["head"]["S"])
        self.layers = [{k: dequant(L[k]["Q"], L[k]["S"]) for k in ("gate", "up", "down")} for L in raw["layers"]]
        self.vocab, self.hidden = self.emb.shape

    def hidden_states(self, tokens: Sequence[int]) -> list:
        """[h_0, h_1, ..., h_L] for a batch of tokens, each [B][hidden]."""
        h = self.emb[np.asarray(tokens, dtype=np.int64)]
        hs = [h]
        for L in self.layers:
            r = rmsnorm(h, self.eps)
            m = silu(r @ L["gate"].T) * (r @ L["up"].T)
            h = h + m @ L["down"].T
            hs.append(h)
        return hs

    def logits(self, tokens: Sequence[int]) -> np.ndarray:
        """[B][vocab] float64."""
        h = self.hidden_states(tokens)[-1]
        return rmsnorm(h, self.eps) @ self.head.T

    def head_abs_terms(self, tokens: Sequence[int]) -> np.ndarray:
        """sum_c |head[v][c] * r[c]| per logit, the scale of a logit's rounding error."""
        h = self.hidden_states(tokens)[-1]
        return np.abs(rmsnorm(h, self.eps)) @ np.abs(self.head).T


def argmax_first(v: np.ndarray) -> int:
    """Index of the largest value; the lowest index wins a tie."""
    v = np.asarray(v, dtype=np.float64)
    best = 0
    for j in range(1, v.shape[0]):
        if v[j] > v[best]:
            best = j
    return best


def softmax_t(logits: np.ndarray, temperature: float) -> np.ndarray:
    """Unnormalised weights exp((l - max) / t) in float64 (the draw compares
    cumulative sums of these against u * their total)."""
    l = np.asarray(logits, dtype=np.float64)
    return np.exp((l - l.max()) / float(temperature))


def sample_inverse_cdf(weights: np.ndarray, u: float, band: float = 0.0):
    """Smallest j with sum_{k<=j} w_k > u * Z, summing in index order.  If
    rounding leaves u * Z at or above the full sum, the last index with w > 0.

    Returns (j, ambiguous): ``ambiguous`` is True when u * Z lies within
    band * Z of the cumulative sum at j or j - 1, i.e. when a sum taken in
    another order could land on the neighbouring index."""
    w = np.asarray(weights, dtype=np.float64)
    Z = 0.0
    for x in w:
        Z += x
    target = u * Z
    run = 0.0
    prev = 0.0
    for j, x in enumerate(w):
        prev = run
        run += x
        if run > target:
            amb = abs(run - target) <= band * Z or (j > 0 and abs(target - prev) <= band * Z)
            return j, amb
    last = int(np.nonzero(w > 0)[0][-1])
    return last, True


def accept_count(inputs: Sequence[int], outputs: Sequence[int]) -> int:
    """1 + the leading run of i >= 1 with inputs[i] == outputs[i-1]."""
    a = 1
    for i in range(1, len(inputs)):
        if inputs[i] != outputs[i - 1]:
            break
        a += 1
    return a


def systolic_decode(draw: Callable[[int, int, int, int], int], first: int, n_streams: int, n_steps: int):
    """The staggered N-stream loop, driven by ``draw(step, slot, stream, token)``
    which returns the model's next token for ``token`` run as ``stream`` in the
    pass slot ``slot`` of ``step`` (slot indexes the uniform it consumes).

    Stream 0 runs on the last committed token; stream i >= 1 runs on its own
    output of the previous step, a guess for the token i positions ahead.
      * Ramp-up (step 0): stream i's first input is drawn by single-stream
        passes, x_i = draw(x_{i-1}), slots N .. 2N-2.
      * Step k >= 1: one N-stream pass (slots 0 .. N-1) gives o_0 .. o_{N-1};
        a = 1 + leading run of x_i == o_{i-1}; o_0 is committed; stream i's
        next input is o_i.
      * If a < N, check a failed: streams a .. N-1 ran on a stale guess, so
        their next inputs are re-drawn by single-stream passes starting from
        o_{a-1} (slots N .. 2N-1-a).
    Returns (committed[n_steps], accepts[n_steps], passes) where passes is a
    list of (step, slot, stream, input, output)."""
    N = n_streams
    passes = []

    def run(step, slot, stream, tok):
        out = draw(step, slot, stream, tok)
        passes.append((step, slot, stream, tok, out))
        return out

    x = [first]
    for i in range(1, N):
        x.append(run(0, N + i - 1, i, x[i - 1]))
    committed, accepts = [], []
    for k in range(1, n_steps + 1):
        outs = [run(k, s, s, x[s]) for s in range(N)]
        a = accept_count(x, outs)
        committed.append(outs[0])
        accepts.append(a)
        nxt = list(outs)
        prev = outs[a - 1] if a < N else None
        for j in range(a, N):
            prev = run(k, N + j - a, j, prev)
            nxt[j] = prev
        x = nxt
    return committed, accepts, passes


def greedy_chain(model: ToyModel, first: int, n: int) -> list:
    """Single-stream greedy decode: n tokens after ``first``."""
    out, t = [], first
    for _ in range(n):
        t = argmax_first(model.logits([t])[0])
        out.append(t)
    return out

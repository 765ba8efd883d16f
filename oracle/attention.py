"""fp64 attention decode step over per-stream KV caches.

TEST INFRASTRUCTURE (part of the oracle): only the tests, the smoke check and
the benchmark's CPU baseline may use it.  Plain numpy float64; shares nothing
with the HIP library.

Pages cited by title and section:
  [Digest] "Packed Twin Inference：无需草稿模型的推测解码新方案，实现2倍吞吐量提升",
           section "技术实现架构" (implementation architecture): twins A and B
           each keep their own KV cache; one pass serves the confirmed stream
           (A) and the speculative stream (B); an accept extends B's cache and
           a reject resets B's state.  The kernel list there includes
           attention and softmax.
  [Notes]  the LLM-inference page, section "从朴素推理到 KV cache" (from naive
           inference to the KV cache): the keys and values of the prefix do
           not change from step to step, so a decode step appends the new
           token's key and value and attends over the cache.

What one step computes, per stream (the streams' caches are independent):
  1. store: the new key and value (fp32 projections, [n_kv_heads][d]) are
     rounded to IEEE binary16 (round to nearest, ties to even) and written
     at position pos of the stream's cache, replacing whatever was there;
  2. attend: for query head h (of n_heads), with kv head g = h // (n_heads /
     n_kv_heads) (grouped heads share a kv head),
         s_j   = (q_h . k_{g,j}) / sqrt(d),           j = 0 .. pos
         p_j   = exp(s_j - max_j s_j) / sum_j exp(s_j - max_j s_j)
         out_h = sum_j p_j v_{g,j}
     in fp64 from the stored binary16 values and the fp32 query.

Twin positions (the pages' state rule, read plainly): a stream's token is
written at the stream's position; on an accept twin B's entry at its position
is correct and B moves on; on a reject B's entry there was computed from a
wrong token, and B's next pass (the redraw) runs at the same position, so the
store in step 1 replaces it.  Nothing else about the cache changes.
"""

from __future__ import annotations

import math

import numpy as np


def f16_round(x) -> np.ndarray:
    """fp32 values rounded to binary16 (RNE), as stored in the cache (values
    beyond the binary16 range become infinities)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float32).astype(np.float16)


def attend(q, K, V, n_heads: int, n_kv_heads: int):
    """q: [H][d] (float); K, V: [Hkv][n][d] (float, n >= 1).
    Returns (out [H][d], vmag [H][d], smax [H]) in float64 where
    vmag[h][i] = sum_j p_j |v_{g,j,i}| and smax[h] = max_j sum_i |q_h,i k_g,j,i|
    (the magnitudes that bound the rounding of a float32 computation)."""
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    H, d = q.shape
    assert H == n_heads and n_heads % n_kv_heads == 0 and K.shape[0] == n_kv_heads and K.shape[2] == d
    group = n_heads // n_kv_heads
    out = np.empty((H, d))
    vmag = np.empty((H, d))
    smax = np.empty(H)
    for h in range(H):
        g = h // group
        s = K[g] @ q[h] / math.sqrt(d)
        e = np.exp(s - s.max())
        p = e / e.sum()
        out[h] = p @ V[g]
        vmag[h] = p @ np.abs(V[g])
        smax[h] = (np.abs(K[g]) @ np.abs(q[h])).max()
    return out, vmag, smax


class Cache:
    """One stream's KV cache: binary16 [n_kv_heads][max_len][d] for K and V."""

    def __init__(self, n_kv_heads: int, max_len: int, d: int):
        self.K = np.zeros((n_kv_heads, max_len, d), np.float16)
        self.V = np.zeros((n_kv_heads, max_len, d), np.float16)

    def step(self, q, k_new, v_new, pos: int, n_heads: int):
        """Store the new entry at pos, then attend over positions 0 .. pos."""
        self.K[:, pos] = f16_round(k_new)
        self.V[:, pos] = f16_round(v_new)
        return attend(q, self.K[:, :pos + 1], self.V[:, :pos + 1], n_heads, self.K.shape[0])

"""First-order rounding-error bounds for the toy decoder stack (test helper).

The library's kernels each carry a per-operation bound:
  * packed GEMV: |y - y_exact| <= GAMMA * sum_c |w_c x_c| (GAMMA = 1e-5, the
    GEMV contract);
  * rmsnorm and silu_mul: within 1 fp32 ulp of the exact value on their fp32
    inputs (fp64 inside, one final rounding), bounded here by 2^-23 |y|;
  * add: one fp32 rounding, 2^-24 |y|.
Propagating an input error bound e through an operation adds its first-order
sensitivity |d op / d input| e (for the norm, d r_i = dh_i / s - h_i
(h . dh) / (n s^3)); second-order terms are below 1e-4 of the first-order ones
at these error sizes and are covered by a 2% margin applied by the callers.

All arithmetic is float64 on the oracle's dequantised weights.
"""

from __future__ import annotations

import numpy as np

from oracle import toy

GAMMA = 1e-5
ULP = 2.0 ** -23  # one fp32 ulp, relative, upper bound
HALF_ULP = 2.0 ** -24
MARGIN = 1.02


def rmsnorm_prop(h, e, eps):
    n = h.shape[-1]
    s = np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)
    r = h / s
    dot = np.sum(np.abs(h) * e, axis=-1, keepdims=True)
    er = e / s + np.abs(h) * dot / (n * s ** 3)
    return r, er + ULP * np.abs(r)


def gemv_prop(W, Wabs, x, ex):
    """y = x W^T for a batch x [B, cols]; bound GAMMA * sum |w x| + |W| ex."""
    y = x @ W.T
    return y, GAMMA * (np.abs(x) @ Wabs.T) + ex @ Wabs.T


class Bounds:
    """Oracle model plus |W| matrices for error propagation."""

    def __init__(self, model: toy.ToyModel):
        self.m = model
        self.abs_layers = [{k: np.abs(L[k]) for k in L} for L in model.layers]
        self.abs_head = np.abs(model.head)

    def layer(self, l, h, e):
        """One layer from h (error bound e) -> (h', e')."""
        L, A = self.m.layers[l], self.abs_layers[l]
        r, er = rmsnorm_prop(h, e, self.m.eps)
        g, eg = gemv_prop(L["gate"], A["gate"], r, er)
        u, eu = gemv_prop(L["up"], A["up"], r, er)
        sg = 1.0 / (1.0 + np.exp(-g))
        s = g * sg
        ds = sg * (1.0 + g * (1.0 - sg))
        m = s * u
        em = np.abs(ds * u) * eg + np.abs(s) * eu + ULP * np.abs(m)
        d, ed = gemv_prop(L["down"], A["down"], m, em)
        h2 = h + d
        return h2, e + ed + HALF_ULP * np.abs(h2)

    def head(self, h, e):
        r, er = rmsnorm_prop(h, e, self.m.eps)
        return gemv_prop(self.m.head, self.abs_head, r, er)

    def forward(self, tokens):
        """Oracle logits and their error bound for the whole GPU forward pass
        (embedding rows are exact, so the chain starts with e = 0)."""
        h = self.m.emb[np.asarray(tokens, dtype=np.int64)]
        e = np.zeros_like(h)
        for l in range(len(self.m.layers)):
            h, e = self.layer(l, h, e)
        y, ey = self.head(h, e)
        return y, MARGIN * ey

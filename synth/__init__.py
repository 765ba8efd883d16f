"""Seeded synthetic inputs for the packed-twin decode path.

This module only draws random numbers.  It holds none of the method's
arithmetic: no packing, no dequantisation, no dot products, no argmax.  Both
sides of every parity check (the fp64 oracle under ``oracle/`` and the HIP
library under ``packed_twin_int8_amd/``) start from the raw arrays produced
here and then do their own work on them.

The weights stand in for a real model's int8 tensors, which are not
available: int8 values uniform over [-127, 127], one f16 scale per 32
consecutive weights of a row, uniform in [1e-3, 1e-2] before rounding to f16,
and fp32 activations ~ N(0, 1).  Shapes follow the workloads measured on the
pages (a Qwen-27B-class FFN projection of 17408 x 5120, the decoder-layer
matrices of a 5120-wide model, and a small 4-layer MLP stack).

Draw order is fixed so that a given seed always yields the same arrays:
twin workloads draw A, B, scale_A, scale_B, x_A, x_B; multi-stream Q8
workloads draw Q, scale, X[0..n-1].  Generators are numpy PCG64.
"""

from __future__ import annotations

import numpy as np

BLOCK = 32  # weights per scale block (both formats)

# seeds of the named workloads
SEED_TINY = 0
SEED_SSQ_FFN = 2
SEED_Q8_FFN = 3
SEED_LAYER = 4
SEED_TOY = 1
SEED_BIG = 5


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def int8_uniform(g: np.random.Generator, shape) -> np.ndarray:
    """int8 uniform over [-127, 127] (inclusive)."""
    return g.integers(-127, 128, size=shape, dtype=np.int8)


def f16_scales(g: np.random.Generator, shape, lo: float = 1e-3, hi: float = 1e-2) -> np.ndarray:
    """f16 bit patterns (uint16) of values drawn uniform in [lo, hi) in float64
    and rounded to binary16 (numpy's cast rounds to nearest even)."""
    return g.uniform(lo, hi, size=shape).astype(np.float16).view(np.uint16)


def activations(g: np.random.Generator, shape) -> np.ndarray:
    """fp32 activations ~ N(0, 1) (drawn in float64, cast to float32)."""
    return g.standard_normal(size=shape).astype(np.float32)


def twin(rows: int, cols: int, seed: int, same: bool = False, same_x: bool = False):
    """Raw twin inputs: dict with A, B (int8 [rows, cols]), sA, sB (uint16
    f16 bits [rows, cols/32]), xA, xB (float32 [cols]).

    ``same``: twin B is a copy of twin A (the self-speculation case: one model
    packed against itself).  ``same_x``: x_B is a copy of x_A."""
    assert cols % BLOCK == 0
    g = rng(seed)
    nb = cols // BLOCK
    A = int8_uniform(g, (rows, cols))
    B = A.copy() if same else int8_uniform(g, (rows, cols))
    sA = f16_scales(g, (rows, nb))
    sB = sA.copy() if same else f16_scales(g, (rows, nb))
    xA = activations(g, (cols,))
    xB = xA.copy() if same_x else activations(g, (cols,))
    return dict(A=A, B=B, sA=sA, sB=sB, xA=xA, xB=xB)


def q8(rows: int, cols: int, n: int, seed: int):
    """Raw single-model inputs: Q (int8 [rows, cols]), S (uint16 f16 bits
    [rows, cols/32]), X (float32 [n, cols])."""
    assert cols % BLOCK == 0
    g = rng(seed)
    Q = int8_uniform(g, (rows, cols))
    S = f16_scales(g, (rows, cols // BLOCK))
    X = activations(g, (n, cols))
    return dict(Q=Q, S=S, X=X)


def logits(n: int, vocab: int, seed: int, scale: float = 1.0) -> np.ndarray:
    """fp32 logits [n, vocab] ~ N(0, scale^2)."""
    g = rng(seed)
    return (g.standard_normal(size=(n, vocab)) * scale).astype(np.float32)


# Decoder-layer matrix shapes of a 5120-wide model with 1024-wide k/v heads and
# a 17408-wide FFN: (name, rows, cols).
LAYER_SHAPES = (
    ("q", 5120, 5120),
    ("k", 1024, 5120),
    ("v", 1024, 5120),
    ("o", 5120, 5120),
    ("gate", 17408, 5120),
    ("up", 17408, 5120),
    ("down", 5120, 17408),
)

# Small random-init MLP-residual stack used by the end-to-end twin decode.
TOY = dict(hidden=2048, ffn=5632, layers=4, vocab=32000)


def toy_weights(seed: int = SEED_TOY, lm_scale_div: float = 1.0, hidden: int | None = None, ffn: int | None = None,
                layers: int | None = None, vocab: int | None = None):
    """Raw weights of the toy stack, drawn in a fixed order: embedding Q8
    [vocab, hidden]; per layer gate [ffn, hidden], up [ffn, hidden],
    down [hidden, ffn]; LM head [vocab, hidden].  Each matrix draws its int8
    values then its f16 scales.  ``lm_scale_div`` divides the LM-head scales
    (before f16 rounding) to flatten the output distribution.  The sizes
    default to TOY; smaller ones give the same distributions at test scale."""
    g = rng(seed)
    h = TOY["hidden"] if hidden is None else hidden
    f = TOY["ffn"] if ffn is None else ffn
    L = TOY["layers"] if layers is None else layers
    V = TOY["vocab"] if vocab is None else vocab

    def mat(r, c, div=1.0):
        q = int8_uniform(g, (r, c))
        s = f16_scales(g, (r, c // BLOCK), 1e-3 / div, 1e-2 / div)
        return dict(Q=q, S=s)

    emb = mat(V, h)
    layers = [dict(gate=mat(f, h), up=mat(f, h), down=mat(h, f)) for _ in range(L)]
    head = mat(V, h, lm_scale_div)
    return dict(emb=emb, layers=layers, head=head)

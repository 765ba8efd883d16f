"""Exact acceptance arithmetic of staggered self-speculation.

TEST INFRASTRUCTURE (part of the oracle).

Pages cited by title and section:
  [README] "打包双子推理（PTI）" (bittide.aicompass.dev, the project README in
           translation), section "接受机制如何工作" (how acceptance works).

What the section fixes, restated: N streams run one model at staggered
positions.  Stream 0 runs on the last confirmed token; stream i >= 1 runs on a
guess for the token that stream i-1 is about to produce, a guess sampled by the
same model one step earlier from the same context.  Check i compares that
guess with stream i-1's fresh output.  Under sampling both are independent
draws from one distribution p, so a check passes with the collision
probability sum_x p(x)^2, with no rejection-sampling correction.  A failed
check voids every later stream, so the tokens gained per step are
1 + P + P^2 + ... + P^(N-1) when every check has the same P.

Everything here is exact rational arithmetic (``fractions.Fraction``) and
brute-force enumeration; it is only meant for tiny vocabularies.
"""

from __future__ import annotations

import itertools
from fractions import Fraction
from typing import Sequence


def collision(p: Sequence[Fraction]) -> Fraction:
    """sum_x p(x)^2."""
    return sum((Fraction(q) ** 2 for q in p), Fraction(0))


def accept_count(guesses: Sequence[int], outputs: Sequence[int]) -> int:
    """1 + length of the leading run of i >= 1 with guesses[i] == outputs[i-1].
    guesses[0] (stream 0's confirmed input) is never checked."""
    a = 1
    for i in range(1, len(guesses)):
        if guesses[i] != outputs[i - 1]:
            break
        a += 1
    return a


def expected_accept_iid(p: Sequence[Fraction], n: int) -> Fraction:
    """E[accept count] by brute force over every draw, for a model whose output
    distribution p is the same at every position (context-free).

    Enumerates the outputs o_0..o_{n-2} (o_{n-1} is never checked) and the
    guesses g_1..g_{n-1}, all independent draws from p, and sums
    Pr(draw) * accept_count exactly."""
    p = [Fraction(q) for q in p]
    assert sum(p) == 1 and n >= 1
    V = len(p)
    total = Fraction(0)
    for outs in itertools.product(range(V), repeat=n - 1):
        po = Fraction(1)
        for o in outs:
            po *= p[o]
        if po == 0:
            continue
        for gs in itertools.product(range(V), repeat=n - 1):
            pr = po
            for g in gs:
                pr *= p[g]
            if pr == 0:
                continue
            a = accept_count((None,) + gs, outs + (None,))
            total += pr * a
    return total


def expected_accept_formula(P: Fraction, n: int) -> Fraction:
    """sum_{i<n} P^i."""
    return sum((Fraction(P) ** i for i in range(n)), Fraction(0))


def expected_accept_markov(T: Sequence[Sequence[Fraction]], inputs: Sequence[int]) -> Fraction:
    """E[accept count] of one step for a model whose next-token distribution
    depends only on the current token (row T[t] of a transition matrix), as an
    MLP-only stack without attention is.

    inputs[0] is stream 0's confirmed token, inputs[i] stream i's guess.  Each
    stream's output o_i is drawn from T[inputs[i]]; the guesses are fixed here
    (the step is conditioned on them).  Enumerates o_0..o_{n-2}."""
    n = len(inputs)
    V = len(T)
    total = Fraction(0)
    for outs in itertools.product(range(V), repeat=n - 1):
        pr = Fraction(1)
        for i, o in enumerate(outs):
            pr *= Fraction(T[inputs[i]][o])
        if pr == 0:
            continue
        total += pr * accept_count(inputs, outs + (None,))
    return total


def expected_accept_markov_fresh(T: Sequence[Sequence[Fraction]], confirmed: int, n: int) -> Fraction:
    """E[accept count] when the guesses themselves were drawn one step earlier
    from the contexts they will be checked in (the steady state of the
    staggered loop): g_1 ~ T[confirmed], g_{i+1} ~ T[g_i].  Enumerates the
    guesses and the outputs."""
    V = len(T)
    total = Fraction(0)
    for gs in itertools.product(range(V), repeat=n - 1):
        pg = Fraction(1)
        prev = confirmed
        for g in gs:
            pg *= Fraction(T[prev][g])
            prev = g
        if pg == 0:
            continue
        total += pg * expected_accept_markov(T, (confirmed,) + gs)
    return total

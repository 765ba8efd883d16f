"""Exact acceptance arithmetic (CPU only).

Brute-force enumeration over every draw, in exact rationals, against the
tokens-per-step formula of the README page's acceptance section
(1 + P + ... + P^(N-1) with P = sum_x p(x)^2) and against the table the page
prints for four streams (tests/golden/accept_table.json)."""

import json
import os
from fractions import Fraction as F

import pytest

from oracle import accept

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

DISTS = [
    [F(1), F(0)],
    [F(1, 2), F(1, 2)],
    [F(3, 4), F(1, 4)],
    [F(1, 3), F(1, 3), F(1, 3)],
    [F(1, 2), F(3, 10), F(1, 5)],
    [F(7, 10), F(1, 5), F(1, 10)],
]


@pytest.mark.parametrize("p", DISTS, ids=[str(i) for i in range(len(DISTS))])
@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_enumeration_equals_formula(p, n):
    P = accept.collision(p)
    assert accept.expected_accept_iid(p, n) == accept.expected_accept_formula(P, n)


def test_collision_bounds_and_special_cases():
    for p in DISTS:
        P = accept.collision(p)
        assert F(1, len(p)) <= P <= 1
    # greedy (a point mass) accepts every check: N tokens per step
    assert accept.expected_accept_iid([F(0), F(1), F(0)], 4) == 4
    # uniform over V: P = 1/V
    assert accept.collision([F(1, 5)] * 5) == F(1, 5)


def test_printed_table():
    with open(os.path.join(GOLDEN, "accept_table.json")) as f:
        g = json.load(f)
    n = g["n_streams"]
    for row in g["rows"]:
        P = F(row["p"])
        ev = accept.expected_accept_formula(P, n)
        assert abs(float(ev) - row["printed_tokens_per_step"]) <= 0.02, row
    assert accept.expected_accept_formula(F(1), n) == 4


def _recursive(T, ctx, k):
    # f_k(ctx) = 1 + sum_t T[ctx][t]^2 f_{k-1}(t), f_1 = 1: a check passes when
    # two independent draws from T[ctx] collide on t, and the next check is
    # then made in context t.
    if k == 1:
        return F(1)
    return 1 + sum(T[ctx][t] ** 2 * _recursive(T, t, k - 1) for t in range(len(T)))


def test_markov_enumeration_matches_collision_recursion():
    T = [[F(1, 2), F(1, 4), F(1, 4)],
         [F(0), F(2, 3), F(1, 3)],
         [F(1, 5), F(1, 5), F(3, 5)]]
    for c in range(3):
        for n in (1, 2, 3, 4):
            assert accept.expected_accept_markov_fresh(T, c, n) == _recursive(T, c, n)


def test_markov_fixed_guesses():
    T = [[F(1, 2), F(1, 2)], [F(1, 4), F(3, 4)]]
    # stream 1's guess g1=1 is accepted when o0 == 1: Pr = T[0][1] = 1/2;
    # then stream 2's guess g2=0 is accepted when o1 == 0: Pr = T[1][0] = 1/4
    assert accept.expected_accept_markov(T, (0, 1, 0)) == 1 + F(1, 2) * (1 + F(1, 4))

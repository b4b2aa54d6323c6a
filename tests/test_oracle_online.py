"""Pins for the online normaliser and the (m, l) combine.

The running-state table of Ch.6 §6.3.2 is a golden fixture; the claim of
Ch.6 §6.3.3 and §6.4.1 that the online form reaches the safe-softmax (max, sum)
for any order and any association tree is checked by brute force against the
three-pass oracle, including -inf entries, ties and +-1000 offsets.
"""

import itertools
import json
import math
import os
import random

import numpy as np
import pytest

from oracle import (EMPTY_STATE, all_trees, combine, online_state, singleton, softmax_rows_ref,
                    tree_reduce)


def _ref_max_sum(xs):
    _, (m, s, _) = softmax_rows_ref(np.array([xs], dtype=np.float64), return_stats=True)
    return m[0], s[0]


def _close(a, b, rel=1e-14):
    (m1, l1), (m2, l2) = a, b
    if m1 == -math.inf or m2 == -math.inf:
        return m1 == m2 and l1 == 0.0 and l2 == 0.0
    return m1 == m2 and abs(l1 - l2) <= rel * max(abs(l1), abs(l2))


def test_trace_table_matches_printed(golden_dir):
    with open(os.path.join(golden_dir, "worked_example_ch6_6_3_2.json")) as f:
        g = json.load(f)
    (m, l), states = online_state(g["x"], trace=True)
    tol = g["abs_tolerance"]["online_l"]
    for st, row in zip(states, g["online_trace"]):
        assert st[0] == row["m"]
        assert abs(st[1] - row["l"]) <= tol
    assert (m, l) == states[-1]


def test_empty_and_all_masked_give_identity():
    assert online_state([]) == EMPTY_STATE
    assert online_state([-math.inf] * 5) == EMPTY_STATE
    assert combine(EMPTY_STATE, EMPTY_STATE) == EMPTY_STATE


def test_identity_is_exact():
    for s in [(1.5, 2.25), (-1000.0, 0.5), (1000.0, 3.0)]:
        assert combine(s, EMPTY_STATE) == s
        assert combine(EMPTY_STATE, s) == s


def test_commutative_exactly():
    rnd = random.Random(7)
    for _ in range(500):
        a = (rnd.uniform(-30, 30), rnd.uniform(0.1, 50))
        b = (rnd.uniform(-30, 30), rnd.uniform(0.1, 50))
        assert combine(a, b) == combine(b, a)


def test_associative_within_rounding():
    rnd = random.Random(8)
    for _ in range(500):
        a, b, c = [(rnd.uniform(-30, 30), rnd.uniform(0.1, 50)) for _ in range(3)]
        assert _close(combine(combine(a, b), c), combine(a, combine(b, c)), rel=1e-13)


VALUE_SETS = [
    [1.0, 5.0, 3.0],
    [0.5, -2.0, 0.5, 7.25, -math.inf],            # a tie and a masked entry
    [-math.inf, -math.inf, 2.0, -1.0],            # leading masked entries
    [1000.0, 999.5, 1001.25, 998.0, 1000.0],      # overflow range, with a tie
    [-1000.0, -999.0, -1001.5],
    [-math.inf, -math.inf, -math.inf],            # fully masked
    [3.0, -4.0, 0.0, 12.0, -7.5, 2.5],
]


@pytest.mark.parametrize("xs", VALUE_SETS)
def test_online_equals_two_pass_every_order(xs):
    want = _ref_max_sum(xs)
    for perm in itertools.permutations(xs):
        got = online_state(perm)
        if want[0] == -math.inf:
            assert got == EMPTY_STATE
        else:
            assert _close(got, want), (perm, got, want)


@pytest.mark.parametrize("xs", VALUE_SETS)
def test_combine_equals_two_pass_every_tree_and_order(xs):
    # Every permutation of the singletons and every parenthesisation of the
    # combine (Catalan many): all must reach the safe-softmax (max, sum).
    want = _ref_max_sum(xs)
    trees = all_trees(0, len(xs))
    for perm in itertools.permutations(xs):
        leaves = [online_state([x]) for x in perm]
        for t in trees:
            got = tree_reduce(t, leaves)
            if want[0] == -math.inf:
                assert got == EMPTY_STATE
            else:
                assert _close(got, want), (perm, t, got, want)


def test_chunked_states_combine_to_whole():
    # Block-wise recurrence (xxqk §3.2): the state of a concatenation is the
    # combine of the states of its pieces, for any split points.
    rnd = random.Random(9)
    xs = [rnd.gauss(0, 4) for _ in range(40)] + [-math.inf] * 3
    rnd.shuffle(xs)
    whole = online_state(xs)
    for _ in range(50):
        cuts = sorted(rnd.sample(range(1, len(xs)), 4))
        pieces = [xs[a:b] for a, b in zip([0] + cuts, cuts + [len(xs)])]
        st = EMPTY_STATE
        for p in pieces:
            st = combine(st, online_state(p))
        assert _close(st, whole, rel=1e-13)
    assert _close(whole, _ref_max_sum(xs), rel=1e-13)


# ---------------------------------------------------------------------------
# The enumeration the every-tree test relies on.  If all_trees returned too
# few trees (an off-by-one in its split range gives none at all), the test
# above would pass without trying the association orders it claims to.
# ---------------------------------------------------------------------------

CATALAN = [1, 1, 2, 5, 14, 42, 132]  # C(n - 1) binary trees over n ordered leaves


def _render(tree):
    """The parenthesisation a tree stands for, written out by the test."""
    if isinstance(tree, int):
        return str(tree)
    return "(" + _render(tree[0]) + "," + _render(tree[1]) + ")"


def _leaves(tree):
    return [tree] if isinstance(tree, int) else _leaves(tree[0]) + _leaves(tree[1])


def _stack_parenthesisations(n):
    """Every full parenthesisation of leaves 0..n-1, enumerated another way:
    each run of a stack machine that pushes the leaves in order and, at any
    point, may pop two entries and push their bracketed pair."""
    found = set()

    def run(stack, nxt):
        if nxt == n and len(stack) == 1:
            found.add(stack[0])
        if nxt < n:
            run(stack + [str(nxt)], nxt + 1)
        if len(stack) >= 2:
            run(stack[:-2] + ["(" + stack[-2] + "," + stack[-1] + ")"], nxt)

    run([], 0)
    return found


@pytest.mark.parametrize("n", range(1, 8))
def test_all_trees_is_every_parenthesisation(n):
    trees = all_trees(0, n)
    rendered = [_render(t) for t in trees]
    assert len(trees) == CATALAN[n - 1]
    assert len(set(rendered)) == len(trees), "trees must be distinct"
    for t in trees:
        assert _leaves(t) == list(range(n)), "leaves in order, each once"
    assert set(rendered) == _stack_parenthesisations(n)


def test_all_trees_on_an_offset_range():
    assert all_trees(3, 4) == [3]
    assert all_trees(2, 4) == [(2, 3)]
    assert sorted(map(_render, all_trees(4, 7))) == ["((4,5),6)", "(4,(5,6))"]


@pytest.mark.parametrize("n", range(1, 7))
def test_tree_reduce_follows_the_tree(n):
    # A non-commutative, non-associative probe operation: the reduction
    # must reproduce the tree's own bracketing, with left and right in place.
    leaves = [str(i) for i in range(n)]
    for t in all_trees(0, n):
        got = tree_reduce(t, leaves, op=lambda a, b: "(" + a + "," + b + ")")
        assert got == _render(t)


def test_singleton_states():
    assert singleton(2.5) == (2.5, 1.0)
    assert singleton(-math.inf) == EMPTY_STATE
    # One element through the recurrence: (x, e^(x - x)) = (x, 1).
    assert online_state([-3.25]) == (-3.25, 1.0)

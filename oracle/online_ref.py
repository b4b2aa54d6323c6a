"""Online normaliser and (m, l) combine, scalar float64 (test infrastructure only).

This module is never compared with the GPU.  It exists so that the tests can
show, by brute force over every order and every association tree of small
inputs, that the online recurrence and its combine reach the same (max, sum) as
the three-pass oracle, which is the property the whole method rests on.

The state (m, l) of a set of values stands for the positive number l * e^m,
which equals the sum of e^x over the set ([Ch6 §6.3.1]: m is the running
maximum and l the sum of e^(x - m)).  Merging two sets adds their numbers, and
[Ch6 §6.4.1] writes that sum against the larger of the two exponents.  The
empty set is the number 0, written (-inf, 0).  Everything below is built from
that one addition: one element x is the state (x, 1), and the element-wise
recurrence of [Ch6 §6.3.1] is the left fold of the addition over the elements.

Parity status: pinned.  ``online_state`` by the running-state table of
[Ch6 §6.3.2] and by brute-force equivalence with
``softmax_ref.softmax_rows_ref`` over every order of small inputs;
``combine`` and ``tree_reduce`` by the same equivalence over every association
tree, and by the monoid laws; ``all_trees`` by the Catalan count of distinct
trees and by comparison with an independent enumeration of parenthesisations
(tests/test_oracle_online.py).
"""

import math

#: The state of the empty set, the number 0 ([Ch6 §6.3.1] starts the running
#: state at m = -inf, l = 0).  It is the identity of ``combine``.
EMPTY_STATE = (-math.inf, 0.0)


def singleton(x):
    """The state of the one-element set {x}: e^x = 1 * e^x, i.e. (x, 1).

    An element equal to -inf adds e^-inf = 0, so its set is the empty state.
    """
    x = float(x)
    return EMPTY_STATE if x == -math.inf else (x, 1.0)


def combine(a, b):
    """Add the numbers two states stand for ([Ch6 §6.4.1]).

    With M = max(m1, m2), l1 e^m1 + l2 e^m2 = (l1 e^(m1 - M) + l2 e^(m2 - M)) e^M,
    so the merged state is (M, l1 e^(m1 - M) + l2 e^(m2 - M)).  Writing it
    against the larger exponent keeps every factor e^(m - M) at most 1.  An
    empty side adds 0 and leaves the other side as it is (this is the guard the
    chapter needs, since e^(-inf - (-inf)) is undefined).
    """
    if a[1] == 0.0:
        return b
    if b[1] == 0.0:
        return a
    big = max(a[0], b[0])
    scaled = [l * math.exp(m - big) for (m, l) in (a, b)]
    return (big, scaled[0] + scaled[1])


def online_state(xs, trace=False):
    """The element-wise online normaliser of [Ch6 §6.3.1] over ``xs``.

    One pass, one element at a time: the running state absorbs each element's
    singleton state with ``combine``.  That is the chapter's update
    m' = max(m, x), l' = l e^(m - m') + e^(x - m') (for x = -inf the state is
    unchanged).

    Returns the final (m, l); with ``trace`` also the list of states after each
    element, which reproduces the running-state table of [Ch6 §6.3.2].
    """
    state = EMPTY_STATE
    states = []
    for x in xs:
        state = combine(state, singleton(x))
        states.append(state)
    return (state, states) if trace else state


def tree_reduce(tree, leaves, op=combine):
    """Reduce leaf states along an explicit binary association tree.

    ``tree`` is either an int (index of a leaf in ``leaves``) or a pair
    ``(left, right)`` of trees; ``op`` (default ``combine``) merges the results
    of the two subtrees, left operand first.  Used to try every
    parenthesisation of a reduction.
    """
    if isinstance(tree, int):
        return leaves[tree]
    left, right = tree
    return op(tree_reduce(left, leaves, op), tree_reduce(right, leaves, op))


def all_trees(lo, hi):
    """Every binary tree whose leaves are lo, lo+1, ..., hi-1 in order.

    A tree over more than one leaf splits its range at some point mid
    (lo < mid < hi) into a left tree over [lo, mid) and a right tree over
    [mid, hi); every choice of mid and of the two subtrees gives one tree.
    """
    if hi - lo == 1:
        return [lo]
    out = []
    for mid in range(lo + 1, hi):
        for left in all_trees(lo, mid):
            for right in all_trees(mid, hi):
                out.append((left, right))
    return out

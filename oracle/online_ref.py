"""Online normaliser and (m, l) combine, scalar float64 (test infrastructure only).

This module is never compared with the GPU.  It exists so that the tests can
show, by brute force over every order and every association tree of small
inputs, that the online recurrence and its combine reach the same (max, sum) as
the three-pass oracle, which is the property the whole method rests on.

Parity status: pinned by the running-state table of [Ch6 §6.3.2] and by the
brute-force equivalence with ``softmax_ref.softmax_rows_ref``.
"""

import math

#: The identity of the combine: "nothing seen yet" ([Ch6 §6.3.1]: m_0 = -inf,
#: l_0 = 0).
EMPTY_STATE = (-math.inf, 0.0)


def _exp(v):
    return 0.0 if v == -math.inf else math.exp(v)


def online_state(xs, trace=False):
    """Run the element-wise online normaliser over ``xs``.

    [Ch6 §6.3.1]: starting from (m_0, l_0) = (-inf, 0), each new element x gives
    m' = max(m, x) and l' = l * e^(m - m') + e^(x - m').  When m' is still -inf
    (only -inf seen so far) the state is left unchanged, since e^(-inf - (-inf))
    would be NaN; that is the guard [Ch6 §6.4] insists on.

    Returns the final (m, l); with ``trace`` also the list of states after each
    element, which reproduces the table of [Ch6 §6.3.2].
    """
    m, l = EMPTY_STATE
    states = []
    for x in xs:
        x = float(x)
        m_new = max(m, x)
        if m_new != -math.inf:
            l = l * _exp(m - m_new) + _exp(x - m_new)
            m = m_new
        states.append((m, l))
    return ((m, l), states) if trace else (m, l)


def combine(a, b):
    """Merge two partial states ([Ch6 §6.4.1]).

    combine((m1, l1), (m2, l2)) = (M, l1 e^(m1 - M) + l2 e^(m2 - M)) with
    M = max(m1, m2).  If both sides are empty (M = -inf) the result is the empty
    state.  The state (m, l) stands for the quantity l * e^m, and combine adds two
    such quantities, which is why it is commutative and associative with
    identity (-inf, 0).
    """
    (m1, l1), (m2, l2) = a, b
    M = max(m1, m2)
    if M == -math.inf:
        return EMPTY_STATE
    return (M, l1 * _exp(m1 - M) + l2 * _exp(m2 - M))


def tree_reduce(tree, leaves):
    """Reduce leaf states along an explicit binary association tree.

    ``tree`` is either an int (index of a leaf in ``leaves``) or a pair
    ``(left, right)`` of trees.  Used to enumerate every parenthesisation.
    """
    if isinstance(tree, int):
        return leaves[tree]
    left, right = tree
    return combine(tree_reduce(left, leaves), tree_reduce(right, leaves))


def all_trees(lo, hi):
    """Every binary tree whose leaves are lo, lo+1, ..., hi-1 in order."""
    if hi - lo == 1:
        return [lo]
    out = []
    for mid in range(lo + 1, hi):
        for left in all_trees(lo, mid):
            for right in all_trees(mid, hi):
                out.append((left, right))
    return out

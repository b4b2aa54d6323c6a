"""Pins for the attention backward oracle.

Central finite differences of the forward oracle (itself pinned in
test_oracle_attention.py), torch's float64 CPU autograd of
scaled_dot_product_attention, closed forms (one visible key, causal row 0) and
three identities that every correct gradient of attention obeys; the
probabilities the gradients are built from, entry by entry from their
definition.
"""

import math

import numpy as np
import pytest
import torch

from oracle import (attention_bwd_head_ref, attention_bwd_ref, attention_dq_rows_ref,
                    attention_head_ref, attention_probs_head_ref)


def _rand(shape, seed, sigma=1.0):
    return sigma * np.random.default_rng(seed).standard_normal(shape)


def _loss(q, k, v, do, scale, causal, kv_len=None, bias=None):
    O, _ = attention_head_ref(q, k, v, scale, causal, kv_len=kv_len, bias=bias)
    return float(np.sum(O * do))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kv_len", [None, 3, 0])
def test_probabilities_brute_force(causal, kv_len):
    # P from its definition, one entry at a time in pure Python: e^s over the
    # sum of e^s of the row's visible keys (causal: key <= row; key < kv_len;
    # bias -inf hides a key); a row with no visible key is all zero.
    n, d = 5, 3
    q, k = _rand((n, d), 21), _rand((n, d), 22)
    bias = _rand((n, n), 23)
    bias[2, 1] = -np.inf
    scale = 0.625  # a float32 value: the oracle takes the scale as float32
    P = attention_probs_head_ref(q, k, scale, causal, kv_len=kv_len, bias=bias)
    for i in range(n):
        vis = [j for j in range(n)
               if (not causal or j <= i) and (kv_len is None or j < kv_len)
               and bias[i, j] != -np.inf]
        e = {j: math.exp(scale * sum(q[i, t] * k[j, t] for t in range(d)) + bias[i, j])
             for j in vis}
        tot = sum(e.values())
        for j in range(n):
            want = e[j] / tot if j in e else 0.0
            assert abs(P[i, j] - want) <= 1e-14, (i, j, P[i, j], want)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d,dv", [(1, 3, 2), (4, 3, 3), (6, 4, 5)])
def test_finite_differences(n, d, dv, causal):
    q, k, v = _rand((n, d), 1), _rand((n, d), 2), _rand((n, dv), 3)
    do = _rand((n, dv), 4)
    scale = 0.6
    grads = attention_bwd_head_ref(q, k, v, do, scale, causal)
    h = 1e-6
    for which, g in zip(range(3), grads):
        base = [q, k, v][which]
        fd = np.zeros_like(base)
        for idx in np.ndindex(*base.shape):
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += h
            lp = _loss(*args, do, scale, causal)
            args[which][idx] -= 2 * h
            lm = _loss(*args, do, scale, causal)
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, fd, atol=2e-8, rtol=0)


def test_finite_differences_kv_len_and_bias():
    n, d = 5, 3
    q, k, v, do = (_rand((n, d), s) for s in (5, 6, 7, 8))
    bias = _rand((n, n), 9)
    bias[1, 0] = -np.inf
    grads = attention_bwd_head_ref(q, k, v, do, 0.9, False, kv_len=3, bias=bias)
    h = 1e-6
    for which, g in zip(range(3), grads):
        base = [q, k, v][which]
        fd = np.zeros_like(base)
        for idx in np.ndindex(*base.shape):
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += h
            lp = _loss(*args, do, 0.9, False, kv_len=3, bias=bias)
            args[which][idx] -= 2 * h
            lm = _loss(*args, do, 0.9, False, kv_len=3, bias=bias)
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, fd, atol=2e-8, rtol=0)
    # Hidden keys get no gradient at all.
    assert (grads[1][3:] == 0).all() and (grads[2][3:] == 0).all()


@pytest.mark.parametrize("causal", [False, True])
def test_torch_autograd_float64(causal):
    B, H, N, D = 2, 3, 37, 16
    q, k, v, do = (_rand((B, H, N, D), s) for s in (11, 12, 13, 14))
    scale = float(np.float32(1 / math.sqrt(D)))
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                           scale=scale)
    out.backward(torch.tensor(do))
    dQ, dK, dV = attention_bwd_ref(q, k, v, do, scale, causal)
    for mine, theirs in ((dQ, tq.grad), (dK, tk.grad), (dV, tv.grad)):
        np.testing.assert_allclose(mine, theirs.numpy(), atol=1e-12, rtol=0)


def test_single_key_closed_form():
    q, k, v, do = (_rand((1, 8), s) for s in (21, 22, 23, 24))
    dQ, dK, dV = attention_bwd_head_ref(q, k, v, do, 0.3, False)
    assert (dQ == 0).all() and (dK == 0).all()
    np.testing.assert_allclose(dV, do, atol=1e-15, rtol=0)


def test_causal_row_zero_has_no_query_gradient():
    n, d = 9, 4
    q, k, v, do = (_rand((n, d), s) for s in (31, 32, 33, 34))
    dQ, dK, dV = attention_bwd_head_ref(q, k, v, do, 0.5, True)
    assert (dQ[0] == 0).all()
    # The last key is seen by the last query only, with weight P[n-1, n-1].
    P_last = math.exp(0.5 * q[-1] @ k[-1] - attention_head_ref(q, k, v, 0.5, True)[1][-1])
    np.testing.assert_allclose(dV[-1], P_last * do[-1], atol=1e-14, rtol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_invariants(causal):
    n, d = 40, 8
    q, k = _rand((n, d), 41, 1.5), _rand((n, d), 42, 1.5)
    v, do = _rand((n, d), 43), _rand((n, d), 44)
    dQ, dK, dV = attention_bwd_head_ref(q, k, v, do, 0.4, causal)
    # Scores shift by q_i . c for every key of row i: O is unchanged.
    np.testing.assert_allclose(dK.sum(axis=0), 0.0, atol=1e-12)
    # Every row of P sums to 1.
    np.testing.assert_allclose(dV.sum(axis=0), do.sum(axis=0), atol=1e-12)
    # S is unchanged by Q -> tQ, K -> K/t.
    assert abs(np.sum(dQ * q) - np.sum(dK * k)) < 1e-11


@pytest.mark.parametrize("causal", [False, True])
def test_dq_rows_match_the_full_gradient(causal):
    n, d = 50, 6
    q, k, v, do = (_rand((n, d), s) for s in (51, 52, 53, 54))
    dQ, _, _ = attention_bwd_head_ref(q, k, v, do, 0.7, causal)
    rows = [0, 1, 17, 49]
    np.testing.assert_allclose(attention_dq_rows_ref(q, k, v, do, 0.7, causal, rows), dQ[rows],
                               atol=1e-13, rtol=0)

"""Pins for the attention oracle.

Closed forms (one visible key, identical keys, all-ones values), a joint
permutation of keys and values, torch's float64 CPU scaled_dot_product_attention
and logsumexp, a pure-Python scalar brute force on tiny sizes, and the
alpha/beta streaming form of Ch.6 §6.6 (which the chapter reports agrees with
the direct form to about 1e-15).
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention_head_ref, attention_ref, blocked_attention_row_ref
import osm_inputs


def _rand(shape, seed, sigma=1.0):
    return sigma * np.random.default_rng(seed).standard_normal(shape)


def _brute(q, k, v, scale, causal):
    """Scalar loops with math.exp: attention by its definition."""
    nq, d = len(q), len(q[0])
    out, lses = [], []
    s = float(np.float32(scale))
    for i in range(nq):
        scores = []
        for j in range(len(k)):
            if causal and j > i:
                continue
            scores.append((j, s * sum(q[i][t] * k[j][t] for t in range(d))))
        mx = max(sc for _, sc in scores)
        w = [(j, math.exp(sc - mx)) for j, sc in scores]
        tot = sum(x for _, x in w)
        out.append([sum(x * v[j][t] for j, x in w) / tot for t in range(len(v[0]))])
        lses.append(mx + math.log(tot))
    return np.array(out), np.array(lses)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(1, 1), (3, 2), (5, 4), (8, 3)])
def test_pure_python_brute_force(n, d, causal):
    q, k, v = _rand((n, d), 1), _rand((n, d), 2), _rand((n, d + 1), 3)
    scale = 0.7
    O, L = attention_head_ref(q, k, v, scale, causal)
    Ob, Lb = _brute(q.tolist(), k.tolist(), v.tolist(), scale, causal)
    np.testing.assert_allclose(O, Ob, atol=1e-13, rtol=0)
    np.testing.assert_allclose(L, Lb, atol=1e-13, rtol=0)


def test_single_key_closed_form():
    q, k, v = _rand((1, 16), 4), _rand((1, 16), 5), _rand((1, 16), 6)
    s = 0.25
    O, L = attention_head_ref(q, k, v, s, causal=False)
    np.testing.assert_allclose(O[0], v[0], rtol=0, atol=1e-15)
    assert abs(L[0] - s * float(q[0] @ k[0])) < 1e-13


def test_causal_row0_sees_only_key0():
    q, k, v = _rand((10, 8), 7), _rand((10, 8), 8), _rand((10, 8), 9)
    s = float(np.float32(1 / math.sqrt(8)))
    O, L = attention_head_ref(q, k, v, s, causal=True)
    np.testing.assert_allclose(O[0], v[0], atol=1e-15, rtol=0)
    assert abs(L[0] - s * float(q[0] @ k[0])) < 1e-13
    # The last row sees every key: same as non-causal.
    On, Ln = attention_head_ref(q, k, v, s, causal=False)
    np.testing.assert_allclose(O[-1], On[-1], atol=1e-14)
    assert abs(L[-1] - Ln[-1]) < 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_visible_values(causal):
    n, d = 12, 8
    q = _rand((n, d), 10)
    k = np.tile(_rand((1, d), 11), (n, 1))
    v = _rand((n, d), 12)
    s = 0.5
    O, L = attention_head_ref(q, k, v, s, causal)
    for i in range(n):
        cnt = i + 1 if causal else n
        np.testing.assert_allclose(O[i], v[:cnt].mean(axis=0), atol=1e-14)
        assert abs(L[i] - (s * float(q[i] @ k[0]) + math.log(cnt))) < 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_all_ones_values(causal):
    q, k = _rand((9, 4), 13, 3.0), _rand((9, 4), 14, 3.0)
    O, _ = attention_head_ref(q, k, np.ones((9, 5)), 1.0, causal)
    np.testing.assert_allclose(O, 1.0, atol=1e-14)


def test_joint_key_value_permutation_invariance():
    q, k, v = _rand((16, 8), 15), _rand((16, 8), 16), _rand((16, 8), 17)
    perm = np.random.default_rng(18).permutation(16)
    O1, L1 = attention_head_ref(q, k, v, 0.3, False)
    O2, L2 = attention_head_ref(q, k[perm], v[perm], 0.3, False)
    np.testing.assert_allclose(O1, O2, atol=1e-14)
    np.testing.assert_allclose(L1, L2, atol=1e-13)
    # ... and permuting only K (not V) does change the result: the pin has teeth.
    O3, _ = attention_head_ref(q, k[perm], v, 0.3, False)
    assert np.abs(O3 - O1).max() > 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_against_torch_sdpa_float64(causal):
    B, H, N, D = 2, 3, 40, 16
    q, k, v = (torch.from_numpy(_rand((B, H, N, D), s)) for s in (19, 20, 21))
    scale = float(np.float32(1 / math.sqrt(D)))
    O, L = attention_ref(q.numpy(), k.numpy(), v.numpy(), scale, causal)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=scale)
    np.testing.assert_allclose(O, ref.numpy(), atol=1e-13, rtol=0)
    S = scale * (q @ k.transpose(-1, -2))
    if causal:
        S = S.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    np.testing.assert_allclose(L, torch.logsumexp(S, -1).numpy(), atol=1e-13, rtol=0)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("block", [1, 7, 64])
def test_blocked_alpha_beta_form_agrees(block, causal):
    n, d = 150, 32
    q, k, v = _rand((n, d), 22), _rand((n, d), 23), _rand((n, d), 24)
    s = float(np.float32(1 / math.sqrt(d)))
    O, L = attention_head_ref(q, k, v, s, causal)
    for i in (0, 1, 63, 64, 149):
        Ob, Lb = blocked_attention_row_ref(q[i], k, v, s, block, n_visible=(i + 1) if causal else None)
        np.testing.assert_allclose(Ob, O[i], atol=1e-12, rtol=0)
        assert abs(Lb - L[i]) < 1e-12


def test_query_row_subset_and_chunking_match_full():
    q, k, v = _rand((70, 8), 25), _rand((70, 8), 26), _rand((70, 8), 27)
    O, L = attention_head_ref(q, k, v, 0.4, True, chunk=512)
    O2, L2 = attention_head_ref(q, k, v, 0.4, True, chunk=9)
    np.testing.assert_array_equal(O, O2)
    rows = [0, 5, 69, 33]
    O3, L3 = attention_head_ref(q, k, v, 0.4, True, query_rows=rows)
    np.testing.assert_array_equal(O3, O[rows])
    np.testing.assert_array_equal(L3, L[rows])


def test_scale_is_taken_at_float32():
    q, k, v = _rand((4, 128), 28), _rand((4, 128), 29), _rand((4, 128), 30)
    s64 = 1 / math.sqrt(128)
    _, L = attention_head_ref(q, k, v, s64, False)
    s32 = float(np.float32(s64))
    assert s32 != s64
    S = s32 * (q @ k.T)
    np.testing.assert_allclose(L, np.log(np.exp(S).sum(axis=1)), atol=1e-13)


def test_workload_slice_small():
    c = osm_inputs.attention_config("attn_small", N=64)
    q, k, v = (t.double().numpy() for t in (c["q"], c["k"], c["v"]))
    O, L = attention_ref(q, k, v, c["scale"], c["causal"], heads=[(0, 0), (0, 7)])
    assert O.shape == (2, 64, 64) and L.shape == (2, 64)
    assert np.isfinite(O).all() and np.isfinite(L).all()

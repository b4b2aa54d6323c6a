"""Pins for the fused-mask / row-length / key-padding / bias forms of the oracle.

Each form is tied to the unmasked oracle by an identity that a sign, index or
broadcast mistake would break, and to one independent closed form: the
softmax of log-weights is the normalised weights.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention_head_ref, attention_ref, masked_softmax_rows_ref, softmax_rows_ref


def _x(rows, cols, seed, sigma=4.0):
    return sigma * np.random.default_rng(seed).standard_normal((rows, cols))


def test_zero_mask_and_full_lengths_are_the_unmasked_softmax():
    x = _x(5, 37, 1)
    want = softmax_rows_ref(x)
    np.testing.assert_array_equal(masked_softmax_rows_ref(x, np.zeros((5, 37))), want)
    np.testing.assert_array_equal(masked_softmax_rows_ref(x, row_len=[37] * 5), want)


def test_minus_inf_mask_equals_minus_inf_logits():
    x = _x(4, 50, 2)
    mask = np.where(np.random.default_rng(3).random((4, 50)) < 0.3, -np.inf, 0.0)
    np.testing.assert_array_equal(masked_softmax_rows_ref(x, mask), softmax_rows_ref(x + mask))
    xm = x.copy()
    xm[np.isneginf(mask)] = -np.inf
    np.testing.assert_allclose(masked_softmax_rows_ref(x, mask), softmax_rows_ref(xm), atol=1e-15)


def test_log_weights_give_normalised_weights():
    # softmax(0 + log w) = w / sum(w): an independent closed form for the
    # additive mask (a sign error or a multiplicative use of the mask fails).
    w = np.random.default_rng(4).uniform(0.1, 3.0, (3, 20))
    y = masked_softmax_rows_ref(np.zeros((3, 20)), np.log(w))
    np.testing.assert_allclose(y, w / w.sum(axis=1, keepdims=True), rtol=1e-14)


def test_row_lengths_truncate_and_zero_pad():
    x = _x(4, 30, 5)
    lens = [30, 7, 0, 1]
    y = masked_softmax_rows_ref(x, row_len=lens)
    for r, n in enumerate(lens):
        np.testing.assert_allclose(y[r, :n], softmax_rows_ref(x[r:r + 1, :n])[0] if n else [],
                                   atol=1e-15)
        assert (y[r, n:] == 0).all()
    # clamping: negative lengths give a zero row, long ones the full row
    y2 = masked_softmax_rows_ref(x[:2], row_len=[-3, 99])
    assert (y2[0] == 0).all()
    np.testing.assert_array_equal(y2[1], softmax_rows_ref(x[1:2])[0])


def test_broadcast_mask_equals_tiled_mask():
    x = _x(6, 16, 6)
    m = np.random.default_rng(7).standard_normal((2, 16))
    np.testing.assert_array_equal(masked_softmax_rows_ref(x, m),
                                  masked_softmax_rows_ref(x, np.tile(m, (3, 1))))
    # a per-row constant mask is a shift: no effect (Ch.6 §6.2)
    c = np.full((6, 16), 0.0) + np.arange(6)[:, None] * 100.0
    np.testing.assert_allclose(masked_softmax_rows_ref(x, c), softmax_rows_ref(x), atol=1e-12)


def _r(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_kv_len_equals_truncated_keys():
    q, k, v = _r((20, 8), 10), _r((20, 8), 11), _r((20, 8), 12)
    O, L = attention_head_ref(q, k, v, 0.35, False, kv_len=13)
    O2, L2 = attention_head_ref(q, k[:13], v[:13], 0.35, False)
    np.testing.assert_allclose(O, O2, atol=1e-14)
    np.testing.assert_allclose(L, L2, atol=1e-13)
    O3, L3 = attention_head_ref(q, k, v, 0.35, False, kv_len=0)
    assert (O3 == 0).all() and np.isneginf(L3).all()


def test_bias_minus_inf_upper_triangle_is_causal():
    q, k, v = _r((16, 4), 13), _r((16, 4), 14), _r((16, 4), 15)
    tri = np.triu(np.full((16, 16), -np.inf), 1)
    O, L = attention_head_ref(q, k, v, 0.5, False, bias=tri)
    Oc, Lc = attention_head_ref(q, k, v, 0.5, True)
    np.testing.assert_allclose(O, Oc, atol=1e-14)
    np.testing.assert_allclose(L, Lc, atol=1e-13)


def test_bias_log_weights_closed_form():
    # identical keys: the scores are equal, so the weights are exp(bias)
    n = 12
    q = _r((n, 4), 16)
    k = np.tile(_r((1, 4), 17), (n, 1))
    v = _r((n, 4), 18)
    w = np.random.default_rng(19).uniform(0.2, 2.0, (n, n))
    O, L = attention_head_ref(q, k, v, 0.3, False, bias=np.log(w))
    np.testing.assert_allclose(O, (w @ v) / w.sum(axis=1, keepdims=True), atol=1e-13)
    np.testing.assert_allclose(L, 0.3 * (q @ k[0]) + np.log(w.sum(axis=1)), atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_against_torch_sdpa_with_float_mask(causal):
    B, H, N, D = 2, 2, 24, 8
    q, k, v = (torch.from_numpy(_r((B, H, N, D), s)) for s in (20, 21, 22))
    bias = torch.from_numpy(_r((1, H, N, N), 23))
    kv_len = [24, 9]
    scale = float(np.float32(1 / math.sqrt(D)))
    O, L = attention_ref(q.numpy(), k.numpy(), v.numpy(), scale, causal, kv_len=kv_len,
                         bias=bias.numpy())
    m = bias.expand(B, H, N, N).clone()
    for b, n in enumerate(kv_len):
        m[b, :, :, n:] = float("-inf")
    if causal:
        m = m.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=scale)
    np.testing.assert_allclose(O, ref.numpy(), atol=1e-13)
    np.testing.assert_allclose(L, torch.logsumexp(scale * (q @ k.transpose(-1, -2)) + m, -1).numpy(),
                               atol=1e-12)

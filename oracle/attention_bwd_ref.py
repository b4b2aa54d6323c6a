"""Attention backward oracle: gradients of materialised-S attention, float64.

Test infrastructure only (see the package docstring).

The pages state that the FlashAttention-2 backward keeps only the output and
one log-sum-exp per query row from the forward and recomputes the scores from
them ([Ch6 §6.5]; [xxqk §5.2], which calls this trading compute for memory).
They do not write the gradient formulas out.  The plain reading taken here is
the gradient of the forward map itself: for O = softmax(S) V with
S = scale * Q K^T (+ bias, masked as in ``attention_head_ref``) and an
upstream gradient dO, the oracle returns dL/dQ, dL/dK, dL/dV of L = <O, dO>.
It is written with the softmax Jacobian, dP_ij/dS_ik = P_ij (delta_jk - P_ik),
from the materialised probabilities; it does not use the output O or the
log-sum-exp at all.

``attention_dq_rows_ref`` gives dQ for chosen query rows only (rows are
independent for dQ), for long sequences where the full P does not fit.

Parity status: pinned.  ``attention_bwd_head_ref`` is checked against central
finite differences of the (separately pinned) forward oracle, against torch's
float64 CPU autograd of scaled_dot_product_attention, against closed forms
(one visible key; causal row 0) and against three identities that any correct
gradient obeys: the key gradients sum to zero (scores are invariant to a shift
of every key), the value gradients sum to the summed dO of the rows with a
visible key (probability rows sum to one), and <dQ, Q> = <dK, K> (scores are
invariant to Q -> t Q, K -> K / t).  ``attention_dq_rows_ref`` is checked
against the rows of ``attention_bwd_head_ref``.
"""

import numpy as np

from .attention_ref import _scale64


def attention_probs_head_ref(q, k, scale, causal, kv_len=None, bias=None):
    """Probabilities P = softmax(scale * Q K^T + bias) of one (batch, head),
    float64, with the masks of ``attention_head_ref`` and its three-pass safe
    softmax ([Ch6 §6.2]).  Rows with no visible key are all zero.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    nq, nk = q.shape[0], k.shape[0]
    if causal and nq != nk:
        raise ValueError("causal attention here assumes len(Q) == len(K)")
    S = _scale64(scale) * (q @ k.T)
    if bias is not None:
        S = S + np.asarray(bias, dtype=np.float64)
    key_idx = np.arange(nk)
    if kv_len is not None:
        S = np.where(key_idx[None, :] >= int(kv_len), -np.inf, S)
    if causal:
        S = np.where(key_idx[None, :] > np.arange(nq)[:, None], -np.inf, S)
    m = np.max(S, axis=1)
    live = m > -np.inf
    E = np.exp(S - np.where(live, m, 0.0)[:, None])
    l = np.sum(E, axis=1)
    P = np.zeros_like(E)
    P[live] = E[live] / l[live, None]
    return P


def attention_bwd_head_ref(q, k, v, do, scale, causal, kv_len=None, bias=None,
                           return_probs=False):
    """Gradients of one (batch, head) slice, float64.

    With P from ``attention_probs_head_ref`` and c the float32 scale widened:
        dV = P^T dO
        dP = dO V^T
        dS = P * (dP - rowsum(P * dP))      (softmax Jacobian, row by row)
        dQ = c dS K,   dK = c dS^T Q.
    Masked entries have P = 0 and therefore dS = 0.

    Returns (dQ, dK, dV) as float64 arrays shaped like q, k, v; with
    ``return_probs`` also P and dS (Nq x Nk).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    c = _scale64(scale)
    P = attention_probs_head_ref(q, k, scale, causal, kv_len=kv_len, bias=bias)
    dV = P.T @ do
    dP = do @ v.T
    dS = P * (dP - np.sum(P * dP, axis=1, keepdims=True))
    dQ = c * (dS @ k)
    dK = c * (dS.T @ q)
    if return_probs:
        return dQ, dK, dV, P, dS
    return dQ, dK, dV


def attention_bwd_ref(q, k, v, do, scale, causal, heads=None, kv_len=None):
    """Gradients over [B, H, N, D] tensors, float64.

    ``heads`` selects (b, h) slices; by default all of them (then the results
    are shaped [B, H, N, D], else [len(heads), N, D]).  ``kv_len`` is an optional
    per-batch count of valid keys.
    """
    q, k, v, do = (np.asarray(t) for t in (q, k, v, do))
    B, H, N, D = q.shape
    sel = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    dQ = np.zeros((len(sel), N, D))
    dK = np.zeros((len(sel), N, D))
    dV = np.zeros((len(sel), N, v.shape[3]))
    for i, (b, h) in enumerate(sel):
        dQ[i], dK[i], dV[i] = attention_bwd_head_ref(
            q[b, h], k[b, h], v[b, h], do[b, h], scale, causal,
            kv_len=None if kv_len is None else int(kv_len[b]))
    if heads is None:
        return (dQ.reshape(B, H, N, D), dK.reshape(B, H, N, D),
                dV.reshape(B, H, N, v.shape[3]))
    return dQ, dK, dV


def attention_dq_rows_ref(q, k, v, do, scale, causal, rows):
    """dQ of the given query rows of one (batch, head), float64.

    The same definition as ``attention_bwd_head_ref`` restricted to those rows:
    for row i, P_i = softmax of its scaled, masked scores, dP_i = V dO_i,
    dS_i = P_i * (dP_i - P_i . dP_i), dQ_i = c dS_i K.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    c = _scale64(scale)
    out = np.zeros((len(rows), q.shape[1]))
    for n, i in enumerate(rows):
        s = c * (k @ q[i])
        if causal:
            s[i + 1:] = -np.inf
        m = np.max(s)
        e = np.exp(s - m)
        P = e / np.sum(e)
        dP = v @ do[i]
        dS = P * (dP - np.sum(P * dP))
        out[n] = c * (dS @ k)
    return out

"""Attention oracle: materialised scores, three-pass softmax, float64.

Test infrastructure only (see the package docstring).

Parity status: pinned.  ``attention_ref`` is checked against closed forms
(one key, identical keys, all-ones values, causal row 0), against a joint
permutation of keys and values, against torch's float64 CPU
scaled_dot_product_attention and logsumexp, against a pure-Python scalar brute
force at tiny sizes, and against ``blocked_attention_row_ref`` (the alpha/beta
streaming form), which [Ch6 §6.6] reports to agree with the direct form to about
1e-15.
"""

import math

import numpy as np


def _scale64(scale):
    # The kernel receives the scale as a float32; the oracle uses exactly that
    # value, widened.  (1/sqrt(64) = 0.125 is exact; 1/sqrt(128) is not.)
    return float(np.float32(scale))


def attention_head_ref(q, k, v, scale, causal, query_rows=None, chunk=512, kv_len=None,
                       bias=None):
    """Attention for one (batch, head) slice, float64.

    The definition of [xxqk §4.2] and [Ch6 §6.6] ("naive attention"):
    S = scale * Q K^T; with ``causal`` an additive -inf mask hides key j from
    query i whenever j > i ([xxqk §6.3]: additive -inf, not a 0/1 multiply);
    P = row softmax of S by the three-pass safe form ([Ch6 §6.2]); O = P V.  The
    log-sum-exp of each row is LSE = m + log l ([Ch6 §6.5]), taken over the
    scaled, masked scores.

    The full rows of S are materialised; query rows are merely processed a
    ``chunk`` at a time to bound memory (rows are independent, so this changes
    no arithmetic).

    Parameters
    ----------
    q : (Nq, D), k : (Nk, D), v : (Nk, Dv) arrays, widened to float64.
    scale : float, a multiplier (taken at float32 precision).
    causal : bool.  Query row i may see keys 0..i (same-length Q and K).
    query_rows : optional iterable of absolute query indices to compute.
    kv_len : optional number of valid keys; keys at or past it are hidden
        (key padding, an additive -inf mask on those columns, [xxqk §6.3]).
    bias : optional (Nq, Nk) additive term on the scaled scores, S = scale *
        q.k + bias ([Ch6 §6.7.3]'s fused additive mask, applied to scores).

    Returns
    -------
    O : (len(rows), Dv) float64;  LSE : (len(rows),) float64.
    A row with every key masked gives O = 0 and LSE = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, d = q.shape
    nk = k.shape[0]
    if causal and nq != nk:
        raise ValueError("causal attention here assumes len(Q) == len(K)")
    rows = np.arange(nq) if query_rows is None else np.asarray(list(query_rows), dtype=np.int64)
    s64 = _scale64(scale)
    out = np.zeros((len(rows), v.shape[1]))
    lse = np.full(len(rows), -np.inf)
    key_idx = np.arange(nk)
    for c0 in range(0, len(rows), chunk):
        r = rows[c0:c0 + chunk]
        S = s64 * (q[r] @ k.T)                       # (rows, Nk)
        if bias is not None:
            S = S + np.asarray(bias, dtype=np.float64)[r]
        if kv_len is not None:
            S = np.where(key_idx[None, :] >= int(kv_len), -np.inf, S)
        if causal:
            S = np.where(key_idx[None, :] > r[:, None], -np.inf, S)
        m = np.max(S, axis=1)                         # pass 1
        live = m > -np.inf
        m_safe = np.where(live, m, 0.0)
        E = np.exp(S - m_safe[:, None])               # exp(-inf) = 0
        l = np.sum(E, axis=1)                         # pass 2
        P = np.zeros_like(E)
        P[live] = E[live] / l[live, None]             # pass 3
        out[c0:c0 + len(r)] = P @ v
        with np.errstate(divide="ignore"):
            lse[c0:c0 + len(r)] = np.where(live, m_safe + np.log(np.where(live, l, 1.0)), -np.inf)
    return out, lse


def attention_ref(q, k, v, scale, causal, heads=None, chunk=512, kv_len=None, bias=None):
    """Attention over [B, H, N, D] tensors, float64.

    ``heads`` selects (b, h) slices; by default all of them.  ``kv_len`` is an
    optional per-batch count of valid keys (length B); ``bias`` an optional
    additive term broadcastable to [B, H, N, N].  Returns
    ``O`` of shape (len(heads), N, D) and ``LSE`` of shape (len(heads), N) when
    ``heads`` is given, else (B, H, N, D) and (B, H, N).
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, H, N, D = q.shape
    sel = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    O = np.zeros((len(sel), N, v.shape[3]))
    L = np.zeros((len(sel), N))
    bias_full = None if bias is None else np.broadcast_to(np.asarray(bias, dtype=np.float64),
                                                          (B, H, N, N))
    for i, (b, h) in enumerate(sel):
        O[i], L[i] = attention_head_ref(
            q[b, h], k[b, h], v[b, h], scale, causal, chunk=chunk,
            kv_len=None if kv_len is None else int(kv_len[b]),
            bias=None if bias_full is None else bias_full[b, h])
    if heads is None:
        return O.reshape(B, H, N, v.shape[3]), L.reshape(B, H, N)
    return O, L


def blocked_attention_row_ref(q_row, k, v, scale, block, n_visible=None):
    """Single-query streaming attention in the alpha/beta form of [Ch6 §6.6].

    Self-check only; never compared with the GPU.  The keys are visited ``block``
    rows at a time.  For each block: local scores, their local max m_b, local
    weights exp(S - m_b) and their sum l_b; then m_new = max(m, m_b),
    alpha = e^(m - m_new), beta = e^(m_b - m_new), O <- O alpha + beta (P_b V_b),
    l <- l alpha + beta l_b.  The output is O / l.  ``n_visible`` keeps only the
    first n keys (the causal prefix of a query row).

    Returns (O, LSE) with LSE = m + log l.
    """
    q_row = np.asarray(q_row, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = k.shape[0] if n_visible is None else int(n_visible)
    s64 = _scale64(scale)
    m, l = -math.inf, 0.0
    O = np.zeros(v.shape[1])
    for j in range(0, n, block):
        kb = k[j:min(j + block, n)]
        vb = v[j:min(j + block, n)]
        sb = s64 * (kb @ q_row)
        m_b = float(np.max(sb))
        p_b = np.exp(sb - m_b)
        l_b = float(np.sum(p_b))
        m_new = max(m, m_b)
        alpha = 0.0 if m == -math.inf else math.exp(m - m_new)
        beta = math.exp(m_b - m_new)
        O = O * alpha + beta * (p_b @ vb)
        l = l * alpha + beta * l_b
        m = m_new
    if l == 0.0:
        return np.zeros_like(O), -math.inf
    return O / l, m + math.log(l)

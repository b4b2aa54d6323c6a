"""Row softmax oracle (test infrastructure only; see the package docstring).

Parity status: pinned.  ``softmax_rows_ref`` is checked against the worked
example of [Ch6 §6.3.2], against torch's CPU softmax in float64, against row-sum
and shift-invariance identities, and on the overflow / -inf rows the pages
discuss ([Ch6 §6.2], [Ch6 §6.4]).  The fully -inf row is defined here to give
all zeros; the chapter notes that torch returns NaN (0/0) for it ([Ch6 §6.7.3]),
and the library's contract fixes 0 instead.
"""

import numpy as np


def softmax_rows_ref(x, return_stats=False):
    """Safe softmax of every row of a 2-D array, in float64, three passes.

    Follows [Ch6 §6.2]: subtract the row maximum ``m = max_j x_j``, sum
    ``exp(x_j - m)``, then divide each ``exp(x_i - m)`` by that sum.  This is the
    plain definition of [Ch6 §6.1] made overflow-free; it is the result the
    online recurrence of [Ch6 §6.3] reaches exactly in real arithmetic.

    Entries equal to -inf contribute exp(-inf) = 0.  A row whose entries are all
    -inf has no finite maximum; its output is all zeros, its sum 0 and its
    log-sum-exp -inf.  +inf and NaN inputs are outside the contract and simply
    propagate.

    Parameters
    ----------
    x : array_like, shape (rows, cols)
        Converted to float64 exactly (float32 and bfloat16 values are exactly
        representable in float64).
    return_stats : bool
        Also return the per-row max ``m``, the sum ``s`` and ``lse = m + log s``
        ([Ch6 §6.5]).

    Returns
    -------
    y : ndarray float64, shape (rows, cols)
    (m, s, lse) : three float64 arrays of shape (rows,), when requested.
    """
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2:
        raise ValueError("softmax_rows_ref expects a 2-D array")
    rows, cols = x.shape
    y = np.zeros((rows, cols), dtype=np.float64)
    m_out = np.full(rows, -np.inf)
    s_out = np.zeros(rows)
    for r in range(rows):
        row = x[r]
        if cols == 0:
            continue
        # Pass 1: the maximum.
        m = np.max(row)
        m_out[r] = m
        if m == -np.inf:
            # Every entry masked: defined as an all-zero row.
            continue
        # Pass 2: the denominator relative to m.
        e = np.exp(row - m)
        s = np.sum(e)
        s_out[r] = s
        # Pass 3: each output.
        y[r] = np.exp(row - m) / s
    if not return_stats:
        return y
    with np.errstate(divide="ignore"):
        lse = np.where(s_out > 0, m_out + np.log(np.where(s_out > 0, s_out, 1.0)), -np.inf)
    return y, (m_out, s_out, lse)


def masked_softmax_rows_ref(x, mask=None, row_len=None):
    """Softmax of ``x + mask`` with per-row lengths, float64.

    The fused additive mask of [Ch6 §6.7.3]: each logit becomes
    ``x[r, i] + mask[r % mask_rows, i]`` (a mask of 0 / -inf hides entries, any
    finite value biases them).  With ``row_len``, only the first
    ``row_len[r]`` entries of row r take part (lengths are clamped to
    [0, cols]); the remaining outputs are 0, as for -inf logits.  Then the
    three-pass safe softmax of ``softmax_rows_ref`` is applied.

    Parity status: pinned (tests: a zero mask and full lengths give the
    unmasked result; a -inf mask equals writing -inf into x; a length equals
    truncating the row and zero-padding; broadcast masks equal tiled masks).
    """
    x = np.asarray(x, dtype=np.float64)
    rows, cols = x.shape
    z = x.copy()
    if mask is not None:
        m = np.asarray(mask, dtype=np.float64)
        if m.ndim == 1:
            m = m[None, :]
        z = z + m[np.arange(rows) % m.shape[0]]
    if row_len is not None:
        lens = np.clip(np.asarray(row_len, dtype=np.int64), 0, cols)
        z = np.where(np.arange(cols)[None, :] < lens[:, None], z, -np.inf)
    return softmax_rows_ref(z)


def naive_softmax_rows_f32(x):
    """The unsafe two-pass softmax of [Ch6 §6.1], evaluated in float32.

    Negative control only: no maximum is subtracted, so rows of values near
    1000 overflow to inf/inf = NaN exactly as [Ch6 §6.2] describes.  Tests use it
    to show that the overflow rows really exercise the overflow they are meant
    to.
    """
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        e = np.exp(x)
        s = np.sum(e, axis=1, keepdims=True, dtype=np.float32)
        return e / s

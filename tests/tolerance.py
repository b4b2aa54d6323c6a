"""Tolerance checks shared by the parity tests (no GPU needed to import).

bfloat16 outputs are held to the bound that round-to-nearest-even meets and
truncation does not: |got - ref| <= ulp(ref) / 2 + slack, where ulp(ref) is
the spacing of bfloat16 values at |ref| (8 significant bits: 2^(e - 7) for
2^e <= |ref| < 2^(e + 1)) and the slack covers the float32 arithmetic before
the final rounding.  A float32 result within relative error r of the exact
value, rounded to the nearest bfloat16, is within ulp/2 + r |ref| of it, also
where the two straddle a power of two.  Truncation errs by up to a whole ulp
and exceeds the bound on about half of all values.
"""

import numpy as np

#: Relative slack for the float32 arithmetic ahead of the bfloat16 rounding:
#: 2^-15, at most 1/128 of a bfloat16 ulp.  The row softmax's float32 result
#: is within about 2^-17 relative of the exact value (the largest seen over
#: 8M outputs of the 32768 x 8192 workload): e = 2^((x - m) log2 e) carries
#: the rounding of the product (x - m) log2 e, up to 2^-19 log2 units at
#: |x - m| near 30, the hardware 2^x adds about an ulp, and the row's scale
#: factor and sum a few more.  The slack leaves a factor 4 over that.
BF16_REL_SLACK = 2.0 ** -15


def bf16_ulp(y):
    """Spacing of bfloat16 values at |y| (normal range; 2^-133 below it)."""
    y = np.abs(np.asarray(y, dtype=np.float64))
    e = np.floor(np.log2(np.where(y > 0, y, 1.0)))
    return np.maximum(np.exp2(e - 7), 2.0 ** -133)


def bf16_rne_bound(ref, abs_slack=0.0, rel_slack=BF16_REL_SLACK):
    """Largest error a round-to-nearest-even bfloat16 result may have."""
    ref = np.asarray(ref, dtype=np.float64)
    return 0.5 * bf16_ulp(ref) + rel_slack * np.abs(ref) + abs_slack


def bf16_rne_violations(got, ref, abs_slack=0.0, rel_slack=BF16_REL_SLACK):
    """Boolean array: where |got - ref| exceeds the nearest-even bound."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return np.abs(got - ref) > bf16_rne_bound(ref, abs_slack, rel_slack)


#: Absolute slack of the attention rounding-mode test (O in [4, 8) with equal
#: weights): float32 accumulation of up to ~1000 values below 8 before the
#: division by their count.  Half an ulp there is 2^-6, so the bound stays
#: below the 2e-2 budget for O.
O_ABS_SLACK = 2.0 ** -12

#: Rows of the constant-V test need this many visible keys, so that the
#: rounding errors of P average out far below half a bfloat16 ulp of O.
CONSTANT_V_MIN_KEYS = 128

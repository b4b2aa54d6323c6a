"""The bfloat16 bound of the parity tests has teeth (CPU only).

The bound (tests/tolerance.py) must accept the oracle's own values rounded to
nearest even and reject the same values truncated, so that a kernel that
truncated its bfloat16 outputs (softmax y, attention O) would fail the GPU
parity tests.  The same check runs on the attention output of the
rounding-mode test (values in [4, 8), where a truncated O also leaves the
2e-2 budget).
"""

import numpy as np
import torch

import osm_inputs
from oracle import attention_ref, softmax_rows_ref
from tolerance import CONSTANT_V_MIN_KEYS, O_ABS_SLACK, bf16_rne_bound, bf16_rne_violations, bf16_ulp


def _rne(y):
    return torch.from_numpy(np.asarray(y, dtype=np.float64)).float().to(torch.bfloat16) \
        .double().numpy()


def _truncate(y):
    bits = torch.from_numpy(np.asarray(y, dtype=np.float64)).float().view(torch.int32)
    return (bits & -65536).view(torch.float32).double().numpy()


def test_ulp_values():
    assert bf16_ulp(1.0) == 2.0 ** -7
    assert bf16_ulp(1.99) == 2.0 ** -7
    assert bf16_ulp(0.5) == 2.0 ** -8
    assert bf16_ulp(6.0) == 2.0 ** -5
    assert bf16_ulp(-3.0) == 2.0 ** -6
    # One ulp is the gap between a value and the next bfloat16 above it.
    x = torch.tensor([1.0, 3.0, 0.75], dtype=torch.bfloat16)
    nxt = torch.nextafter(x.float(), torch.tensor(10.0)).to(torch.bfloat16)
    assert nxt.double().numpy().tolist() == [1.0, 3.0, 0.75]  # float32 step rounds back
    up = (x.view(torch.int16) + 1).view(torch.bfloat16).double().numpy()
    assert np.allclose(up - x.double().numpy(), bf16_ulp(x.double().numpy()))


def test_softmax_bound_accepts_nearest_even_and_rejects_truncation():
    x = osm_inputs.softmax_rows(64, 8192, seed=2, sigma=4.0, ninf_prob=0.01)
    ref = softmax_rows_ref(x.to(torch.bfloat16).double().numpy())
    assert not bf16_rne_violations(_rne(ref), ref).any()
    bad = bf16_rne_violations(_truncate(ref), ref)
    live = ref > 0
    assert bad[live].mean() > 0.4, bad[live].mean()
    # The old bound of one whole ulp could not tell the two apart.
    assert (np.abs(_truncate(ref) - ref) <= bf16_ulp(ref)).all()


def test_float32_error_inside_the_slack_passes():
    # A float32 result up to 2^-17 off, then rounded to nearest even, stays
    # inside the bound (the slack is 2^-15 relative).
    rng = np.random.default_rng(3)
    ref = np.exp(rng.uniform(-60, 0, 200000))
    noisy = ref * (1 + rng.uniform(-2.0 ** -17, 2.0 ** -17, ref.shape))
    assert not bf16_rne_violations(_rne(noisy), ref).any()


def test_attention_rounding_case_has_teeth():
    # The GPU rounding-mode case: Q = 0, so every visible key weighs the same,
    # and V in [4, 8), so O lies in [4, 8) where the bfloat16 ulp is 2^-5.
    B, H, N, D = 1, 2, 300, 64
    q, k, v = osm_inputs.attention_rounding_inputs(B, H, N, D, seed=41)
    for causal in (False, True):
        O, _ = attention_ref(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                             0.125, causal)
        assert O.min() >= 4.0 and O.max() < 8.0
        assert not bf16_rne_violations(_rne(O), O, abs_slack=O_ABS_SLACK).any()
        trunc_err = np.abs(_truncate(O) - O)
        assert bf16_rne_violations(_truncate(O), O, abs_slack=O_ABS_SLACK).mean() > 0.3
        # Truncation also leaves the general 2e-2 budget for O; RNE stays in it.
        assert trunc_err.max() > 2e-2
        assert np.abs(_rne(O) - O).max() <= 2.0 ** -6 + 1e-12  # ties: exactly half an ulp
        assert (bf16_rne_bound(O, abs_slack=O_ABS_SLACK) < 2e-2).all()


def _o_with_rounded_p(q, k, v, scale, causal, rounding):
    """O with every weight rounded to bfloat16 before the product, in float64
    apart from that rounding (a model of the kernel's P, for the teeth test
    only): P = e^(S - max) as float32, rounded, O = (P V) / sum of unrounded P."""
    S = scale * (q @ k.T)
    if causal:
        S = np.where(np.arange(S.shape[1])[None, :] > np.arange(S.shape[0])[:, None], -np.inf, S)
    P = np.exp(S - S.max(axis=1, keepdims=True))
    return (rounding(P) @ v) / P.sum(axis=1, keepdims=True)


def test_constant_v_case_has_teeth():
    # The GPU case for the rounding of P: with every key row of V equal to c,
    # O = c exactly whatever the weights, and the kernel's O rounds back to c
    # when P is rounded to nearest even (errors average out over the keys),
    # but not when P is truncated (every weight loses 0.28% on average).
    N, D = 1024, 64
    q, k, v = osm_inputs.attention_constant_v_inputs(1, 1, N, D, seed=43)
    q, k, v = (t[0, 0].double().numpy() for t in (q, k, v))
    for causal in (False, True):
        rows = slice(CONSTANT_V_MIN_KEYS - 1, None) if causal else slice(None)
        o_rne = _o_with_rounded_p(q, k, v, 0.125, causal, _rne)[rows]
        o_trunc = _o_with_rounded_p(q, k, v, 0.125, causal, _truncate)[rows]
        c = v[0]
        assert (_rne(o_rne) == c).all()
        assert (_rne(o_trunc) != c).mean() > 0.5

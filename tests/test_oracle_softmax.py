"""Pins for the row-softmax oracle against what the pages and mathematics fix.

CPU only.  The oracle is checked against: the worked example printed in
Ch.6 §6.3.2 (golden fixture), torch's float64 CPU softmax (a library routine
for the same definition), row sums, shift invariance (Ch.6 §6.2), the overflow
rows (Ch.6 §6.2), and the -inf rows of Ch.6 §6.4.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import naive_softmax_rows_f32, softmax_rows_ref
import osm_inputs


def _golden(golden_dir):
    with open(os.path.join(golden_dir, "worked_example_ch6_6_3_2.json")) as f:
        return json.load(f)


def test_worked_example_matches_printed_values(golden_dir):
    g = _golden(golden_dir)
    y, (m, s, lse) = softmax_rows_ref(np.array([g["x"]]), return_stats=True)
    tol = g["abs_tolerance"]
    assert m[0] == g["m"]
    assert abs(s[0] - g["sum"]) <= tol["sum"]
    np.testing.assert_allclose(y[0], g["y"], atol=tol["y"], rtol=0)
    # The individual exponentials the page prints.
    np.testing.assert_allclose(np.exp(np.array(g["x"]) - m[0]), g["exp_terms"], atol=tol["exp_terms"], rtol=0)
    # LSE = m + log(l) (Ch.6 §6.5) for the same row.
    assert abs(lse[0] - (5.0 + math.log(s[0]))) < 1e-15


def test_worked_example_closed_form():
    # Independent closed form: y = (e^-4, 1, e^-2) / (e^-4 + 1 + e^-2).
    d = math.exp(-4) + 1 + math.exp(-2)
    want = [math.exp(-4) / d, 1 / d, math.exp(-2) / d]
    y = softmax_rows_ref(np.array([[1.0, 5.0, 3.0]]))
    np.testing.assert_allclose(y[0], want, rtol=1e-15, atol=0)


def _special_matrix():
    return osm_inputs.softmax_small()["x"].double().numpy()


def test_agrees_with_torch_softmax_float64():
    x = _special_matrix()
    y = softmax_rows_ref(x)
    ref = torch.softmax(torch.from_numpy(x[:60]), dim=1).numpy()
    np.testing.assert_allclose(y[:60], ref, atol=1e-15, rtol=0)
    # Short rows, as a separate call (cols = 100).
    xs = x[62:64, :100]
    np.testing.assert_allclose(softmax_rows_ref(xs), torch.softmax(torch.from_numpy(xs), 1).numpy(),
                               atol=1e-15, rtol=0)


def test_rows_sum_to_one_and_shift_invariance():
    x = _special_matrix()[:60]
    y = softmax_rows_ref(x)
    np.testing.assert_allclose(y.sum(axis=1), 1.0, atol=1e-12, rtol=0)
    for c in (1000.0, -1000.0):
        y2 = softmax_rows_ref(x[:48] + c)
        np.testing.assert_allclose(y2, y[:48], atol=1e-12, rtol=0)


def test_overflow_rows_are_finite_and_naive_form_is_not():
    x = _special_matrix()[48:56]
    assert x.min() > 900
    y = softmax_rows_ref(x)
    assert np.isfinite(y).all()
    np.testing.assert_allclose(y.sum(axis=1), 1.0, atol=1e-12)
    # Negative control (Ch.6 §6.1-6.2): without the max subtraction, float32
    # overflows to inf/inf = NaN on exactly these rows.
    naive = naive_softmax_rows_f32(x.astype(np.float32))
    assert np.isnan(naive).all()
    # ... while it is fine on the ordinary rows.
    ok = naive_softmax_rows_f32(_special_matrix()[:48].astype(np.float32))
    assert np.isfinite(ok).all()


def test_masked_rows():
    x = _special_matrix()
    y = softmax_rows_ref(x)
    # Rows 56-59: first 300 entries -inf -> exact zeros there; the rest is the
    # softmax of the unmasked part.
    assert (y[56:60, :300] == 0.0).all()
    np.testing.assert_allclose(y[56:60, 300:], softmax_rows_ref(x[56:60, 300:]), atol=1e-15)
    np.testing.assert_allclose(y[56:60].sum(axis=1), 1.0, atol=1e-12)
    # Rows 60-61: every entry -inf -> all zeros (the library contract; torch
    # would give NaN, Ch.6 §6.7.3).
    assert (y[60:62] == 0.0).all()
    assert np.isnan(torch.softmax(torch.from_numpy(x[60:62]), 1).numpy()).all()


def test_single_and_empty_columns():
    y, (m, s, lse) = softmax_rows_ref(np.array([[7.5], [-np.inf]]), return_stats=True)
    assert y[0, 0] == 1.0 and y[1, 0] == 0.0
    assert lse[0] == 7.5 and lse[1] == -np.inf
    assert softmax_rows_ref(np.zeros((3, 0))).shape == (3, 0)


def test_lse_matches_torch_logsumexp():
    x = _special_matrix()[:60]
    _, (m, s, lse) = softmax_rows_ref(x, return_stats=True)
    np.testing.assert_allclose(lse, torch.logsumexp(torch.from_numpy(x), 1).numpy(), rtol=1e-14)
    np.testing.assert_array_equal(m, x.max(axis=1))


@pytest.mark.parametrize("seed", [0, 1])
def test_bandwidth_workload_rows_against_torch(seed):
    # A slice of the 4*N(0,1), 1%-(-inf) distribution used at bandwidth scale.
    x = osm_inputs.softmax_rows(16, 8192, seed=seed).double().numpy()
    assert np.isneginf(x).any()
    # 8192-term sums: the two summation orders differ by a few float64 ulps.
    np.testing.assert_allclose(softmax_rows_ref(x), torch.softmax(torch.from_numpy(x), 1).numpy(),
                               atol=1e-14, rtol=0)

"""Pins of the float64 backward oracle (oracle/kata_backward.py).

The pages give no backward pass, so the pins are the calculus of the forward they define:
central finite differences of the (already pinned) forward oracles in float64, and exact
identities of the forward: its invariance to the scale of every query and key row
(normalisation onto the unit sphere, rank-one lift paragraph) makes each row's gradient
orthogonal to the row, and the convex-combination readout (normalized-readout paragraph)
makes the value gradients of a row sum to its output gradient.
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import kata_backward as kb
from oracle import kata_families as kf

RNG = np.random.default_rng(2024)


def _loss(q, k, v, go, family, g):
    return float(np.sum(kf.naive_family(q, k, v, family, g) * go))


@pytest.mark.parametrize("family,g", [("full", 1), ("sigma", 2), ("block", 2), ("sigma", 3)])
def test_central_finite_differences(family, g):
    T, p, dv = 7, 6, 3
    q, k, v, go = (RNG.standard_normal(s) for s in ((2, T, p), (2, T, p), (2, T, dv), (2, T, dv)))
    dq, dk, dv_ = kb.backward(q, k, v, go, family, g)
    h = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv_)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            x[idx] += h
            lp = _loss(q, k, v, go, family, g)
            x[idx] -= 2 * h
            lm = _loss(q, k, v, go, family, g)
            x[idx] += h
            num[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(num - grad)) / max(1e-12, np.max(np.abs(grad)))
        assert err < 1e-6, (name, err)


@pytest.mark.parametrize("family,g", [("full", 1), ("sigma", 2), ("block", 4)])
def test_scale_invariance_and_value_sums(family, g):
    T, p, dv = 40, 8, 5
    q, k, v, go = (RNG.standard_normal(s) for s in ((T, p), (T, p), (T, dv), (T, dv)))
    dq, dk, dv_ = kb.backward(q, k, v, go, family, g)
    # o does not change when any q_t or k_s is rescaled: every row gradient is orthogonal
    np.testing.assert_allclose(np.sum(q * dq, axis=-1), 0.0, atol=1e-12)
    np.testing.assert_allclose(np.sum(k * dk, axis=-1), 0.0, atol=1e-12)
    # o_t is a convex combination of v_1..v_t: sum_s d o_t / d v_s = I
    np.testing.assert_allclose(dv_.sum(axis=0), go.sum(axis=0), rtol=1e-12, atol=1e-12)


def test_zero_rows_and_zero_gradient():
    T, p, dv = 12, 4, 2
    q, k, v, go = (RNG.standard_normal(s) for s in ((T, p), (T, p), (T, dv), (T, dv)))
    q[3] = 0.0
    k[5] = 0.0
    dq, dk, dv_ = kb.backward(q, k, v, go)
    assert np.all(dq[3] == 0.0) and np.all(dk[5] == 0.0)
    # the zero key has weight 0 everywhere, so its value receives no gradient
    assert np.all(dv_[5] == 0.0)
    z = kb.backward(q, k, v, np.zeros_like(go))
    assert all(np.all(t == 0.0) for t in z)

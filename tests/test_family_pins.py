"""Pins of the reduced-family oracle (KATA-Sigma g, KATA-M g) against facts the pages and
mathematics fix, independently of its formulas.

Source: "Kernelized Linear Attention: Breaking the Capacity Wall with Symmetric Cones"
(arXiv 2607.17419), arXiv HTML page: the reduced PSD families paragraph (block split,
the Sigma g and M g feature maps with their inner-product identities, the two state-size
displays, recovery of the full map at g = 1) and Eq. (8) with the d = 64 width printed
next to it; the feature-value state display for the recurrent form.

Each test compares with a hand-computed value, the already pinned full-map oracle, or an
invariant that a wrong block index, a missing cross term or a transposed operand breaks.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import kata_families as kf
from oracle import kata_oracle as ko

RNG = np.random.default_rng(4321)


def test_state_widths_from_the_size_displays():
    # Sigma g: (d/g)(d/g + 1)/2; M g: d (d/g + 1)/2; the full map at d = 64 has 2080
    assert kf.family_dim(64, "full") == 2080
    assert kf.family_dim(64, "sigma", 1) == 2080 and kf.family_dim(64, "block", 1) == 2080
    assert kf.family_dim(64, "sigma", 2) == 528 and kf.family_dim(64, "block", 2) == 1056
    assert kf.family_dim(64, "sigma", 4) == 136 and kf.family_dim(64, "block", 4) == 544
    assert kf.family_dim(32, "sigma", 2) == 136 and kf.family_dim(32, "block", 2) == 272
    with pytest.raises(ValueError):
        kf.family_dim(32, "sigma", 3)


@pytest.mark.parametrize("family", ["sigma", "block"])
def test_g1_is_the_full_map(family):
    u = RNG.standard_normal((5, 7, 12))
    assert np.array_equal(kf.lift_family(u, family, 1), ko.lift(u))
    q, k, v = (RNG.standard_normal((2, 40, 12)) for _ in range(3))
    np.testing.assert_allclose(kf.naive_family(q, k, v, family, 1), ko.naive(q, k, v), rtol=0, atol=1e-13)


def test_worked_example_exact():
    """q = (1,2,3,4), k = (2,0,1,1), g = 2 (blocks of 2). By hand: q1.k1 = 2, q1.k2 = 3,
    q2.k1 = 6, q2.k2 = 7, q.k = 9, |q|^2 = 30, |k|^2 = 6, so the weights are
    Sigma 2: (4+9+36+49)/180 = 49/90; M 2: (4+49)/180 = 53/180; full: 81/180 = 9/20."""
    q = np.array([1.0, 2.0, 3.0, 4.0])
    k = np.array([2.0, 0.0, 1.0, 1.0])
    want = {"sigma": Fraction(49, 90), "block": Fraction(53, 180), "full": Fraction(9, 20)}
    for fam, val in want.items():
        g = 1 if fam == "full" else 2
        through_psi = float(kf.lift_family(q, fam, g) @ kf.lift_family(k, fam, g))
        direct = float(kf.weights_family(ko.normalize(q[None]), ko.normalize(k[None]), fam, g)[0, 0])
        assert abs(through_psi - float(val)) < 1e-15, fam
        assert abs(direct - float(val)) < 1e-15, fam


@pytest.mark.parametrize("family,g", [("sigma", 2), ("sigma", 4), ("block", 2), ("block", 4), ("sigma", 8)])
def test_psi_inner_product_equals_block_dot_products(family, g):
    """<psi(q), psi(k)> through the packed lift equals the displayed sum of squared block
    dot products (two independent constructions: index tables and sqrt(2) vs matmuls)."""
    q, k = RNG.standard_normal((6, 16)), RNG.standard_normal((9, 16))
    via_psi = kf.lift_family(q, family, g) @ kf.lift_family(k, family, g).T
    direct = kf.weights_family(ko.normalize(q), ko.normalize(k), family, g)
    np.testing.assert_allclose(via_psi, direct, rtol=1e-12, atol=1e-15)


def test_cross_block_interaction():
    """q on block 1 only and k on block 2 only: M g sees nothing, Sigma g sees exactly the
    full-map weight of the two m-vectors (pinned full-map oracle)."""
    m = 4
    qa, kb = RNG.standard_normal(m), RNG.standard_normal(m)
    q = np.concatenate([qa, np.zeros(m)])
    k = np.concatenate([np.zeros(m), kb])
    wq, wk = ko.normalize(q[None]), ko.normalize(k[None])
    assert kf.weights_family(wq, wk, "block", 2)[0, 0] == 0.0
    full_m = float(ko.lift(qa) @ ko.lift(kb))
    assert abs(kf.weights_family(wq, wk, "sigma", 2)[0, 0] - full_m) < 1e-14
    # same block: every family reduces to the full map
    k2 = np.concatenate([kb, np.zeros(m)])
    full = float(ko.lift(q) @ ko.lift(k2))
    for fam in ("sigma", "block"):
        assert abs(kf.weights_family(wq, ko.normalize(k2[None]), fam, 2)[0, 0] - full) < 1e-14


def test_invariances_that_tell_the_families_apart():
    g, m = 4, 3
    q, k = RNG.standard_normal((5, g * m)), RNG.standard_normal((7, g * m))
    w = {f: kf.weights_family(ko.normalize(q), ko.normalize(k), f, 1 if f == "full" else g)
         for f in ("full", "sigma", "block")}
    blk = lambda x: x.reshape(x.shape[0], g, m)

    def weights(qq, kk, f):
        return kf.weights_family(ko.normalize(qq), ko.normalize(kk), f, 1 if f == "full" else g)
    # permuting the blocks of q alone: Sigma g (a sum over blocks) does not notice
    qp = blk(q)[:, [2, 0, 3, 1]].reshape(q.shape)
    np.testing.assert_allclose(weights(qp, k, "sigma"), w["sigma"], rtol=1e-12)
    assert not np.allclose(weights(qp, k, "block"), w["block"])
    assert not np.allclose(weights(qp, k, "full"), w["full"])
    # flipping the sign of one block of q: both reduced families square block products
    qs = blk(q).copy(); qs[:, 1] *= -1; qs = qs.reshape(q.shape)
    np.testing.assert_allclose(weights(qs, k, "sigma"), w["sigma"], rtol=1e-12)
    np.testing.assert_allclose(weights(qs, k, "block"), w["block"], rtol=1e-12)
    assert not np.allclose(weights(qs, k, "full"), w["full"])
    # independent rotation of each block of both q and k: M g keeps every block product
    R = [np.linalg.qr(RNG.standard_normal((m, m)))[0] for _ in range(g)]
    rot = lambda x: np.stack([blk(x)[:, a] @ R[a].T for a in range(g)], axis=1).reshape(x.shape)
    np.testing.assert_allclose(weights(rot(q), rot(k), "block"), w["block"], rtol=1e-12)
    assert not np.allclose(weights(rot(q), rot(k), "sigma"), w["sigma"])
    # one common rotation of every block: Sigma g keeps every cross product too
    rot1 = lambda x: (blk(x) @ R[0].T).reshape(x.shape)
    np.testing.assert_allclose(weights(rot1(q), rot1(k), "sigma"), w["sigma"], rtol=1e-12)


@pytest.mark.parametrize("family,g", [("sigma", 2), ("block", 2), ("sigma", 4), ("block", 4)])
def test_recurrent_equals_definition_and_decode_continues(family, g):
    """The psi-state recurrence equals the definition; a prefill state plus decode steps
    continues it (feature-value state display)."""
    q, k, v = RNG.standard_normal((2, 30, 8)), RNG.standard_normal((2, 30, 8)), RNG.standard_normal((2, 30, 3))
    k[0, 4] = 0.0
    ref = kf.naive_family(q, k, v, family, g)
    np.testing.assert_allclose(kf.recurrent_family(q, k, v, family, g), ref, rtol=1e-11, atol=1e-13)
    T0 = 21
    S0, Z0 = kf.prefill_state_family(k[:, :T0], v[:, :T0], family, g)
    mv = lambda x: np.moveaxis(x[:, T0:], 1, 0)
    outs, _, _ = kf.decode_steps_family(S0, Z0, mv(q), mv(k), mv(v), family, g)
    np.testing.assert_allclose(np.moveaxis(outs, 0, 1), ref[:, T0:], rtol=1e-11, atol=1e-13)


def test_weights_nonnegative_and_outputs_in_hull():
    q, k, v = RNG.standard_normal((40, 8)), RNG.standard_normal((40, 8)), RNG.standard_normal((40, 2))
    for fam, g in (("sigma", 2), ("block", 4)):
        w = kf.weights_family(ko.normalize(q), ko.normalize(k), fam, g)
        assert (w >= 0).all()
        o = kf.naive_family(q, k, v, fam, g)
        for t in range(40):
            assert (o[t] >= v[: t + 1].min(0) - 1e-12).all() and (o[t] <= v[: t + 1].max(0) + 1e-12).all()


# ------------------------------------------------------------------ higher even orders
def test_order_dims_and_r1_is_the_full_map():
    # binom(p + 2r - 1, 2r): by hand, p=4 r=2 -> binom(7, 4) = 35; p=16 r=2 -> 3876
    assert kf.order_dim(4, 2) == 35 and kf.order_dim(16, 2) == 3876 and kf.order_dim(3, 3) == 28
    assert kf.order_dim(64, 1) == 2080
    u = RNG.standard_normal((6, 9))
    np.testing.assert_array_equal(kf.lift_order(u, 1), ko.lift(u))


def test_order_worked_example_p2_r2():
    """u = (a, b) on the circle: psi_4 = (a^4, 2a^3 b, sqrt(6) a^2 b^2, 2 a b^3, b^4) (the
    multinomial coefficients 1, 4, 6, 4, 1 under square roots)."""
    a, b = 0.6, 0.8
    want = [a ** 4, 2 * a ** 3 * b, math.sqrt(6) * a ** 2 * b ** 2, 2 * a * b ** 3, b ** 4]
    np.testing.assert_allclose(kf.lift_order(np.array([a, b]), 2), want, rtol=0, atol=1e-15)


@pytest.mark.parametrize("p,r", [(3, 2), (4, 2), (5, 3), (2, 4)])
def test_order_identities(p, r):
    """||psi_2r(u_hat)|| = 1 and <psi_2r(u), psi_2r(v)> = (u_hat . v_hat)^{2r}; the weights of
    the naive form equal the packed inner products."""
    u, v = RNG.standard_normal((7, p)), RNG.standard_normal((5, p))
    fu, fv = kf.lift_order(u, r), kf.lift_order(v, r)
    np.testing.assert_allclose(np.linalg.norm(fu, axis=-1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(fu @ fv.T, (ko.normalize(u) @ ko.normalize(v).T) ** (2 * r), rtol=1e-12, atol=1e-15)
    q, k, vv = RNG.standard_normal((12, p)), RNG.standard_normal((12, p)), RNG.standard_normal((12, 2))
    fq, fk = kf.lift_order(q, r), kf.lift_order(k, r)
    w = np.tril(fq @ fk.T)
    ref = (w @ vv) / w.sum(axis=-1, keepdims=True)
    np.testing.assert_allclose(kf.naive_order(q, k, vv, r), ref, rtol=1e-11)

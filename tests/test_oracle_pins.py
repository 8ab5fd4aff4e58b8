"""Pins of the float64 oracle against facts fixed by the pages and by mathematics.

Source: "Kernelized Linear Attention: Breaking the Capacity Wall with Symmetric Cones"
(arXiv 2607.17419), arXiv HTML page: Eq. (8) (packed width), the rank-one lift display
(norm and inner-product identities), Assumption 1 (nonnegative weights) and the
normalized-readout paragraph (convex interpolation), Assumption 2 (isometric
invariance), the feature-value state display, the chunked-forward paragraph (chunk
algebra, associative prefix), and the Idealized Welch-scale retrieval theorem,
Eqs. (11)-(12).

None of these re-types the oracle's formula: each compares it with an independent
value (hand-written fixture, exact rational arithmetic, closed form, textbook routine,
or an invariant that a wrong sign, index, exponent or operand would break).
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import kata_oracle as ko
from kata_inputs import round_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            i, j, expr = line.split(maxsplit=2)
            val = eval(expr, {"__builtins__": {}}, {"sqrt": math.sqrt})
            rows.append((int(i), int(j), float(val)))
    return rows


# ---------------------------------------------------------------- packed width (Eq. 8)
def test_packed_dim_values_printed_on_page():
    # the page prints: at d = 64 the direct outer-product width is 4096, packed 2080
    assert ko.packed_dim(64) == 2080
    assert 64 * 64 == 4096
    # symmetric ambient dimension binom(p + 2r - 1, 2r) of the even-order family at r = 1
    for p in (1, 2, 3, 16, 32, 64):
        assert ko.packed_dim(p) == math.comb(p + 1, 2)
        assert len(ko.packed_pairs(p)[0]) == ko.packed_dim(p)
    with pytest.raises(ValueError):
        ko.packed_dim(0)


# ---------------------------------------------------------------- lift: index map + values
@pytest.mark.parametrize("name,u", [("lift_p3.txt", [1.0, 2.0, 2.0]),
                                    ("lift_p3_neg.txt", [-2.0, 0.0, 6.0, 3.0])])
def test_lift_worked_example(name, u):
    rows = _read_golden(name)
    psi = ko.lift(np.asarray(u))
    ii, jj = ko.packed_pairs(len(u))
    assert len(rows) == len(psi)
    for pos, (i, j, val) in enumerate(rows):
        assert (ii[pos], jj[pos]) == (i, j)
        assert psi[pos] == pytest.approx(val, abs=1e-15)


def test_lift_basis_vectors_place_single_entries():
    p = 5
    ii, jj = ko.packed_pairs(p)
    for i in range(p):
        e = np.zeros(p)
        e[i] = 3.0  # any positive scale: the lift normalises first
        psi = ko.lift(e)
        assert np.count_nonzero(psi) == 1
        pos = int(np.flatnonzero(psi)[0])
        assert (ii[pos], jj[pos]) == (i, i) and psi[pos] == 1.0
    for i in range(p):
        for j in range(i + 1, p):
            u = np.zeros(p)
            u[i] = u[j] = 1.0
            psi = ko.lift(u)
            nz = {(int(ii[x]), int(jj[x])): psi[x] for x in np.flatnonzero(psi)}
            assert set(nz) == {(i, i), (j, j), (i, j)}
            assert nz[(i, i)] == pytest.approx(0.5) and nz[(j, j)] == pytest.approx(0.5)
            assert nz[(i, j)] == pytest.approx(1 / math.sqrt(2))


def test_lift_norm_and_inner_product_identities():
    for p in (3, 16, 32, 64):
        a = RNG.standard_normal((50, p))
        b = RNG.standard_normal((50, p))
        fa, fb = ko.lift(a), ko.lift(b)
        assert np.allclose(np.linalg.norm(fa, axis=-1), 1.0, atol=1e-14)
        ah = a / np.linalg.norm(a, axis=-1, keepdims=True)
        bh = b / np.linalg.norm(b, axis=-1, keepdims=True)
        # Frobenius inner product of the unpacked outer products, via the trace
        frob = np.array([np.trace(np.outer(x, x) @ np.outer(y, y)) for x, y in zip(ah, bh)])
        assert np.allclose(np.sum(fa * fb, axis=-1), frob, atol=1e-13)
        assert np.all(np.sum(fa * fb, axis=-1) >= -1e-15)


def test_lift_zero_vector_is_zero():
    assert np.all(ko.lift(np.zeros(8)) == 0.0)


# ---------------------------------------------------------------- exact rational brute force
# Unit vectors with rational coordinates (Pythagorean quadruples) so that the whole
# forward can be done exactly with Fractions in plain Python.
_QUADS = [(1, 2, 2, 3), (2, 3, 6, 7), (1, 4, 8, 9), (2, 6, 9, 11), (4, 4, 7, 9),
          (6, 6, 7, 11), (2, 10, 11, 15), (1, 12, 12, 17), (8, 9, 12, 17), (3, 4, 12, 13)]


def _rational_unit_vectors(T, seed):
    rng = np.random.default_rng(seed)
    ints, fracs = [], []
    for _ in range(T):
        a, b, c, d = _QUADS[rng.integers(len(_QUADS))]
        comp = [a, b, c]
        perm = rng.permutation(3)
        signs = rng.choice([-1, 1], size=3)
        vec = [int(signs[x] * comp[perm[x]]) for x in range(3)]
        scale = int(rng.integers(1, 4))           # non-unit input: the forward normalises
        ints.append([scale * x for x in vec])
        fracs.append([Fraction(x, d) for x in vec])
    return np.asarray(ints, dtype=np.float64), fracs


def _exact_forward(qf, kf, vint):
    T = len(qf)
    out = []
    for t in range(T):
        num = [Fraction(0)] * len(vint[0])
        den = Fraction(0)
        for s in range(t + 1):
            dot = sum(x * y for x, y in zip(qf[t], kf[s]))
            w = dot * dot
            den += w
            num = [nv + w * Fraction(int(vv)) for nv, vv in zip(num, vint[s])]
        out.append([float(x / den) if den != 0 else 0.0 for x in num])
    return np.asarray(out)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_forms_match_exact_rational_forward(seed):
    T = 9
    q, qf = _rational_unit_vectors(T, 100 + seed)
    k, kf = _rational_unit_vectors(T, 200 + seed)
    v = np.random.default_rng(300 + seed).integers(-5, 6, size=(T, 2)).astype(np.float64)
    exact = _exact_forward(qf, kf, v)
    assert np.allclose(ko.naive(q, k, v), exact, rtol=1e-12, atol=1e-12)
    assert np.allclose(ko.recurrent(q, k, v), exact, rtol=1e-12, atol=1e-12)
    for C in (1, 2, 4, 5):
        for scan in ("sequential", "associative"):
            assert np.allclose(ko.chunked(q, k, v, C, scan), exact, rtol=1e-12, atol=1e-12)
    assert np.allclose(ko.naive_rows(q, k, v, [0, 4, 8]), exact[[0, 4, 8]], atol=1e-12)


# ---------------------------------------------------------------- special cases
def test_first_token_returns_its_value():
    q, k, v = RNG.standard_normal((3, 4, 7, 5)), RNG.standard_normal((3, 4, 7, 5)), RNG.standard_normal((3, 4, 7, 6))
    for f in (ko.naive(q, k, v), ko.recurrent(q, k, v), ko.chunked(q, k, v, 3)):
        assert np.allclose(f[..., 0, :], v[..., 0, :], atol=1e-14)


def test_p1_and_identical_keys_give_cumulative_mean():
    T, dv = 40, 3
    v = RNG.standard_normal((T, dv))
    cummean = np.cumsum(v, axis=0) / np.arange(1, T + 1)[:, None]
    # p = 1: every weight is (+-1)^2 = 1
    q1 = RNG.standard_normal((T, 1))
    k1 = RNG.standard_normal((T, 1))
    assert np.allclose(ko.naive(q1, k1, v), cummean, atol=1e-13)
    # every key equal to every query direction (up to sign and scale): weights all 1
    d = RNG.standard_normal(8)
    qs = d[None, :] * RNG.choice([-2.0, 0.5, 3.0], size=(T, 1))
    ks = d[None, :] * RNG.choice([-1.0, 1.5], size=(T, 1))
    assert np.allclose(ko.naive(qs, ks, v), cummean, atol=1e-13)
    assert np.allclose(ko.recurrent(qs, ks, v), cummean, atol=1e-13)


def test_orthonormal_keys_select_one_value():
    p, dv = 6, 4
    k = np.eye(p)                       # key at position s is e_s
    v = RNG.standard_normal((p, dv))
    for t in range(p):
        for j in range(t + 1):
            q = RNG.standard_normal((p, p))
            q[t] = 0.0
            q[t, j] = -2.5              # query e_j (sign and scale do not matter)
            o = ko.naive(q, k, v)
            assert np.allclose(o[t], v[j], atol=1e-14)
            assert np.allclose(ko.recurrent(q, k, v)[t], v[j], atol=1e-14)


def test_zero_query_or_zero_denominator_gives_zero_row():
    q = RNG.standard_normal((5, 4)); k = RNG.standard_normal((5, 4)); v = RNG.standard_normal((5, 3))
    q[2] = 0.0
    for f in (ko.naive, ko.recurrent):
        assert np.all(f(q, k, v)[2] == 0.0)
    # a query orthogonal to every key so far has denominator 0
    k2 = np.zeros((3, 4)); k2[:, 0] = 1.0
    q2 = np.zeros((3, 4)); q2[:, 1] = 1.0
    assert np.all(ko.naive(q2, k2, np.ones((3, 2))) == 0.0)


# ---------------------------------------------------------------- invariants
def test_outputs_lie_in_convex_hull_of_past_values():
    q, k, v = RNG.standard_normal((2, 64, 8)), RNG.standard_normal((2, 64, 8)), RNG.standard_normal((2, 64, 5))
    o = ko.naive(q, k, v)
    lo = np.minimum.accumulate(v, axis=-2)
    hi = np.maximum.accumulate(v, axis=-2)
    assert np.all(o >= lo - 1e-12) and np.all(o <= hi + 1e-12)


def test_isometric_sign_and_scale_invariance():
    T, p, dv = 48, 8, 5
    q, k, v = RNG.standard_normal((T, p)), RNG.standard_normal((T, p)), RNG.standard_normal((T, dv))
    U, _ = np.linalg.qr(RNG.standard_normal((p, p)))
    base = ko.naive(q, k, v)
    assert np.allclose(ko.naive(q @ U.T, k @ U.T, v), base, atol=1e-12)
    sq = RNG.choice([-3.0, -0.5, 0.25, 2.0], size=(T, 1))
    sk = RNG.choice([-1.0, 4.0, 0.1], size=(T, 1))
    assert np.allclose(ko.naive(q * sq, k * sk, v), base, atol=1e-12)
    # the output is not invariant under exchanging the roles of q and k (causal order)
    assert not np.allclose(ko.naive(k, q, v), base, atol=1e-3)


# ---------------------------------------------------------------- Idealized Welch-scale retrieval
def test_psnr_closed_form_eq12():
    p, T = 4, 16
    eps = (T - p) / (p * (T - 1))
    assert eps == pytest.approx(0.2)
    star = 5                                  # position of the matched key
    e1 = np.zeros(p); e1[0] = 1.0
    keys = np.zeros((T, p))
    for j in range(T):
        if j == star:
            keys[j] = e1
        else:
            w = RNG.standard_normal(p); w[0] = 0.0; w /= np.linalg.norm(w)
            keys[j] = math.sqrt(eps) * e1 + math.sqrt(1 - eps) * w
    vals = np.eye(T)                          # orthonormal values, d_v = T
    qs = RNG.standard_normal((T, p)); qs[-1] = e1   # the query of interest is at position T
    o = ko.naive(qs, keys, vals)[-1]
    psnr = o[star] ** 2 / (np.sum(o ** 2) - o[star] ** 2)
    assert psnr == pytest.approx(p * p * (T - 1) / (T - p) ** 2, rel=1e-10)   # Eq. (12)
    assert psnr == pytest.approx(1 / ((T - 1) * eps ** 2), rel=1e-10)
    assert psnr == pytest.approx(5 / 3, rel=1e-10)
    # a first-order (linear) readout of the same geometry gives Eq. (11) instead
    a = keys @ e1
    lin = a[star] ** 2 / (np.sum(a ** 2) - a[star] ** 2)
    assert lin == pytest.approx(p / (T - p), rel=1e-10)


# ---------------------------------------------------------------- chunk and scan algebra
def _state_form_bound(q, k, v):
    """Rounding bound for a state-form row against the definition.

    The state forms get each weight as the inner product of two packed lifts, a sum of
    n = p(p+1)/2 terms of both signs whose absolute values sum to at most
    ||psi(q^)|| ||psi(k^)|| = 1, so each weight carries an absolute error of about n*eps,
    however small (q^.k^)^2 is. Row t therefore errs by up to about
    n * eps * (t + 1) * max|v| / D_t, with D_t the row's exact denominator; a row whose
    weights are all tiny (t = 0 with q^ nearly orthogonal to k^) has a large bound.
    """
    qn = q / np.linalg.norm(q, axis=-1, keepdims=True)
    kn = k / np.linalg.norm(k, axis=-1, keepdims=True)
    T, p = q.shape[-2], q.shape[-1]
    w = np.tril(np.einsum("...tp,...sp->...ts", qn, kn) ** 2)
    D = w.sum(-1)
    n = p * (p + 1) // 2
    t1 = np.arange(1, T + 1, dtype=np.float64)
    return 64 * n * np.finfo(np.float64).eps * (t1 * np.abs(v).max(axis=(-2, -1), keepdims=False)[..., None] / D)[..., None]


@pytest.mark.parametrize("C", [1, 7, 32, 64])
def test_chunked_equals_naive_for_any_chunk(C):
    rng = np.random.default_rng(4100 + C)
    q, k, v = rng.standard_normal((2, 3, 150, 8)), rng.standard_normal((2, 3, 150, 8)), rng.standard_normal((2, 3, 150, 4))
    ref = ko.naive(q, k, v)
    tol = 1e-13 + _state_form_bound(q, k, v)
    for scan in ("sequential", "associative"):
        assert np.all(np.abs(ko.chunked(q, k, v, C, scan) - ref) <= tol)
    assert np.all(np.abs(ko.recurrent(q, k, v) - ref) <= tol)
    # the bound is tight enough to matter: a dropped token or a wrong sign exceeds it
    assert np.median(tol) < 1e-10


def test_hillis_steele_matches_cumsum():
    x = RNG.standard_normal((37, 3, 2))
    exc = ko._hillis_steele_exclusive(x)
    ref = np.concatenate([np.zeros((1, 3, 2)), np.cumsum(x, axis=0)[:-1]])
    assert np.allclose(exc, ref, atol=1e-13)


def test_decode_matches_prefix_forward():
    H, Th, Ts, p, dv = 3, 20, 6, 5, 4
    k_hist, v_hist = RNG.standard_normal((H, Th, p)), RNG.standard_normal((H, Th, dv))
    q_s, k_s, v_s = RNG.standard_normal((Ts, H, p)), RNG.standard_normal((Ts, H, p)), RNG.standard_normal((Ts, H, dv))
    S0, Z0 = ko.prefill_state(k_hist, v_hist)
    # state identities: Z = sum of lifts, trace-like check on the diagonal entries
    ii, jj = ko.packed_pairs(p)
    kh = k_hist / np.linalg.norm(k_hist, axis=-1, keepdims=True)
    assert np.allclose(Z0[:, ii == jj].sum(axis=-1), Th)          # sum_s ||k_hat_s||^2
    o, S, Z = ko.decode_steps(S0, Z0, q_s, k_s, v_s)
    # full forward over history + steps, with dummy history queries
    q_all = np.concatenate([RNG.standard_normal((H, Th, p)), np.swapaxes(q_s, 0, 1)], axis=1)
    k_all = np.concatenate([k_hist, np.swapaxes(k_s, 0, 1)], axis=1)
    v_all = np.concatenate([v_hist, np.swapaxes(v_s, 0, 1)], axis=1)
    ref = ko.naive(q_all, k_all, v_all)[:, Th:]
    assert np.allclose(np.swapaxes(o, 0, 1), ref, rtol=1e-11, atol=1e-12)
    S_ref, Z_ref = ko.prefill_state(k_all, v_all)
    assert np.allclose(S, S_ref, atol=1e-11) and np.allclose(Z, Z_ref, atol=1e-11)
    # from an empty state the first step returns its own value
    o1, _, _ = ko.decode_steps(np.zeros_like(S0), np.zeros_like(Z0), q_s[:1], k_s[:1], v_s[:1])
    assert np.allclose(o1[0], v_s[0], atol=1e-14)


# ---------------------------------------------------------------- helpers
def test_row_rel_err():
    r = np.array([[1.0, -2.0], [0.0, 0.0]])
    assert ko.row_rel_err(r, r) == 0.0
    g = np.array([[1.0, -2.2], [0.0, 0.0]])
    assert ko.row_rel_err(g, r) == pytest.approx(0.1)
    g2 = np.array([[1.0, -2.0], [1e-30, 0.0]])
    assert ko.row_rel_err(g2, r) == float("inf")
    assert ko.row_rel_err(np.array([[np.nan, 0.0]]), np.array([[1.0, 0.0]])) == float("inf")


def test_round_bf16_known_patterns():
    x = np.array([1.0, 1 + 2**-8, 1 + 3 * 2**-8, 1 + 2**-8 + 2**-20, -3.140625, 65280.0 + 128.0],
                 dtype=np.float32)
    y = round_bf16(x)
    assert y[0] == 1.0
    assert y[1] == 1.0                       # tie -> even
    assert y[2] == 1 + 2**-6                 # tie -> even (up)
    assert y[3] == 1 + 2**-7                 # above the tie -> up
    assert y[4] == np.float32(-3.140625)     # exactly representable
    assert y[5] == 65536.0                   # tie at 65408 -> even mantissa (rounds up)
    assert np.all((y.view(np.uint32) & 0xFFFF) == 0)

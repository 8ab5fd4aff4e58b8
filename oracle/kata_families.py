"""Plain float64 oracle of the reduced PSD feature families KATA-Sigma g and KATA-M g, and of
the higher even-order lifts psi_2r (bottom of the file).

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` (and nothing on the product path).
Imports numpy and the full-map oracle's normalisation and packing helpers only.

Source: "Kernelized Linear Attention: Breaking the Capacity Wall with Symmetric Cones"
(Ghriss & Chakraborty, arXiv 2607.17419), arXiv HTML page, reduced PSD families paragraph
(KATA-PSD state section): with g dividing the width d and m = d / g, every projected query
or key is split into g consecutive blocks u = (u_1, ..., u_g) of m components;
  * KATA-Sigma g: psi(u) = sum_a u_a u_a^T, one m x m PSD matrix; the Frobenius inner
    product of two features is sum_{a,b} (q_a . k_b)^2; state m(m+1)/2 x dv;
  * KATA-M g: psi(u) = (u_1 u_1^T, ..., u_g u_g^T), one PSD matrix per block; inner product
    sum_a (q_a . k_a)^2; state g m(m+1)/2 x dv;
  * both are the full rank-one map at g = 1.
The readout is the same normalised form as for the full map (normalized-readout
paragraph): o_t = sum_{s<=t} w_ts v_s / sum_{s<=t} w_ts with w_ts = <psi(q_t), psi(k_s)>.

Readings taken where the pages are silent:
  * the whole d-vector is projected onto the unit sphere first (the full map's
    preprocessing), then split into blocks; at g = 1 this is the full map;
  * packed order: Sigma g uses the full map's order for an m x m matrix (row-major upper
    triangle, sqrt(2) off the diagonal); M g concatenates the g blocks' packed m x m
    coordinates, block 1 first.

Parity status: every function below is pinned by tests/test_family_pins.py.
"""
from __future__ import annotations

import math

import numpy as np

from oracle.kata_oracle import _divide_rows, normalize, packed_dim, packed_pairs

FAMILIES = ("full", "sigma", "block")

__all__ = ["FAMILIES", "family_dim", "lift_family", "weights_family", "naive_family",
           "recurrent_family", "prefill_state_family", "decode_steps_family", "order_dim",
           "order_multisets", "lift_order", "naive_order"]


def _check(p: int, family: str, g: int) -> int:
    if family not in FAMILIES:
        raise ValueError(f"family must be one of {FAMILIES}")
    if g < 1 or p % g != 0:
        raise ValueError("g must divide p")
    if family == "full" and g != 1:
        raise ValueError("the full map has g = 1")
    return p // g


def family_dim(p: int, family: str, g: int = 1) -> int:
    """Packed feature width n_psi: p(p+1)/2 (full), m(m+1)/2 (Sigma g), g m(m+1)/2 (M g)."""
    m = _check(p, family, g)
    if family == "full":
        return packed_dim(p)
    return packed_dim(m) * (1 if family == "sigma" else g)


def lift_family(u: np.ndarray, family: str, g: int = 1) -> np.ndarray:
    """Packed feature of the unit-normalised rows of u: [..., p] -> [..., n_psi]."""
    uh = normalize(u)
    p = uh.shape[-1]
    m = _check(p, family, g)
    if family == "full":
        g, m = 1, p
    ii, jj = packed_pairs(m)
    scale = np.where(ii == jj, 1.0, math.sqrt(2.0))
    blocks = [uh[..., a * m:(a + 1) * m] for a in range(g)]
    per_block = [b[..., ii] * b[..., jj] * scale for b in blocks]   # u_a u_a^T, packed
    if family == "sigma":
        return np.sum(per_block, axis=0)
    return np.concatenate(per_block, axis=-1)


def weights_family(qh: np.ndarray, kh: np.ndarray, family: str, g: int = 1) -> np.ndarray:
    """Weights w_ts from block dot products of already normalised rows (the inner-product
    identities of the two displays): qh [..., Tq, p], kh [..., Tk, p] -> [..., Tq, Tk]."""
    p = qh.shape[-1]
    m = _check(p, family, g)
    if family == "full":
        a = qh @ np.swapaxes(kh, -1, -2)
        return a * a
    w = 0.0
    for a in range(g):
        qa = qh[..., a * m:(a + 1) * m]
        for b in range(g):
            if family == "block" and b != a:
                continue
            kb = kh[..., b * m:(b + 1) * m]
            d = qa @ np.swapaxes(kb, -1, -2)
            w = w + d * d
    return w


def naive_family(q: np.ndarray, k: np.ndarray, v: np.ndarray, family: str, g: int = 1) -> np.ndarray:
    """Causal output by the definition, O(T^2), weights from block dot products.
    q, k: [..., T, p]; v: [..., T, dv]."""
    qh, kh = normalize(q), normalize(k)
    v = np.asarray(v, dtype=np.float64)
    T = qh.shape[-2]
    w = weights_family(qh, kh, family, g)
    w = np.where(np.tril(np.ones((T, T), dtype=bool)), w, 0.0)
    return _divide_rows(w @ v, w.sum(axis=-1))


def recurrent_family(q: np.ndarray, k: np.ndarray, v: np.ndarray, family: str, g: int = 1) -> np.ndarray:
    """Token-by-token recurrent form through the packed features:
    S_t = S_{t-1} + psi(k_t) v_t^T, Z_t = Z_{t-1} + psi(k_t), o_t = psi(q_t)^T S_t / psi(q_t)^T Z_t."""
    fq, fk = lift_family(q, family, g), lift_family(k, family, g)
    v = np.asarray(v, dtype=np.float64)
    lead, T, dv = v.shape[:-2], v.shape[-2], v.shape[-1]
    n = fq.shape[-1]
    S, Z = np.zeros(lead + (n, dv)), np.zeros(lead + (n,))
    out = np.zeros(v.shape)
    for t in range(T):
        S += fk[..., t, :, None] * v[..., t, None, :]
        Z += fk[..., t, :]
        num = np.einsum("...f,...fd->...d", fq[..., t, :], S)
        den = np.einsum("...f,...f->...", fq[..., t, :], Z)
        out[..., t, :] = _divide_rows(num, den)
    return out


def prefill_state_family(k: np.ndarray, v: np.ndarray, family: str, g: int = 1):
    """State after a history: S = Psi(K)^T V [..., n, dv], Z = Psi(K)^T 1 [..., n]."""
    fk = lift_family(k, family, g)
    v = np.asarray(v, dtype=np.float64)
    return np.swapaxes(fk, -1, -2) @ v, fk.sum(axis=-2)


def decode_steps_family(S0, Z0, q, k, v, family: str, g: int = 1):
    """Recurrent inference from (S0, Z0): per step update, then read out.
    q, k: [steps, ..., p]; v: [steps, ..., dv]. Returns (o [steps, ..., dv], S, Z)."""
    S = np.array(S0, dtype=np.float64, copy=True)
    Z = np.array(Z0, dtype=np.float64, copy=True)
    fq, fk = lift_family(q, family, g), lift_family(k, family, g)
    v = np.asarray(v, dtype=np.float64)
    outs = np.zeros(v.shape)
    for st in range(v.shape[0]):
        S += fk[st][..., :, None] * v[st][..., None, :]
        Z += fk[st]
        num = np.einsum("...f,...fd->...d", fq[st], S)
        den = np.einsum("...f,...f->...", fq[st], Z)
        outs[st] = _divide_rows(num, den)
    return outs, S, Z


# ------------------------------------------------------------------ higher even orders
# Source: arXiv HTML page, paragraph after the spherical-code discussion (display of
# psi_2r): the same p-dimensional projection generates psi_2r(u) = u^{(x) 2r}, with
# <psi_2r(u), psi_2r(v)> = (u . v)^{2r} >= 0 and symmetric ambient dimension
# binom(p + 2r - 1, 2r); the pages use r = 1.
# Reading (the pages give only the dimension): the symmetric tensor is packed over multisets
# i_1 <= ... <= i_2r in lexicographic order, coordinate sqrt(multinomial) * prod u_i, so the
# packed Euclidean inner product is the tensor one (r = 1: the full map's packing).

def order_dim(p: int, r: int) -> int:
    """binom(p + 2r - 1, 2r) packed coordinates of u^{(x) 2r}."""
    if p < 1 or r < 1:
        raise ValueError("p and r must be >= 1")
    return math.comb(p + 2 * r - 1, 2 * r)


def order_multisets(p: int, r: int) -> list[tuple[int, ...]]:
    """Multisets of size 2r over range(p) in lexicographic order."""
    out = []

    def rec(start, prefix):
        if len(prefix) == 2 * r:
            out.append(tuple(prefix))
            return
        for i in range(start, p):
            rec(i, prefix + [i])
    rec(0, [])
    return out


def lift_order(u: np.ndarray, r: int) -> np.ndarray:
    """Packed psi_2r of the unit-normalised rows of u: [..., p] -> [..., binom(p+2r-1, 2r)]."""
    uh = normalize(u)
    p = uh.shape[-1]
    cols = []
    for ms in order_multisets(p, r):
        counts = np.bincount(np.asarray(ms), minlength=p)
        coef = math.factorial(2 * r)
        for c in counts:
            coef //= math.factorial(int(c))
        val = np.ones(uh.shape[:-1])
        for i in ms:
            val = val * uh[..., i]
        cols.append(math.sqrt(coef) * val)
    return np.stack(cols, axis=-1)


def naive_order(q: np.ndarray, k: np.ndarray, v: np.ndarray, r: int) -> np.ndarray:
    """Causal output with weights (q_hat_t . k_hat_s)^{2r}, by the definition, O(T^2)."""
    qh, kh = normalize(q), normalize(k)
    v = np.asarray(v, dtype=np.float64)
    T = qh.shape[-2]
    a = qh @ np.swapaxes(kh, -1, -2)
    w = np.where(np.tril(np.ones((T, T), dtype=bool)), a ** (2 * r), 0.0)
    return _divide_rows(w @ v, w.sum(axis=-1))

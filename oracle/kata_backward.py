"""Plain float64 gradients of the causal KATA forward (full map and the reduced families).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``; never by the product path. Imports
numpy and the forward oracles' normalisation only.

The pages describe no backward pass (the 340M-parameter runs of the abstract imply one), so
this is the plain calculus of the forward the pages define, written out step by step:
  forward (normalized-readout paragraph, rank-one lift display, reduced PSD families
  paragraph):  q_hat = q / |q|,  k_hat = k / |k|,
      w_ts = sum over the family's block pairs (a, b) of (q_hat_t,a . k_hat_s,b)^2, s <= t,
      D_t = sum_s w_ts,  o_t = sum_s w_ts v_s / D_t   (o_t = 0 where D_t = 0);
  with g_t = dL/do_t and delta_t = g_t . o_t:
      dL/dv_s = sum_{t>=s} (w_ts / D_t) g_t
      dL/dw_ts = (g_t . v_s - delta_t) / D_t
      dL/dq_hat_t,a = sum_{s<=t} dL/dw_ts sum_b 2 (q_hat_t,a . k_hat_s,b) k_hat_s,b
      dL/dk_hat_s,b = sum_{t>=s} dL/dw_ts sum_a 2 (q_hat_t,a . k_hat_s,b) q_hat_t,a
      dL/du = (dL/du_hat - u_hat (u_hat . dL/du_hat)) / |u|   (0 for a zero row)
(the pair sums run over all (a, b) for Sigma g, over a = b for M g, and the full map is g = 1).

Parity status: pinned by tests/test_backward_pins.py (central finite differences in float64
and exact identities of the forward).
"""
from __future__ import annotations

import numpy as np

from oracle.kata_oracle import normalize

__all__ = ["backward"]


def _pairs(g: int, family: str):
    if family == "full":
        return [(0, 0)]
    return [(a, b) for a in range(g) for b in range(g) if family == "sigma" or a == b]


def _unnormalize_grad(u: np.ndarray, d_hat: np.ndarray) -> np.ndarray:
    """Chain rule through u_hat = u / |u| (rows; a zero row gets a zero gradient)."""
    u = np.asarray(u, dtype=np.float64)
    nrm = np.sqrt(np.sum(u * u, axis=-1, keepdims=True))
    uh = normalize(u)
    proj = d_hat - uh * np.sum(uh * d_hat, axis=-1, keepdims=True)
    out = np.zeros_like(u)
    np.divide(proj, nrm, out=out, where=nrm > 0)
    return out


def backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, g_out: np.ndarray, family: str = "full",
             g: int = 1) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(dq, dk, dv) of L with dL/do = g_out. q, k: [..., T, p]; v, g_out: [..., T, dv]."""
    qh, kh = normalize(q), normalize(k)
    v = np.asarray(v, dtype=np.float64)
    go = np.asarray(g_out, dtype=np.float64)
    p, T = qh.shape[-1], qh.shape[-2]
    if family == "full":
        g = 1
    m = p // g
    causal = np.tril(np.ones((T, T), dtype=bool))
    blocks_q = [qh[..., a * m:(a + 1) * m] for a in range(g)]
    blocks_k = [kh[..., b * m:(b + 1) * m] for b in range(g)]
    dots = {}
    w = 0.0
    for (a, b) in _pairs(g, family):
        d = blocks_q[a] @ np.swapaxes(blocks_k[b], -1, -2)          # [..., T, T] : t, s
        dots[(a, b)] = d
        w = w + d * d
    w = np.where(causal, w, 0.0)
    D = w.sum(axis=-1)                                               # [..., T]
    inv = np.zeros_like(D)
    np.divide(1.0, D, out=inv, where=D > 0)
    o = (w @ v) * inv[..., None]
    delta = np.sum(go * o, axis=-1)                                  # [..., T]
    P = w * inv[..., None]                                           # w_ts / D_t
    dv = np.swapaxes(P, -1, -2) @ go
    gv = go @ np.swapaxes(v, -1, -2)                                 # g_t . v_s
    dw = np.where(causal, (gv - delta[..., None]) * inv[..., None], 0.0)
    dqh = np.zeros_like(qh)
    dkh = np.zeros_like(kh)
    for (a, b), d in dots.items():
        coef = 2.0 * dw * d                                          # dL/d(q_a . k_b)
        dqh[..., a * m:(a + 1) * m] += coef @ blocks_k[b]
        dkh[..., b * m:(b + 1) * m] += np.swapaxes(coef, -1, -2) @ blocks_q[a]
    return _unnormalize_grad(q, dqh), _unnormalize_grad(k, dkh), dv

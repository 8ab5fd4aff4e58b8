"""Plain float64 oracle of the KATA causal linear-attention forward.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``; never by the product path. Shares no code with
the HIP kernels (it imports numpy only).

Source: "Kernelized Linear Attention: Breaking the Capacity Wall with Symmetric Cones"
(Ghriss & Chakraborty, arXiv 2607.17419), arXiv HTML page:
  * Eq. (8): a symmetric p x p matrix has n = p(p+1)/2 free coordinates.
  * rank-one lift display (paragraph after Eq. (8)): project once to the unit sphere,
    psi(u) = u u^T, ||u u^T||_F = 1, <u u^T, v v^T>_F = (u.v)^2.
  * normalized-readout paragraph (opening of the mixer discussion): the output is
    psi(q_t)^T S_t / psi(q_t)^T Z_t with an explicit denominator; the readout is a
    convex interpolation, the state update additive and commutative.
  * feature-value state display (KATA-PSD state paragraph): S_t = Psi(K_{1:t})^T V_{1:t}.
  * chunked-forward paragraph (three kernels, wall-clock model): the inter-chunk
    recurrence is an associative prefix sum of per-chunk (S_loc, Z_loc).

Readings taken where the pages are silent:
  * packed order = row-major upper triangle incl. diagonal; off-diagonals scaled by
    sqrt(2) so that the packed Euclidean inner product equals the Frobenius one;
  * no epsilon in the normalisation (a zero vector lifts to zero) and none in the
    denominator (a zero denominator gives a zero output row);
  * causality is inclusive (s <= t): the state S_t contains token t;
  * no temperature, scale or bias: the weight is exactly (q_hat . k_hat)^2.

Parity status: every function below is pinned by tests/test_oracle_pins.py.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "packed_dim", "packed_pairs", "normalize", "lift", "naive", "naive_rows",
    "recurrent", "chunked", "decode_steps", "prefill_state", "row_rel_err",
]


def packed_dim(p: int) -> int:
    """Number of free coordinates of a symmetric p x p matrix (Eq. (8))."""
    if p < 1:
        raise ValueError("p must be >= 1")
    return p * (p + 1) // 2


def packed_pairs(p: int) -> tuple[np.ndarray, np.ndarray]:
    """(i, j) pairs of the packed coordinates: upper triangle incl. the diagonal,
    row by row (i ascending, then j ascending, j >= i)."""
    ii, jj = [], []
    for i in range(p):
        for j in range(i, p):
            ii.append(i)
            jj.append(j)
    return np.asarray(ii, dtype=np.int64), np.asarray(jj, dtype=np.int64)


def normalize(u: np.ndarray) -> np.ndarray:
    """Project rows onto the unit sphere S^{p-1} (rank-one lift paragraph). A zero row
    stays zero (no epsilon: the pages state none)."""
    u = np.asarray(u, dtype=np.float64)
    nrm = np.sqrt(np.sum(u * u, axis=-1, keepdims=True))
    out = np.zeros_like(u)
    np.divide(u, nrm, out=out, where=nrm > 0)
    return out


def lift(u: np.ndarray) -> np.ndarray:
    """Packed rank-one PSD feature psi(u_hat) = u_hat u_hat^T (rank-one lift display).

    Coordinate (i, j), i <= j, holds u_i u_j on the diagonal and sqrt(2) u_i u_j off it,
    so that <psi(a), psi(b)> = <a a^T, b b^T>_F = (a.b)^2.  [..., p] -> [..., n]."""
    uh = normalize(u)
    p = uh.shape[-1]
    ii, jj = packed_pairs(p)
    scale = np.where(ii == jj, 1.0, math.sqrt(2.0))
    return uh[..., ii] * uh[..., jj] * scale


def _divide_rows(num: np.ndarray, den: np.ndarray) -> np.ndarray:
    out = np.zeros_like(num)
    np.divide(num, den[..., None], out=out, where=den[..., None] > 0)
    return out


def naive(q: np.ndarray, k: np.ndarray, v: np.ndarray, block: int = 1024) -> np.ndarray:
    """Causal KATA output by its definition, O(T^2):

        o_t = sum_{s<=t} (q_hat_t . k_hat_s)^2 v_s  /  sum_{s<=t} (q_hat_t . k_hat_s)^2

    (normalized readout with explicit denominator; weight identity of the rank-one lift
    display). q, k: [..., T, p]; v: [..., T, dv]. Evaluated in float64, blocked over
    query rows only to bound memory."""
    qh = normalize(q)
    kh = normalize(k)
    v = np.asarray(v, dtype=np.float64)
    T = qh.shape[-2]
    lead = int(np.prod(qh.shape[:-2])) if qh.ndim > 2 else 1
    # bound the [..., rows, T] score block to about 32 M doubles
    block = max(16, min(block, (1 << 25) // max(1, lead * T)))
    out = np.zeros(v.shape, dtype=np.float64)
    for t0 in range(0, T, block):
        t1 = min(T, t0 + block)
        a = qh[..., t0:t1, :] @ np.swapaxes(kh[..., :t1, :], -1, -2)   # [..., bt, t1]
        w = a * a
        s_idx = np.arange(t1)[None, :]
        t_idx = np.arange(t0, t1)[:, None]
        w = np.where(s_idx <= t_idx, w, 0.0)
        num = w @ v[..., :t1, :]
        den = w.sum(axis=-1)
        out[..., t0:t1, :] = _divide_rows(num, den)
    return out


def naive_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, rows) -> np.ndarray:
    """The same definition evaluated for selected query rows only, one sequence:
    q, k: [T, p], v: [T, dv]; returns [len(rows), dv]."""
    qh = normalize(q)
    kh = normalize(k)
    v = np.asarray(v, dtype=np.float64)
    res = []
    for t in rows:
        a = kh[: t + 1] @ qh[t]
        w = a * a
        den = w.sum()
        res.append(w @ v[: t + 1] / den if den > 0 else np.zeros(v.shape[-1]))
    return np.asarray(res)


def recurrent(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Token-by-token recurrent form (feature-value state display):
    S_t = S_{t-1} + psi(k_t) v_t^T, Z_t = Z_{t-1} + psi(k_t), o_t = psi(q_t)^T S_t /
    psi(q_t)^T Z_t. q, k: [..., T, p]; v: [..., T, dv]."""
    fq = lift(q)
    fk = lift(k)
    v = np.asarray(v, dtype=np.float64)
    lead = v.shape[:-2]
    T, dv = v.shape[-2], v.shape[-1]
    n = fq.shape[-1]
    S = np.zeros(lead + (n, dv))
    Z = np.zeros(lead + (n,))
    out = np.zeros(v.shape)
    for t in range(T):
        S += fk[..., t, :, None] * v[..., t, None, :]
        Z += fk[..., t, :]
        num = np.einsum("...f,...fd->...d", fq[..., t, :], S)
        den = np.einsum("...f,...f->...", fq[..., t, :], Z)
        out[..., t, :] = _divide_rows(num, den)
    return out


def _hillis_steele_exclusive(x: np.ndarray) -> np.ndarray:
    """Exclusive prefix sum along axis 0 in ceil(log2 N) rounds of pairwise adds
    (the log-depth associative scan of the chunked-forward paragraph)."""
    n = x.shape[0]
    inc = x.copy()
    d = 1
    while d < n:
        nxt = inc.copy()
        nxt[d:] = inc[d:] + inc[:-d]
        inc = nxt
        d *= 2
    exc = np.zeros_like(x)
    exc[1:] = inc[:-1]
    return exc


def chunked(q: np.ndarray, k: np.ndarray, v: np.ndarray, C: int,
            scan: str = "sequential") -> np.ndarray:
    """Exact chunked-state form (chunked-forward paragraph). Per chunk c:
    (S_loc, Z_loc) = (Psi(K_c)^T V_c, Psi(K_c)^T 1); the state entering chunk c is the
    exclusive prefix of (S_loc, Z_loc) over chunks, taken either sequentially or by a
    log-depth scan; the chunk output adds the inter-chunk readout psi(q_t)^T S_prefix to
    the intra-chunk causal block (q_hat_t . k_hat_s)^2 over s <= t inside the chunk."""
    if scan not in ("sequential", "associative"):
        raise ValueError("scan must be 'sequential' or 'associative'")
    qh = normalize(q)
    kh = normalize(k)
    fq = lift(q)
    fk = lift(k)
    v = np.asarray(v, dtype=np.float64)
    T = v.shape[-2]
    NC = -(-T // C)
    lead = v.shape[:-2]
    n, dv = fq.shape[-1], v.shape[-1]
    S_loc = np.zeros((NC,) + lead + (n, dv))
    Z_loc = np.zeros((NC,) + lead + (n,))
    for c in range(NC):
        sl = slice(c * C, min(T, (c + 1) * C))
        S_loc[c] = np.swapaxes(fk[..., sl, :], -1, -2) @ v[..., sl, :]
        Z_loc[c] = fk[..., sl, :].sum(axis=-2)
    if scan == "sequential":
        S_pre = np.zeros_like(S_loc)
        Z_pre = np.zeros_like(Z_loc)
        for c in range(1, NC):
            S_pre[c] = S_pre[c - 1] + S_loc[c - 1]
            Z_pre[c] = Z_pre[c - 1] + Z_loc[c - 1]
    else:
        S_pre = _hillis_steele_exclusive(S_loc)
        Z_pre = _hillis_steele_exclusive(Z_loc)
    out = np.zeros(v.shape)
    for c in range(NC):
        sl = slice(c * C, min(T, (c + 1) * C))
        L = sl.stop - sl.start
        num = fq[..., sl, :] @ S_pre[c]
        den = np.einsum("...tf,...f->...t", fq[..., sl, :], Z_pre[c])
        a = qh[..., sl, :] @ np.swapaxes(kh[..., sl, :], -1, -2)
        w = np.where(np.tril(np.ones((L, L), dtype=bool)), a * a, 0.0)
        num = num + w @ v[..., sl, :]
        den = den + w.sum(axis=-1)
        out[..., sl, :] = _divide_rows(num, den)
    return out


def prefill_state(k_hist: np.ndarray, v_hist: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """State after a history: S = Psi(K)^T V, Z = Psi(K)^T 1 (feature-value state
    display). k_hist: [..., T, p]; v_hist: [..., T, dv] -> (S [..., n, dv], Z [..., n])."""
    fk = lift(k_hist)
    v = np.asarray(v_hist, dtype=np.float64)
    return np.swapaxes(fk, -1, -2) @ v, fk.sum(axis=-2)


def decode_steps(S0: np.ndarray, Z0: np.ndarray, q: np.ndarray, k: np.ndarray,
                 v: np.ndarray) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Constant-time recurrent inference: for each step, update then read out.
    S0: [..., n, dv]; Z0: [..., n]; q, k: [steps, ..., p]; v: [steps, ..., dv].
    Returns (o [steps, ..., dv], S, Z) in float64."""
    S = np.array(S0, dtype=np.float64, copy=True)
    Z = np.array(Z0, dtype=np.float64, copy=True)
    fq = lift(q)
    fk = lift(k)
    v = np.asarray(v, dtype=np.float64)
    outs = np.zeros(v.shape)
    for st in range(v.shape[0]):
        S += fk[st][..., :, None] * v[st][..., None, :]
        Z += fk[st]
        num = np.einsum("...f,...fd->...d", fq[st], S)
        den = np.einsum("...f,...f->...", fq[st], Z)
        outs[st] = _divide_rows(num, den)
    return outs, S, Z


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """Max over output rows of ||got_t - ref_t||_inf / ||ref_t||_inf. A reference row
    that is exactly zero requires an exactly zero result row (error inf otherwise)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    g = got.reshape(-1, got.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    num = np.max(np.abs(g - r), axis=-1)
    den = np.max(np.abs(r), axis=-1)
    zero = den == 0
    rel = np.zeros_like(num)
    rel[~zero] = num[~zero] / den[~zero]
    rel[zero & (num > 0)] = np.inf
    if not np.all(np.isfinite(g)):
        return float("inf")
    return float(rel.max()) if rel.size else 0.0

"""F1: the quadratic masked (parallel) form, fp64, numpy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Per sequence of n tokens with decay lam (the glossary page "Lightning
Attention", features list, parallel form for training):
    D[i, j] = lam^(i-j) if i >= j else 0
    P = (Q K^T) * D,  O = P V  [+ diag(lam^(t+1)) Q S0]
    S_final = lam^n S0 + sum_j lam^(n-1-j) k_j v_j^T
Backward of L = <dO, O> + <F, S_final> (F: gradient arriving at the final state):
    G = (dO V^T) * D,  dQ = G K [+ diag(lam^(t+1)) dO S0^T],
    dK = G^T Q + diag(lam^(n-1-j)) V F^T,  dV = P^T dO + diag(lam^(n-1-j)) K F,
    dS0 = Q^T diag(lam^(t+1)) dO + lam^n F.
The n x n matrices make this form usable for n up to a few thousand only.
"""
from __future__ import annotations

import numpy as np

from . import feature


def decay_matrix(n: int, lam: float) -> np.ndarray:
    """D[i, j] = lam^(i-j) for i >= j, 0 above the diagonal (lam^0 = 1, also for lam = 0)."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    e = np.where(i >= j, i - j, 0).astype(np.float64)
    return np.where(i >= j, np.power(np.float64(lam), e), 0.0)


def _powers(lam: float, exps: np.ndarray) -> np.ndarray:
    return np.power(np.float64(lam), exps.astype(np.float64))


def fwd_quadratic(q, k, v, lam, s_init=None, phi="identity"):
    """One sequence: q, k, v [n, d]; returns (O [n, d], S_final [d, d]) with the feature map
    ``phi`` (oracle.feature) on q and k."""
    q = feature.phi(q, phi)
    k = feature.phi(k, phi)
    v = np.asarray(v, dtype=np.float64)
    n = q.shape[0]
    lam = float(np.float64(lam))
    D = decay_matrix(n, lam)
    P = (q @ k.T) * D
    o = P @ v
    w = _powers(lam, np.arange(n - 1, -1, -1))  # lam^(n-1-j)
    s_final = (k * w[:, None]).T @ v
    if s_init is not None:
        s0 = np.asarray(s_init, dtype=np.float64)
        o = o + _powers(lam, np.arange(1, n + 1))[:, None] * (q @ s0)
        s_final = s_final + (lam ** n) * s0
    return o, s_final


def bwd_quadratic(q, k, v, dout, lam, s_init=None, g_final=None, phi="identity"):
    """One sequence: returns (dQ, dK, dV, dS0) of L = <dO, O> + <F, S_final>, F = g_final
    (zero when None), with the feature map ``phi`` on q and k (dQ, dK with respect to the
    raw q and k)."""
    q_raw = np.asarray(q, dtype=np.float64)
    k_raw = np.asarray(k, dtype=np.float64)
    q = feature.phi(q_raw, phi)
    k = feature.phi(k_raw, phi)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(dout, dtype=np.float64)
    n, d = q.shape
    lam = float(np.float64(lam))
    D = decay_matrix(n, lam)
    G = (g @ v.T) * D
    P = (q @ k.T) * D
    dq = G @ k
    if s_init is not None:
        s0 = np.asarray(s_init, dtype=np.float64)
        dq = dq + _powers(lam, np.arange(1, n + 1))[:, None] * (g @ s0.T)
    dk = G.T @ q
    dv = P.T @ g
    ds0 = q.T @ (_powers(lam, np.arange(1, n + 1))[:, None] * g)
    if g_final is not None:
        f = np.asarray(g_final, dtype=np.float64)
        w = _powers(lam, np.arange(n - 1, -1, -1))[:, None]  # lam^(n-1-j)
        dk = dk + w * (v @ f.T)
        dv = dv + w * (k @ f)
        ds0 = ds0 + (lam ** n) * f
    return dq * feature.dphi(q_raw, phi), dk * feature.dphi(k_raw, phi), dv, ds0


def _dpowers(lam: float, exps: np.ndarray) -> np.ndarray:
    """e lam^(e-1) for each e (0 for e = 0, without forming lam^-1)."""
    e = exps.astype(np.float64)
    return np.where(e > 0, e * np.power(np.float64(lam), np.maximum(e - 1, 0)), 0.0)


def dlam_quadratic(q, k, v, dout, lam, s_init=None, g_final=None, phi="identity"):
    """One sequence: dL/dlam of L = <dO, O> + <F, S_final> (F = g_final, zero when None),
    term by term from the parallel form, where lam enters only through
        D[i, j] = lam^(i-j)  ->  D'[i, j] = (i-j) lam^(i-j-1)  (i > j; 0 on and above the diagonal),
        lam^(t+1) q_t S0     ->  (t+1) lam^t q_t S0,
        S_final = lam^n S0 + sum_j lam^(n-1-j) k_j v_j^T
                             ->  n lam^(n-1) S0 + sum_j (n-1-j) lam^(n-2-j) k_j v_j^T."""
    q = feature.phi(q, phi)
    k = feature.phi(k, phi)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(dout, dtype=np.float64)
    n = q.shape[0]
    lam = float(np.float64(lam))
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    dD = np.where(i > j, _dpowers(lam, np.where(i > j, i - j, 0)), 0.0)
    total = float(np.sum((q @ k.T) * dD * (g @ v.T)))
    s0 = None if s_init is None else np.asarray(s_init, dtype=np.float64)
    if s0 is not None:
        w = _dpowers(lam, np.arange(1, n + 1))  # (t+1) lam^t
        total += float(np.sum(w[:, None] * (q @ s0) * g))
    if g_final is not None:
        f = np.asarray(g_final, dtype=np.float64)
        w = _dpowers(lam, np.arange(n - 1, -1, -1))  # (n-1-j) lam^(n-2-j)
        dS = (k * w[:, None]).T @ v
        if s0 is not None:
            dS = dS + _dpowers(lam, np.array([n]))[0] * s0
        total += float(np.sum(f * dS))
    return total


def dlam_magnitude(q, k, v, dout, lam, s_init=None, g_final=None, phi="identity"):
    """One sequence: the sum of the magnitudes of the terms dlam_quadratic adds up,
        sum_{i>j} |D'[i, j] (q_i . k_j)(v_j . dO_i)| + sum_t |(t+1) lam^t q_t S0 dO_t^T|
        + sum_j |(n-1-j) lam^(n-2-j) k_j F v_j^T| + |n lam^(n-1) <F, S0>|.
    Rounding each term moves the sum by up to this much times the unit roundoff, whatever
    the size of the sum itself, so it is the scale an approximate dL/dlam is judged
    against.  With every term of one sign it equals |dL/dlam|."""
    q = feature.phi(q, phi)
    k = feature.phi(k, phi)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(dout, dtype=np.float64)
    n = q.shape[0]
    lam = float(np.float64(lam))
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    dD = np.where(i > j, _dpowers(lam, np.where(i > j, i - j, 0)), 0.0)
    total = float(np.sum(np.abs((q @ k.T) * dD * (g @ v.T))))
    s0 = None if s_init is None else np.asarray(s_init, dtype=np.float64)
    if s0 is not None:
        w = _dpowers(lam, np.arange(1, n + 1))  # (t+1) lam^t
        total += float(np.sum(np.abs(w * np.einsum("td,de,te->t", q, s0, g))))
    if g_final is not None:
        f = np.asarray(g_final, dtype=np.float64)
        w = _dpowers(lam, np.arange(n - 1, -1, -1))  # (n-1-j) lam^(n-2-j)
        total += float(np.sum(np.abs(w * np.einsum("td,de,te->t", k, f, v))))
        if s0 is not None:
            total += abs(float(_dpowers(lam, np.array([n]))[0] * np.sum(f * s0)))
    return total


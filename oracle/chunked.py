"""Chunk-parallel fp64 form of the gated delta rule (second formulation).

TEST INFRASTRUCTURE ONLY.  It exists to pin the token recurrence in
gdn_oracle.c: the two are algebraically identical, so on the same inputs they
must agree to fp64 rounding.  It follows the chunked forward the pages build
on (#2497 page, "What does this PR do?": 64-token chunks, WY-transformed W,
state QDQ at each chunk boundary; #2506 page: exact solve, per-key-channel
pairwise decays taken from prefix differences of the cumulative log-gates).

Per chunk of n tokens entering with state S0 (dv x dk), gamma = inclusive
cumulative sum of the log-gates inside the chunk (a vector per token for the
per-key-channel gate):
    A[r, s] = beta_r * sum_c k[r, c] k[s, c] exp(gamma[r, c] - gamma[s, c])   (s < r)
    T       = (I + A)^-1 diag(beta)                       (exact solve)
    W       = T (K * exp(gamma)),   U = T V               (WY / UT transform)
    U'      = U - W S0^T                                   (pseudo-values)
    P[r, s] = sum_c q[r, c] k[s, c] exp(gamma[r, c] - gamma[s, c])  (s <= r)
    O       = (Q * exp(gamma)) S0^T + P U'
    S_n     = S0 diag(exp(gamma_n)) + U'^T (K * exp(gamma_n - gamma))
then S_n <- QDQ(S_n) when chunk-boundary QDQ is on.
"""
from __future__ import annotations

import numpy as np

from . import oracle as _orc


def _qdq_f64(S):
    out, _, _ = _orc.qdq_states(S.astype(np.float32))
    return out.astype(np.float64)


def gdn_chunked(q, k, v, beta, g, *, chunk=64, qdq=True, S0=None):
    """Chunked forward over a whole sequence (prefix length = L).

    q, k: [L, dk]; v: [L, dv]; beta: [L]; g: [L] or [L, dk]; float64.
    Returns dict(o [L, dv], S [dv, dk])."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    beta = np.asarray(beta, np.float64)
    g = np.asarray(g, np.float64)
    L, dk = k.shape
    dv = v.shape[1]
    per_channel = g.ndim == 2
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((L, dv))
    for c0 in range(0, L, chunk):
        c1 = min(L, c0 + chunk)
        n = c1 - c0
        Q, K, V, b = q[c0:c1], k[c0:c1], v[c0:c1], beta[c0:c1]
        if per_channel:
            gam = np.cumsum(g[c0:c1], axis=0)                         # [n, dk]
            diff = gam[:, None, :] - gam[None, :, :]                  # [r, s, c]
            lower = np.tril(np.ones((n, n), dtype=bool), -1)
            incl = np.tril(np.ones((n, n), dtype=bool))[:, :, None]
            dec = np.where(incl, np.exp(np.where(incl, diff, 0.0)), 0.0)   # s <= r only
            A = b[:, None] * np.einsum("rc,sc,rsc->rs", K, K, dec) * lower
            Pm = np.einsum("rc,sc,rsc->rs", Q, K, dec)
            eg = np.exp(gam)                                          # [n, dk]
            egn = np.exp(gam[-1][None, :] - gam)                      # [n, dk]
            T = np.linalg.solve(np.eye(n) + A, np.diag(b))
            W = T @ (K * eg)
            U = T @ V
            Up = U - W @ S.T
            o[c0:c1] = (Q * eg) @ S.T + Pm @ Up
            S = S * np.exp(gam[-1])[None, :] + Up.T @ (K * egn)
        else:
            gam = np.cumsum(g[c0:c1])                                 # [n]
            diff = gam[:, None] - gam[None, :]
            lower = np.tril(np.ones((n, n), dtype=bool), -1)
            incl = np.tril(np.ones((n, n), dtype=bool))
            dec = np.where(incl, np.exp(np.where(incl, diff, 0.0)), 0.0)
            A = (b[:, None] * dec * (K @ K.T)) * lower
            Pm = dec * (Q @ K.T)
            T = np.linalg.solve(np.eye(n) + A, np.diag(b))
            W = T @ (K * np.exp(gam)[:, None])
            U = T @ V
            Up = U - W @ S.T
            o[c0:c1] = (Q * np.exp(gam)[:, None]) @ S.T + Pm @ Up
            S = np.exp(gam[-1]) * S + Up.T @ (K * np.exp(gam[-1] - gam)[:, None])
        if qdq:
            S = _qdq_f64(S)
    return {"o": o, "S": S}

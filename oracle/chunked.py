"""Chunk-parallel fp64 form of the gated delta rule (second formulation).

TEST INFRASTRUCTURE ONLY.  It has two uses:
  - it pins the token recurrence in gdn_oracle.c: with W QDQ off the two are
    algebraically identical, so on the same inputs they must agree to fp64
    rounding;
  - it is the reference for W QDQ, which only exists in the chunked form.
It follows the chunked forward the pages build on (#2497 page, "What does this
PR do?": 64-token chunks, WY-transformed W, state QDQ at each chunk boundary,
independent dynamic FP8 fake QDQ of the WY-transformed W; #2506 page: exact
solve, per-key-channel pairwise decays taken from prefix differences of the
cumulative log-gates).

Per chunk of n tokens entering with state S0 (dv x dk), gamma = inclusive
cumulative sum of the log-gates inside the chunk (a vector per token for the
per-key-channel gate):
    A[r, s] = beta_r * sum_c k[r, c] k[s, c] exp(gamma[r, c] - gamma[s, c])   (s < r)
    T       = (I + A)^-1 diag(beta)                       (exact solve)
    W       = T (K * exp(gamma)),   U = T V               (WY / UT transform)
    W       <- QDQ per row of W (one scale per token and head, amax over the
               key axis; #2497 Usage: the W quantizer keeps axes (0, 1, 2) of
               W [batch, token, head, key]) when W QDQ is on; the decision is
               taken on W stored to fp32, as for the state
    U'      = U - W S0^T                                   (pseudo-values)
    P[r, s] = sum_c q[r, c] k[s, c] exp(gamma[r, c] - gamma[s, c])  (s <= r)
    O       = (Q * exp(gamma)) S0^T + P U'
    S_n     = S0 diag(exp(gamma_n)) + U'^T (K * exp(gamma_n - gamma))
then S_n <- QDQ(S_n) at the boundary when the QDQ flags ask for it.  W only
enters U' (through W S0^T), so with S0 = 0 its QDQ has no effect.
"""
from __future__ import annotations

import numpy as np

from . import oracle as _orc


def _qdq_f64(S):
    out, _, _ = _orc.qdq_states(S.astype(np.float32))
    return out.astype(np.float64)


def qdq_w(W):
    """W QDQ: W (n x dk, fp64) stored to fp32, then each row quantized with
    its own scale.  Returns (Wq fp64, scales fp32 [n])."""
    out, sc, _ = _orc.qdq_rows(np.asarray(W, np.float64).astype(np.float32))
    return out.astype(np.float64), sc


def chunk_operators(Q, K, b, g, *, w_qdq=False, Wq=None):
    """The state-independent operators of one chunk of n <= 64 tokens, fp64:
    T = (I + A)^-1 diag(b), W = T (K o e^gamma), Wq (the quantized W with
    w_qdq, else W; a given Wq is used as is), Pm (P[r][s] = e^{gamma_r -
    gamma_s} q_r . k_s for s <= r), eg = e^gamma, egn = e^{gamma_n - gamma}
    ([n, 1] for the scalar gate, [n, dk] per channel) and end = e^{gamma_n}
    (the decay of the entering state)."""
    n = K.shape[0]
    lower = np.tril(np.ones((n, n), dtype=bool), -1)
    if g.ndim == 2:
        gam = np.cumsum(g, axis=0)                                # [n, dk]
        diff = gam[:, None, :] - gam[None, :, :]                  # [r, s, c]
        incl = np.tril(np.ones((n, n), dtype=bool))[:, :, None]
        dec = np.where(incl, np.exp(np.where(incl, diff, 0.0)), 0.0)   # s <= r only
        A = b[:, None] * np.einsum("rc,sc,rsc->rs", K, K, dec) * lower
        Pm = np.einsum("rc,sc,rsc->rs", Q, K, dec)
        eg = np.exp(gam)                                          # [n, dk]
        egn = np.exp(gam[-1][None, :] - gam)                      # [n, dk]
        end = np.exp(gam[-1])[None, :]                            # S0 diag(exp(gamma_n))
    else:
        gam = np.cumsum(g)                                        # [n]
        diff = gam[:, None] - gam[None, :]
        incl = np.tril(np.ones((n, n), dtype=bool))
        dec = np.where(incl, np.exp(np.where(incl, diff, 0.0)), 0.0)
        A = (b[:, None] * dec * (K @ K.T)) * lower
        Pm = dec * (Q @ K.T)
        eg = np.exp(gam)[:, None]
        egn = np.exp(gam[-1] - gam)[:, None]
        end = np.exp(gam[-1])
    T = np.linalg.solve(np.eye(n) + A, np.diag(b))
    W = T @ (K * eg)
    w_scales = None
    if Wq is None:
        if w_qdq:
            Wq, w_scales = qdq_w(W)
        else:
            Wq = W
    return dict(T=T, W=W, Wq=Wq, w_scales=w_scales, Pm=Pm, eg=eg, egn=egn, end=end)


def chunk_step(Q, K, V, b, g, S, *, w_qdq=False, Wq=None):
    """One chunk of n <= 64 tokens from state S (dv x dk), all fp64.

    g: [n] (scalar gate) or [n, dk].  Wq: optional n x dk matrix used in
    place of the (quantized) W (teacher forcing).  Returns dict(o [n, dv],
    S [dv, dk] before any boundary QDQ, W [n, dk] before QDQ, Wq [n, dk]
    the matrix that entered W S^T, w_scales [n] or None)."""
    op = chunk_operators(Q, K, b, g, w_qdq=w_qdq, Wq=Wq)
    T, W, Wq, w_scales = op["T"], op["W"], op["Wq"], op["w_scales"]
    Pm, eg, egn, end = op["Pm"], op["eg"], op["egn"], op["end"]
    U = T @ V
    Up = U - Wq @ S.T
    o = (Q * eg) @ S.T + Pm @ Up
    S_new = S * end + Up.T @ (K * egn)
    return {"o": o, "S": S_new, "W": W, "Wq": Wq, "w_scales": w_scales}


def gdn_chunked(q, k, v, beta, g, *, chunk=64, qdq=True, S0=None, prefix_len=None, flags=None,
                w_qdq=False, record=False):
    """Chunked forward of one (sequence, head).

    q, k: [L, dk]; v: [L, dv]; beta: [L]; g: [L] or [L, dk]; float64.
    Without prefix_len and flags: the whole sequence chunked, state QDQ at
    every chunk boundary (including t = L) when qdq.  With prefix_len P or
    flags (oracle.QDQ_CHUNK | QDQ_WRITE bits): tokens 1..P chunked, QDQ after
    a chunk when QDQ_CHUNK, or when it ends at t = P and QDQ_WRITE; tokens
    P < t <= L run through the token recurrence (gdn_oracle.c) with QDQ
    after every write when QDQ_WRITE.  Returns dict(o [L, dv], S [dv, dk]),
    plus, when record, per chunk: bound_pre / bound_post [nb, dv, dk], W,
    Wq [nb, chunk, dk] (rows past a chunk's end zero), w_scales [nb, chunk]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    beta = np.asarray(beta, np.float64)
    g = np.asarray(g, np.float64)
    L, dk = k.shape
    dv = v.shape[1]
    if flags is None:
        flags = (_orc.QDQ_CHUNK | _orc.QDQ_WRITE) if qdq else 0
    P = L if prefix_len is None else int(prefix_len)
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((L, dv))
    nb = (P + chunk - 1) // chunk
    rec = None
    if record:
        rec = {"bound_pre": np.zeros((nb, dv, dk)), "bound_post": np.zeros((nb, dv, dk)),
               "W": np.zeros((nb, chunk, dk)), "Wq": np.zeros((nb, chunk, dk)),
               "w_scales": np.ones((nb, chunk), np.float32)}
    for i, c0 in enumerate(range(0, P, chunk)):
        c1 = min(P, c0 + chunk)
        r = chunk_step(q[c0:c1], k[c0:c1], v[c0:c1], beta[c0:c1], g[c0:c1], S, w_qdq=w_qdq)
        o[c0:c1] = r["o"]
        pre = r["S"]
        S = pre
        if (flags & _orc.QDQ_CHUNK) or ((flags & _orc.QDQ_WRITE) and c1 == P):
            S = _qdq_f64(pre)
        if record:
            n = c1 - c0
            rec["bound_pre"][i] = pre
            rec["bound_post"][i] = S
            rec["W"][i, :n] = r["W"]
            rec["Wq"][i, :n] = r["Wq"]
            if r["w_scales"] is not None:
                rec["w_scales"][i, :n] = r["w_scales"]
    if P < L:
        sfx = _orc.gdn_sequence(q[P:], k[P:], v[P:], beta[P:], g[P:], prefix_len=0,
                                flags=flags & _orc.QDQ_WRITE, S0=S)
        o[P:] = sfx["o"]
        S = sfx["S"]
    out = {"o": o, "S": S}
    if record:
        out.update(rec)
    return out

"""State gradients of the gated delta rule (reverse recurrence), fp64.

TEST INFRASTRUCTURE ONLY: the tests compare the library's chunked backward
state recurrence against this.

The pages train through the state QDQ with identity straight-through
gradients (#2497 page, "What does this PR do?": "identity straight-through
gradients for QAT/QAD"), so in the backward every QDQ is the identity map.
For a loss that is linear in the outputs and the final state,
    L = sum_t o_t . do_t + <S_L, dS_L>,
the gradient with respect to any state is then that of the plain recurrence
    S_t = a_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  o_t = S_t q_t,
and does not depend on the states themselves.  Written out token by token
backwards (G the gradient with respect to S_t):
    G <- dS_L
    for t = L .. 1:   G <- G + do_t q_t^T                (o_t = S_t q_t)
                      G <- a_t G (I - beta_t k_t k_t^T)   (now d L / d S_{t-1})
The state entering chunk c of the chunked prefix is S_{64c}; its gradient
dh_c is G right after token 64c + 1 has been taken back.  v_t enters only
through beta_t v_t k_t^T, so its gradient is beta_t G k_t with G the
gradient of S_t (before taking token t back).  A per-key-channel
gate (S_{t-1} diag(a_t) in place of a_t S_{t-1}) gives G <- G (I - beta k
k^T) diag(a_t).
"""
from __future__ import annotations

import numpy as np

CHUNK = 64


def state_grads(q, k, beta, g, do, dS_L=None, *, chunk=CHUNK, want_dv=False):
    """One (sequence, head).  q, k: [L, dk]; beta: [L]; g: [L] or [L, dk];
    do: [L, dv]; dS_L: [dv, dk] or None (zero).  float64.

    Returns (dh [ceil(L / chunk), dv, dk] the gradient of each chunk's
    entering state, dS0 [dv, dk] the gradient of the initial state), and
    with want_dv also dv [L, dv], the gradient of the values."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    beta = np.asarray(beta, np.float64)
    g = np.asarray(g, np.float64)
    do = np.asarray(do, np.float64)
    L, dk = k.shape
    dv = do.shape[1]
    G = np.zeros((dv, dk)) if dS_L is None else np.array(dS_L, dtype=np.float64)
    nb = (L + chunk - 1) // chunk
    dh = np.zeros((nb, dv, dk))
    dvals = np.zeros((L, dv))
    for t in range(L, 0, -1):
        i = t - 1
        G = G + np.outer(do[i], q[i])
        Gk = G @ k[i]
        dvals[i] = beta[i] * Gk
        G = G - beta[i] * np.outer(Gk, k[i])
        G = G * np.exp(g[i]) if g.ndim == 1 else G * np.exp(g[i])[None, :]
        if (t - 1) % chunk == 0:
            dh[(t - 1) // chunk] = G
    if want_dv:
        return dh, G, dvals
    return dh, G


def packed_state_grads(q, k, beta, g, do, cu_seqlens, *, seq_lens=None, dS_L=None):
    """Packed layout: q, k [T, H, dk], beta [T, H], g [T, H] or [T, H, dk],
    do [T, H, dv], dS_L [N, H, dv, dk] or None.  Returns (dh [n_bounds, H,
    dv, dk] with chunk b of sequence n at b = sum_{m<n} ceil(L_m/64) + i,
    dS0 [N, H, dv, dk], dv [T, H, dv] with zero padding rows)."""
    cu = np.asarray(cu_seqlens, np.int64)
    N = cu.size - 1
    H, dk = k.shape[1], k.shape[2]
    dv = do.shape[2]
    lens = (cu[1:] - cu[:-1]) if seq_lens is None else np.asarray(seq_lens, np.int64)
    nbs = [(int(L) + CHUNK - 1) // CHUNK for L in lens]
    offs = np.concatenate([[0], np.cumsum(nbs)]).astype(np.int64)
    dh = np.zeros((int(offs[-1]), H, dv, dk))
    dS0 = np.zeros((N, H, dv, dk))
    dvals = np.zeros(do.shape)
    for n in range(N):
        s0, L = int(cu[n]), int(lens[n])
        sl = slice(s0, s0 + L)
        for h in range(H):
            gg = g[sl, h] if g.ndim == 2 else g[sl, h, :]
            r_dh, r_0, r_v = state_grads(q[sl, h], k[sl, h], beta[sl, h], gg, do[sl, h],
                                         None if dS_L is None else dS_L[n, h], want_dv=True)
            dh[offs[n]:offs[n + 1], h] = r_dh
            dS0[n, h] = r_0
            dvals[sl, h] = r_v
    return dh, dS0, dvals


def chunked_state_grads(q, k, beta, g, do, dS_L=None, *, w_qdq=False, want_dv=False, Wq=None):
    """The same gradients through the chunk-level forward of the chunked
    prefix (one (sequence, head), the whole sequence chunked by 64), which is
    where W QDQ lives.  Per chunk with entering state h, the forward
    (oracle.chunked.chunk_step) is
        U' = T V - Wq h^T,   O = (Q o e^gamma) h^T + P U',
        h' = h e^{gamma_n} + U'^T (K o e^{gamma_n - gamma})
    with Wq = Q(W) under W QDQ (else W = T (K o e^gamma)); the quantizer's
    identity straight-through rule (#2497 page, "What does this PR do?")
    makes the gradient of h the one of that linear map with Wq fixed, so
    with G' = dL/dh' and dO the chunk's output gradient, backwards:
        dU' = P^T dO + (K o e^{gamma_n - gamma}) G'^T
        dh  = G' e^{gamma_n} + dO^T (Q o e^gamma) - dU'^T Wq
        dV  = T^T dU'                     (V enters only through U = T V)
    (e^{gamma_n} multiplies columns, i.e. key channels, for the
    per-key-channel gate).  Without W QDQ this equals state_grads.  Wq:
    optional [n_chunks, 64, dk] matrices used as each chunk's Wq (rows past
    the chunk's end ignored; teacher forcing).  Returns (dh [n_chunks, dv,
    dk], dS0) and with want_dv also dv [L, dv]."""
    from .chunked import chunk_operators
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    beta = np.asarray(beta, np.float64)
    g = np.asarray(g, np.float64)
    do = np.asarray(do, np.float64)
    L, dk = k.shape
    dv = do.shape[1]
    G = np.zeros((dv, dk)) if dS_L is None else np.array(dS_L, dtype=np.float64)
    nb = (L + CHUNK - 1) // CHUNK
    dh = np.zeros((nb, dv, dk))
    dvals = np.zeros((L, dv))
    for c in range(nb - 1, -1, -1):
        c0, c1 = c * CHUNK, min(L, (c + 1) * CHUNK)
        op = chunk_operators(q[c0:c1], k[c0:c1], beta[c0:c1], g[c0:c1], w_qdq=w_qdq,
                             Wq=None if Wq is None else np.asarray(Wq[c][:c1 - c0], np.float64))
        dO = do[c0:c1]
        dU = op["Pm"].T @ dO + (k[c0:c1] * op["egn"]) @ G.T
        dvals[c0:c1] = op["T"].T @ dU
        G = G * op["end"] + dO.T @ (q[c0:c1] * op["eg"]) - dU.T @ op["Wq"]
        dh[c] = G
    if want_dv:
        return dh, G, dvals
    return dh, G


def packed_chunked_state_grads(q, k, beta, g, do, cu_seqlens, *, seq_lens=None, dS_L=None, w_qdq=False):
    """packed_state_grads through chunked_state_grads (the W-QDQ forward's
    gradients with w_qdq)."""
    cu = np.asarray(cu_seqlens, np.int64)
    N = cu.size - 1
    H, dk = k.shape[1], k.shape[2]
    dv = do.shape[2]
    lens = (cu[1:] - cu[:-1]) if seq_lens is None else np.asarray(seq_lens, np.int64)
    nbs = [(int(L) + CHUNK - 1) // CHUNK for L in lens]
    offs = np.concatenate([[0], np.cumsum(nbs)]).astype(np.int64)
    dh = np.zeros((int(offs[-1]), H, dv, dk))
    dS0 = np.zeros((N, H, dv, dk))
    dvals = np.zeros(do.shape)
    for n in range(N):
        s0, L = int(cu[n]), int(lens[n])
        sl = slice(s0, s0 + L)
        for h in range(H):
            gg = g[sl, h] if g.ndim == 2 else g[sl, h, :]
            r_dh, r_0, r_v = chunked_state_grads(q[sl, h], k[sl, h], beta[sl, h], gg, do[sl, h],
                                                 None if dS_L is None else dS_L[n, h], w_qdq=w_qdq,
                                                 want_dv=True)
            dh[offs[n]:offs[n + 1], h] = r_dh
            dS0[n, h] = r_0
            dvals[sl, h] = r_v
    return dh, dS0, dvals

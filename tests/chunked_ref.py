"""fp64 chunked (WY / UT-transform) form of the KDA recurrence -- a test-side derivation.

It is a second, independent route to the recurrence that the oracle computes token by
token (page "colibri/c/kimi_k3.c", header comment "KDA per-head recurrence"), used to
pin the oracle (the two must agree to rounding) and to check the chunk algebra that the
prefill kernel implements.  It works on already-normalised q, k, the values v, the
log-decays gk and beta, i.e. it covers the state update and readout only.

Derivation.  With D_t = Diag(exp(gk_t)) the update is S_t = D_t S_{t-1} + k_t u_t^T where
u_t = beta_t (v_t - S_{t-1}^T (exp(gk_t) * k_t)).  Inside a chunk with initial state S0
and G_t = sum_{s<=t} gk_s (per key channel):

    S_t = Diag(e^{G_t}) S0 + sum_{s<=t} Diag(e^{G_t - G_s}) k_s u_s^T
    (I + A) U = diag(beta) V - diag(beta) (K * e^G) S0,
        A_ts = beta_t sum_i k_ti k_si e^{G_ti - G_si}           (s < t)
    U = T diag(beta) V - T diag(beta)(K * e^G) S0 = U' - W S0,  T = (I + A)^-1
    O = (Q * e^G) S0 + P U,  P_ts = sum_i q_ti k_si e^{G_ti - G_si}   (s <= t)
    S_L = Diag(e^{G_L}) S0 + (K * e^{G_L - G})^T U

The products e^{G_t - G_s} are formed as e^{G_t - r} * e^{r - G_s} with the reference
r taken at the end of the sub-chunk before t's sub-chunk (0 for the first), so that in
fp32 neither factor leaves the representable range when sub-chunks are at most 16
tokens long and |gk| < 5.
"""
from __future__ import annotations

import numpy as np


def chunk_step(S0, q, k, v, gk, beta, sub: int = 16):
    """One chunk of L tokens.  q, k, gk: [L, dk]; v: [L, dv]; beta: [L]; S0: [dk, dv].
    Returns (O [L, dv], S_L [dk, dv])."""
    L = q.shape[0]
    G = np.cumsum(gk, axis=0)
    nsub = (L + sub - 1) // sub
    ref = np.zeros((nsub, G.shape[1]))
    for I in range(1, nsub):
        ref[I] = G[I * sub - 1]
    A = np.zeros((L, L))
    P = np.zeros((L, L))
    for I in range(nsub):
        ti = slice(I * sub, min(L, (I + 1) * sub))
        row = np.exp(G[ti] - ref[I])
        kr, qr = k[ti] * row, q[ti] * row
        for J in range(I + 1):
            sj = slice(J * sub, min(L, (J + 1) * sub))
            col = k[sj] * np.exp(ref[I] - G[sj])
            A[ti, sj] = kr @ col.T
            P[ti, sj] = qr @ col.T
    A = np.tril(A, -1) * beta[:, None]
    P = np.tril(P, 0)
    # T = (I + A)^-1 by forward substitution
    T = np.eye(L)
    for t in range(1, L):
        T[t, :t] = -A[t, :t] @ T[:t, :t]
    W = T @ (beta[:, None] * k * np.exp(G))
    Up = T @ (beta[:, None] * v)
    U = Up - W @ S0
    O = (q * np.exp(G)) @ S0 + P @ U
    SL = np.exp(G[-1])[:, None] * S0 + (k * np.exp(G[-1] - G)).T @ U
    return O, SL


def chunked(S0, q, k, v, gk, beta, chunk: int = 64, sub: int = 16):
    """Whole sequence in chunks of ``chunk`` tokens (the last one partial)."""
    T = q.shape[0]
    S = np.array(S0, dtype=np.float64)
    O = np.zeros((T, v.shape[1]))
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        O[c0:c1], S = chunk_step(S, q[c0:c1], k[c0:c1], v[c0:c1], gk[c0:c1], beta[c0:c1], sub)
    return O, S

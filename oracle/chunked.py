"""Independent fp64 chunked form of the KDA recurrence (test infrastructure only).

Used only to pin the token-by-token oracle: for any chunk size C the two must
agree to fp64 rounding.  It follows from the recurrence
    S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,  o_t = S_t^T q_t
by unrolling one chunk from its entry state S.  With gamma_r = sum_{s<=r} g_s
(per key channel, inclusive, inside the chunk) and E_rs = exp(gamma_r - gamma_s):
    A[r,s] = beta_r sum_c k_rc k_sc E_rs,c   (s < r)
    P[r,s] = sum_c q_rc k_sc E_rs,c           (s <= r)
    (I + A) Delta = diag(beta) (V - (K * e^gamma) S)
    O = scale * ((Q * e^gamma) S + P Delta)
    S <- Diag(e^gamma_C) S + (K * e^(gamma_C - gamma))^T Delta
Exponent differences are taken exactly (no factoring), and the triangular
system is solved with a library solver.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular

from .api import f64


def _chunk(q, k, v, g, beta, S, scale):
    L = q.shape[0]
    G = np.cumsum(g, axis=0)                                  # [L, dk]
    diff = G[:, None, :] - G[None, :, :]                      # gamma_r - gamma_s
    causal = np.tril(np.ones((L, L), dtype=bool))             # s <= r
    E = np.exp(np.where(causal[:, :, None], diff, -np.inf))   # 0 above the diagonal
    KK = np.einsum("rc,sc,rsc->rs", k, k, E)
    A = np.tril(KK, -1) * beta[:, None]
    P = np.einsum("rc,sc,rsc->rs", q, k, E)
    eg = np.exp(G)
    rhs = beta[:, None] * (v - (k * eg) @ S)
    Delta = solve_triangular(np.eye(L) + A, rhs, lower=True, unit_diagonal=True)
    O = scale * ((q * eg) @ S + P @ Delta)
    S_new = np.exp(G[-1])[:, None] * S + (k * np.exp(G[-1][None, :] - G)).T @ Delta
    return O, S_new


def prefill_chunked(q, k, v, g, beta, cu_seqlens, initial_state=None, scale=1.0, C=64):
    q, k, v, g, beta = f64(q), f64(k), f64(v), f64(g), f64(beta)
    cu = [int(c) for c in np.asarray(cu_seqlens)]
    T, H, dk = q.shape
    dv = v.shape[2]
    N = len(cu) - 1
    o = np.zeros((T, H, dv))
    Sf = np.zeros((N, H, dk, dv))
    for n in range(N):
        for h in range(H):
            S = np.zeros((dk, dv)) if initial_state is None else f64(initial_state)[n, h].copy()
            for t0 in range(cu[n], cu[n + 1], C):
                t1 = min(t0 + C, cu[n + 1])
                O, S = _chunk(q[t0:t1, h], k[t0:t1, h], v[t0:t1, h], g[t0:t1, h],
                              beta[t0:t1, h], S, scale)
                o[t0:t1, h] = O
            Sf[n, h] = S
    return o, Sf

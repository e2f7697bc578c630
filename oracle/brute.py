"""Brute-force dense-matrix evaluation of the GDN recurrence for tiny inputs.

TEST INFRASTRUCTURE ONLY (pins the token oracle; imported by tests alone).

Instead of the rank-1 loop, each token's transition is built as an explicit
K x K matrix  M_i = exp(g_i) (I - beta_i k_i k_i^T),  and the state after token
t is evaluated from the closed expansion of the gated delta rule

    S_t = (M_t ... M_1) S_0 + sum_{j <= t} (M_t ... M_{j+1}) beta_j k_j v_j^T

with o_t = scale * S_t^T q_t.  Every product is recomputed from scratch for
every t, so the cost is O(T^3 K^3): use T <= 16.
"""
from __future__ import annotations

import numpy as np


def fwd_one(q, k, v, g, beta, scale, S0):
    """q,k [L,K], v [L,V], g,beta [L], S0 [K,V] -> o [L,V], S_L."""
    L, K = k.shape
    M = [np.exp(g[i]) * (np.eye(K) - beta[i] * np.outer(k[i], k[i])) for i in range(L)]

    def prod(lo, hi):  # M_hi ... M_lo (inclusive, 0-based), identity if empty
        P = np.eye(K)
        for i in range(lo, hi + 1):
            P = M[i] @ P
        return P

    o = np.zeros((L, v.shape[1]))
    S = S0
    for t in range(L):
        S = prod(0, t) @ S0
        for j in range(t + 1):
            S = S + prod(j + 1, t) @ (beta[j] * np.outer(k[j], v[j]))
        o[t] = scale * (S.T @ q[t])
    return o, S


def fwd(q, k, v, g, beta, scale=None, initial_state=None):
    """Whole problem without cu_seqlens (B rows), fp64."""
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    B, T, Hq, K = q.shape
    Hv, V = v.shape[2], v.shape[3]
    grp = Hv // Hq
    if scale is None:
        scale = K ** -0.5
    o = np.zeros((B, T, Hv, V))
    ht = np.zeros((B, Hv, K, V))
    for b in range(B):
        for h in range(Hv):
            S0 = (np.zeros((K, V)) if initial_state is None
                  else np.asarray(initial_state[b, h], dtype=np.float64))
            o[b, :, h], ht[b, h] = fwd_one(q[b, :, h // grp], k[b, :, h // grp],
                                           v[b, :, h], g[b, :, h], beta[b, :, h],
                                           scale, S0)
    return o, ht

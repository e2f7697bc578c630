"""Chunked (WY-form) fp64 NumPy implementation of the GDN forward and backward.

TEST INFRASTRUCTURE ONLY.  It exists to pin the token-recurrence oracle
(``gdn_oracle.c``) from a second, separately written formulation, and to give
per-chunk intermediates (gate cumsum, the inverse T) to compare against.  Only
tests, the smoke check and the benchmark's CPU-baseline leg may import it.

The FlashQLA pages name the chunked prefill of the gated delta rule and say its
reformulation is strictly equivalent to the plain recurrence (aiwebcool
"flashqla-resource", section 三, second feature; zhengruan news, "技术内核"),
and the low-level forward returns a processed gate ``g`` and a matrix ``A``
(FlashQLA article, "底层 API").  The pages print no formulas.  The chunk form
used here, per chunk of n tokens with entering state S (K x V):

    gamma   = inclusive cumsum of g inside the chunk
    E[r,j]  = exp(gamma_r - gamma_j)                       (j <= r)
    A       = strict_lower( diag(beta) K K^T * E )
    T       = (I + A)^-1
    w       = T diag(beta * exp(gamma)) K,   u = T diag(beta) V
    Vn      = u - w S
    P       = lower_incl( Q K^T * E )
    O       = scale (diag(exp(gamma)) Q S + P Vn)
    S'      = exp(gamma_L) S + K^T diag(exp(gamma_L - gamma)) Vn

and the backward is the reverse mode of exactly these steps (chunk by chunk,
in reverse).  ``chunk`` may be any positive size; chunks never cross
sequences.
"""
from __future__ import annotations

import numpy as np


def _units(q, v, cu_seqlens):
    B, T, Hq, K = q.shape
    Hv = v.shape[2]
    if cu_seqlens is None:
        spans = [(b, 0, T) for b in range(B)]  # (batch row, start, end)
    else:
        cu = [int(x) for x in cu_seqlens]
        spans = [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]
    return spans, Hq, Hv, Hv // Hq


def chunk_forward_one(q, k, v, g, beta, scale, S, chunk):
    """One (sequence, v-head): q,k [L,K], v [L,V], g,beta [L], S [K,V].

    Returns o [L,V], final S, and per-chunk intermediates
    (list of dicts with gamma, T, S_in).
    """
    L = q.shape[0]
    o = np.zeros((L, v.shape[1]))
    inter = []
    for s in range(0, L, chunk):
        e = min(s + chunk, L)
        Q, Kc, Vc = q[s:e], k[s:e], v[s:e]
        gam = np.cumsum(g[s:e])
        b = beta[s:e]
        E = np.exp(gam[:, None] - gam[None, :])
        n = e - s
        low_strict = np.tril(np.ones((n, n)), -1)
        low_incl = np.tril(np.ones((n, n)))
        E = E * low_incl  # only j <= r is ever used
        A = low_strict * (b[:, None] * (Kc @ Kc.T) * E)
        Tm = np.linalg.inv(np.eye(n) + A)
        w = Tm @ ((b * np.exp(gam))[:, None] * Kc)
        u = Tm @ (b[:, None] * Vc)
        Vn = u - w @ S
        P = low_incl * ((Q @ Kc.T) * E)
        o[s:e] = scale * (np.exp(gam)[:, None] * (Q @ S) + P @ Vn)
        inter.append(dict(gamma=gam, T=Tm, S_in=S.copy()))
        gL = gam[-1]
        S = np.exp(gL) * S + Kc.T @ (np.exp(gL - gam)[:, None] * Vn)
    return o, S, inter


def chunk_backward_one(q, k, v, g, beta, scale, S0, do, dST, chunk):
    """Reverse mode of :func:`chunk_forward_one` for one (sequence, v-head).

    Returns dq, dk, dv, dbeta, dg (w.r.t. raw g), dS0.
    """
    L, Kd = q.shape
    # forward pass, remembering each chunk's entering state
    starts = list(range(0, L, chunk))
    S = S0.copy()
    S_in = []
    for s in starts:
        e = min(s + chunk, L)
        S_in.append(S.copy())
        _, S, _ = chunk_forward_one(q[s:e], k[s:e], v[s:e], g[s:e], beta[s:e],
                                    scale, S, e - s)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    db = np.zeros_like(beta)
    dg = np.zeros_like(g)
    dS = dST.copy()  # gradient w.r.t. the state leaving the current chunk
    for ci in range(len(starts) - 1, -1, -1):
        s = starts[ci]
        e = min(s + chunk, L)
        n = e - s
        Q, Kc, Vc, dO = q[s:e], k[s:e], v[s:e], do[s:e]
        b = beta[s:e]
        S = S_in[ci]
        gam = np.cumsum(g[s:e])
        eg = np.exp(gam)
        gL = gam[-1]
        low_strict = np.tril(np.ones((n, n)), -1)
        low_incl = np.tril(np.ones((n, n)))
        E = np.exp(gam[:, None] - gam[None, :]) * low_incl
        KK = Kc @ Kc.T
        QK = Q @ Kc.T
        A = low_strict * (b[:, None] * KK * E)
        Tm = np.linalg.inv(np.eye(n) + A)
        Kb = (b * eg)[:, None] * Kc
        Vb = b[:, None] * Vc
        w = Tm @ Kb
        u = Tm @ Vb
        Vn = u - w @ S
        P = low_incl * (QK * E)
        QS = Q @ S
        decay_out = np.exp(gL - gam)
        Kt = decay_out[:, None] * Kc  # K~

        dgam = np.zeros(n)
        # S' = exp(gL) S + K~^T Vn
        dVn = scale * P.T @ dO + Kt @ dS
        dKt = Vn @ dS.T
        dS_in = np.exp(gL) * dS
        dgam[-1] += np.exp(gL) * np.sum(dS * S)
        c = np.sum(dKt * Kt, axis=1)  # d/d(gL - gam_r)
        dgam[-1] += c.sum()
        dgam -= c
        dKc = decay_out[:, None] * dKt
        # O = scale (diag(eg) Q S + P Vn)
        dP = scale * (dO @ Vn.T) * low_incl
        dQS = scale * eg[:, None] * dO
        dgam += eg * scale * np.sum(dO * QS, axis=1)
        dQ = dQS @ S.T
        dS_in += Q.T @ dQS
        # P = lower_incl(QK * E)
        dQK = dP * E
        dQ += dQK @ Kc
        dKc += dQK.T @ Q
        PdP = dP * P
        dgam += PdP.sum(axis=1) - PdP.sum(axis=0)
        # Vn = u - w S
        du = dVn
        dw = -dVn @ S.T
        dS_in += -w.T @ dVn
        # u = T Vb, w = T Kb
        dT = du @ Vb.T + dw @ Kb.T
        dVb = Tm.T @ du
        dKb = Tm.T @ dw
        dv[s:e] = b[:, None] * dVb
        db[s:e] += np.sum(dVb * Vc, axis=1)
        db[s:e] += eg * np.sum(dKb * Kc, axis=1)
        dgam += b * eg * np.sum(dKb * Kc, axis=1)
        dKc += (b * eg)[:, None] * dKb
        # T = (I + A)^-1
        dA = -(Tm.T @ dT @ Tm.T) * low_strict
        # A = strict_lower(diag(b) KK * E)
        db[s:e] += np.sum(dA * KK * E, axis=1)
        dKK = b[:, None] * dA * E
        dKc += (dKK + dKK.T) @ Kc
        AdA = dA * A
        dgam += AdA.sum(axis=1) - AdA.sum(axis=0)
        # gamma = cumsum(g): dg_t = sum_{r >= t} dgam_r
        dg[s:e] = np.cumsum(dgam[::-1])[::-1]
        dq[s:e] = dQ
        dk[s:e] = dKc
        dS = dS_in
    return dq, dk, dv, db, dg, dS


def fwd(q, k, v, g, beta, scale=None, initial_state=None, cu_seqlens=None,
        chunk=64):
    """Chunked forward over a whole problem (layouts as the token oracle)."""
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    spans, Hq, Hv, grp = _units(q, v, cu_seqlens)
    Kd, Vd = q.shape[3], v.shape[3]
    if scale is None:
        scale = Kd ** -0.5
    o = np.zeros(v.shape)
    ht = np.zeros((len(spans), Hv, Kd, Vd))
    for n, (bi, s0, s1) in enumerate(spans):
        for h in range(Hv):
            hq = h // grp
            S = (np.zeros((Kd, Vd)) if initial_state is None
                 else np.asarray(initial_state[n, h], dtype=np.float64).copy())
            if s1 > s0:
                oo, S, _ = chunk_forward_one(q[bi, s0:s1, hq], k[bi, s0:s1, hq],
                                             v[bi, s0:s1, h], g[bi, s0:s1, h],
                                             beta[bi, s0:s1, h], scale, S, chunk)
                o[bi, s0:s1, h] = oo
            ht[n, h] = S
    return o, ht


def bwd(q, k, v, g, beta, do, dht=None, scale=None, initial_state=None,
        cu_seqlens=None, chunk=64):
    """Chunked backward over a whole problem; dq/dk summed over GQA groups."""
    q, k, v, g, beta, do = (np.asarray(x, dtype=np.float64)
                            for x in (q, k, v, g, beta, do))
    spans, Hq, Hv, grp = _units(q, v, cu_seqlens)
    Kd, Vd = q.shape[3], v.shape[3]
    if scale is None:
        scale = Kd ** -0.5
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    db = np.zeros(beta.shape)
    dg = np.zeros(g.shape)
    dh0 = np.zeros((len(spans), Hv, Kd, Vd))
    for n, (bi, s0, s1) in enumerate(spans):
        for h in range(Hv):
            hq = h // grp
            S0 = (np.zeros((Kd, Vd)) if initial_state is None
                  else np.asarray(initial_state[n, h], dtype=np.float64))
            dST = (np.zeros((Kd, Vd)) if dht is None
                   else np.asarray(dht[n, h], dtype=np.float64))
            if s1 == s0:
                dh0[n, h] = dST
                continue
            r = chunk_backward_one(q[bi, s0:s1, hq], k[bi, s0:s1, hq],
                                   v[bi, s0:s1, h], g[bi, s0:s1, h],
                                   beta[bi, s0:s1, h], scale, S0,
                                   do[bi, s0:s1, h], dST, chunk)
            dq[bi, s0:s1, hq] += r[0]
            dk[bi, s0:s1, hq] += r[1]
            dv[bi, s0:s1, h] = r[2]
            db[bi, s0:s1, h] = r[3]
            dg[bi, s0:s1, h] = r[4]
            dh0[n, h] = r[5]
    return dq, dk, dv, db, dg, dh0

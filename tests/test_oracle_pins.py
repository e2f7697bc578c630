"""Pins of the fp64 oracle against things other than itself.

The pages print no worked example, no formula and no reference values (the
FlashQLA article's API sections give only signatures), so the oracle is pinned
by: brute-force dense evaluation on tiny inputs, a separately written chunked
(WY) form at several chunk sizes, closed forms of degenerate gates/strengths,
invariants of the recurrence (linearity, resume, packing, GQA grouping,
contraction) and central finite differences for every gradient.
"""
import numpy as np
import pytest

from oracle import brute, chunked, token


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def problem(B=1, T=12, Hq=1, Hv=2, K=5, V=3, seed=0, h0=True, lengths=None,
            normalize=True):
    rng = np.random.default_rng(seed)
    if lengths is not None:
        B, T = 1, int(sum(lengths))
    q = rng.standard_normal((B, T, Hq, K))
    k = rng.standard_normal((B, T, Hq, K))
    if normalize:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, Hv, V))
    g = -np.logaddexp(0, rng.standard_normal((B, T, Hv)))
    beta = 1 / (1 + np.exp(-rng.standard_normal((B, T, Hv))))
    N = B if lengths is None else len(lengths)
    S0 = rng.standard_normal((N, Hv, K, V)) if h0 else None
    cu = None if lengths is None else np.concatenate([[0], np.cumsum(lengths)])
    return dict(q=q, k=k, v=v, g=g, beta=beta, initial_state=S0, cu_seqlens=cu)


# ---------------------------------------------------------------- forward pins

@pytest.mark.parametrize("shape", [dict(B=2, T=9, Hq=1, Hv=2, K=5, V=3),
                                   dict(B=1, T=16, Hq=2, Hv=2, K=3, V=6),
                                   dict(B=1, T=11, Hq=1, Hv=3, K=4, V=4)])
def test_token_fwd_matches_brute_force(shape):
    p = problem(**shape, seed=1)
    o, ht = token.fwd(p["q"], p["k"], p["v"], p["g"], p["beta"], scale=0.7,
                      initial_state=p["initial_state"])
    ob, hb = brute.fwd(p["q"], p["k"], p["v"], p["g"], p["beta"], scale=0.7,
                       initial_state=p["initial_state"])
    assert rel(o, ob) < 1e-12
    assert rel(ht, hb) < 1e-12


@pytest.mark.parametrize("chunk", [1, 7, 16, 64, 1000])
def test_token_fwd_matches_chunked(chunk):
    p = problem(B=2, T=70, Hq=2, Hv=4, K=6, V=5, seed=2)
    o, ht = token.fwd(p["q"], p["k"], p["v"], p["g"], p["beta"],
                      initial_state=p["initial_state"])
    oc, hc = chunked.fwd(p["q"], p["k"], p["v"], p["g"], p["beta"],
                         initial_state=p["initial_state"], chunk=chunk)
    assert rel(o, oc) < 1e-12
    assert rel(ht, hc) < 1e-12


def test_varlen_chunked_and_packing():
    lengths = [5, 0, 67, 1, 64]
    p = problem(Hq=1, Hv=2, K=4, V=3, lengths=lengths, seed=3)
    o, ht = token.fwd(**{k: p[k] for k in ("q", "k", "v", "g", "beta",
                                            "initial_state", "cu_seqlens")})
    oc, hc = chunked.fwd(**{k: p[k] for k in ("q", "k", "v", "g", "beta",
                                               "initial_state", "cu_seqlens")},
                         chunk=16)
    assert rel(o, oc) < 1e-12 and rel(ht, hc) < 1e-12
    # packing: one packed call == one call per sequence
    cu = p["cu_seqlens"]
    for n, L in enumerate(lengths):
        s, e = cu[n], cu[n + 1]
        sl = lambda x: x[:, s:e]
        on, hn = token.fwd(sl(p["q"]), sl(p["k"]), sl(p["v"]), sl(p["g"]),
                           sl(p["beta"]), initial_state=p["initial_state"][n:n + 1])
        assert rel(o[:, s:e], on) < 1e-15 or L == 0
        assert rel(ht[n:n + 1], hn) < 1e-15
    # a zero-length sequence passes its initial state through
    assert np.array_equal(ht[1], p["initial_state"][1])


def test_closed_form_beta_zero():
    p = problem(B=1, T=10, Hq=1, Hv=2, K=4, V=3, seed=4)
    beta = np.zeros_like(p["beta"])
    o, ht = token.fwd(p["q"], p["k"], p["v"], p["g"], beta, scale=0.5,
                      initial_state=p["initial_state"])
    G = np.cumsum(p["g"], axis=1)  # [B,T,Hv]
    for h in range(2):
        S0 = p["initial_state"][0, h]
        for t in range(10):
            exp = 0.5 * np.exp(G[0, t, h]) * S0.T @ p["q"][0, t, 0]
            assert np.allclose(o[0, t, h], exp, rtol=1e-13, atol=1e-15)
        assert np.allclose(ht[0, h], np.exp(G[0, -1, h]) * S0, rtol=1e-13, atol=0)


def test_closed_form_full_forget():
    p = problem(B=1, T=8, Hq=1, Hv=2, K=4, V=3, seed=5)
    g = np.full_like(p["g"], -1e4)  # exp(g) == 0 exactly
    o, ht = token.fwd(p["q"], p["k"], p["v"], g, p["beta"], scale=0.9,
                      initial_state=p["initial_state"])
    q, k, v, b = p["q"][0, :, 0], p["k"][0, :, 0], p["v"][0], p["beta"][0]
    for h in range(2):
        for t in range(8):
            exp = 0.9 * b[t, h] * (q[t] @ k[t]) * v[t, h]
            assert np.allclose(o[0, t, h], exp, rtol=1e-13, atol=1e-15)
        assert np.allclose(ht[0, h], b[-1, h] * np.outer(k[-1], v[-1, h]), rtol=1e-13)


def test_closed_form_one_hot_keys_is_decayed_linear_attention():
    T, K, V = 6, 8, 3
    p = problem(B=1, T=T, Hq=1, Hv=1, K=K, V=V, seed=6, h0=False)
    k = np.zeros((1, T, 1, K))
    for t in range(T):
        k[0, t, 0, t] = 1.0
    o, _ = token.fwd(p["q"], k, p["v"], p["g"], p["beta"], scale=1.3)
    G = np.cumsum(p["g"][0, :, 0])
    b = p["beta"][0, :, 0]
    q, v = p["q"][0, :, 0], p["v"][0, :, 0]
    for t in range(T):
        exp = 1.3 * sum(np.exp(G[t] - G[j]) * b[j] * q[t, j] * v[j] for j in range(t + 1))
        assert np.allclose(o[0, t, 0], exp, rtol=1e-13, atol=1e-15)


def test_closed_form_unit_write_retrieves_value():
    # beta = 1 and ||k|| = 1: S_t^T k_t = v_t exactly, whatever the history
    p = problem(B=1, T=20, Hq=1, Hv=2, K=6, V=4, seed=7)
    beta = np.ones_like(p["beta"])
    o, _ = token.fwd(p["k"], p["k"], p["v"], p["g"], beta, scale=1.0,
                     initial_state=p["initial_state"])
    assert np.abs(o - p["v"]).max() < 1e-13


def test_linearity_in_values_and_state_and_scale():
    p = problem(B=1, T=30, Hq=1, Hv=2, K=5, V=4, seed=8)
    r = np.random.default_rng(9)
    v2 = r.standard_normal(p["v"].shape)
    S2 = r.standard_normal(p["initial_state"].shape)
    a, b = 0.3, -1.7
    f = lambda v, S, sc=1.0: token.fwd(p["q"], p["k"], v, p["g"], p["beta"], scale=sc,
                                       initial_state=S)
    o1, h1 = f(p["v"], p["initial_state"])
    o2, h2 = f(v2, S2)
    o3, h3 = f(a * p["v"] + b * v2, a * p["initial_state"] + b * S2)
    assert rel(o3, a * o1 + b * o2) < 1e-13 and rel(h3, a * h1 + b * h2) < 1e-13
    o4, _ = f(p["v"], p["initial_state"], 2.5)
    assert rel(o4, 2.5 * o1) < 1e-15


def test_resume_equals_single_run():
    p = problem(B=1, T=50, Hq=1, Hv=2, K=4, V=5, seed=10)
    o, ht = token.fwd(p["q"], p["k"], p["v"], p["g"], p["beta"],
                      initial_state=p["initial_state"])
    T1 = 23
    s1 = lambda x: x[:, :T1]
    s2 = lambda x: x[:, T1:]
    oa, ha = token.fwd(s1(p["q"]), s1(p["k"]), s1(p["v"]), s1(p["g"]), s1(p["beta"]),
                       initial_state=p["initial_state"])
    ob, hb = token.fwd(s2(p["q"]), s2(p["k"]), s2(p["v"]), s2(p["g"]), s2(p["beta"]),
                       initial_state=ha)
    assert rel(np.concatenate([oa, ob], axis=1), o) < 1e-14
    assert rel(hb, ht) < 1e-14


def test_gqa_grouping_equals_repeated_heads():
    p = problem(B=1, T=20, Hq=2, Hv=6, K=4, V=3, seed=11)
    o, ht = token.fwd(p["q"], p["k"], p["v"], p["g"], p["beta"],
                      initial_state=p["initial_state"])
    qr = np.repeat(p["q"], 3, axis=2)  # v-head h reads q/k head h // 3
    kr = np.repeat(p["k"], 3, axis=2)
    o2, h2 = token.fwd(qr, kr, p["v"], p["g"], p["beta"], initial_state=p["initial_state"])
    assert np.array_equal(o, o2) and np.array_equal(ht, h2)


def test_contraction_bound():
    p = problem(B=1, T=40, Hq=1, Hv=1, K=5, V=4, seed=12)
    S = p["initial_state"]
    for t in range(40):
        sl = lambda x: x[:, t:t + 1]
        _, S_new = token.fwd(sl(p["q"]), sl(p["k"]), sl(p["v"]), sl(p["g"]),
                             sl(p["beta"]), initial_state=S)
        bound = (np.exp(p["g"][0, t, 0]) * np.linalg.norm(S[0, 0], 2)
                 + p["beta"][0, t, 0] * np.linalg.norm(p["v"][0, t, 0]))
        assert np.linalg.norm(S_new[0, 0], 2) <= bound * (1 + 1e-12)
        S = S_new


def test_affine_segment_composition():
    # S_end(S0) = Phi(S0) + H with Phi linear: the identity the context-parallel
    # split relies on.  Phi is obtained from the run with v = 0.
    p = problem(B=1, T=37, Hq=1, Hv=1, K=4, V=3, seed=13)
    _, H = token.fwd(p["q"], p["k"], p["v"], p["g"], p["beta"], initial_state=None)
    _, Phi = token.fwd(p["q"], p["k"], np.zeros_like(p["v"]), p["g"], p["beta"],
                       initial_state=p["initial_state"])
    _, full = token.fwd(p["q"], p["k"], p["v"], p["g"], p["beta"],
                        initial_state=p["initial_state"])
    assert rel(full, Phi + H) < 1e-14


# --------------------------------------------------------------- backward pins

def _loss(p, do, dht, scale, **over):
    args = {k: p[k] for k in ("q", "k", "v", "g", "beta", "initial_state", "cu_seqlens")}
    args.update(over)
    o, ht = token.fwd(args["q"], args["k"], args["v"], args["g"], args["beta"],
                      scale=scale, initial_state=args["initial_state"],
                      cu_seqlens=args["cu_seqlens"])
    return float(np.sum(o * do) + np.sum(ht * dht))


@pytest.mark.parametrize("kw", [dict(B=1, T=9, Hq=1, Hv=2, K=3, V=4),
                                dict(lengths=[4, 0, 7], Hq=2, Hv=2, K=4, V=2)])
def test_token_bwd_matches_finite_differences(kw):
    p = problem(seed=14, **kw)
    r = np.random.default_rng(15)
    o, ht = token.fwd(p["q"], p["k"], p["v"], p["g"], p["beta"], scale=0.8,
                      initial_state=p["initial_state"], cu_seqlens=p["cu_seqlens"])
    do = r.standard_normal(o.shape)
    dht = r.standard_normal(ht.shape)
    grads = token.bwd(p["q"], p["k"], p["v"], p["g"], p["beta"], do, dht, scale=0.8,
                      initial_state=p["initial_state"], cu_seqlens=p["cu_seqlens"])
    names = ["q", "k", "v", "beta", "g", "initial_state"]
    eps = 1e-6
    for name, gr in zip(names, [grads[0], grads[1], grads[2], grads[3], grads[4], grads[5]]):
        x = p[name]
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = x.copy(); xp[idx] += eps
            xm = x.copy(); xm[idx] -= eps
            fd[idx] = (_loss(p, do, dht, 0.8, **{name: xp})
                       - _loss(p, do, dht, 0.8, **{name: xm})) / (2 * eps)
        assert rel(gr, fd) < 1e-6, name


@pytest.mark.parametrize("chunk", [1, 5, 16, 64])
def test_token_bwd_matches_chunked_bwd(chunk):
    p = problem(B=2, T=70, Hq=2, Hv=4, K=6, V=5, seed=16)
    r = np.random.default_rng(17)
    do = r.standard_normal(p["v"].shape)
    dht = r.standard_normal(p["initial_state"].shape)
    a = token.bwd(p["q"], p["k"], p["v"], p["g"], p["beta"], do, dht,
                  initial_state=p["initial_state"])
    b = chunked.bwd(p["q"], p["k"], p["v"], p["g"], p["beta"], do, dht,
                    initial_state=p["initial_state"], chunk=chunk)
    for x, y in zip(a, b):
        assert rel(x, y) < 1e-12


def test_bwd_varlen_chunked():
    lengths = [3, 70, 0, 1, 33]
    p = problem(Hq=1, Hv=2, K=4, V=3, lengths=lengths, seed=18)
    r = np.random.default_rng(19)
    do = r.standard_normal(p["v"].shape)
    dht = r.standard_normal(p["initial_state"].shape)
    kw = dict(initial_state=p["initial_state"], cu_seqlens=p["cu_seqlens"])
    a = token.bwd(p["q"], p["k"], p["v"], p["g"], p["beta"], do, dht, **kw)
    b = chunked.bwd(p["q"], p["k"], p["v"], p["g"], p["beta"], do, dht, chunk=16, **kw)
    for x, y in zip(a, b):
        assert rel(x, y) < 1e-12


def test_closed_form_gradients_beta_zero():
    # beta = 0: S_t = e^{G_t} S0, so dS0 = sum_t scale e^{G_t} q_t do_t^T + e^{G_T} dht,
    # dq_t = scale e^{G_t} S0 do_t, dv = 0, and
    # dg_t = sum_{s>=t} scale e^{G_s} <S0^T q_s, do_s> + e^{G_T} <S0, dht>.
    p = problem(B=1, T=7, Hq=1, Hv=1, K=3, V=4, seed=20)
    r = np.random.default_rng(21)
    do = r.standard_normal(p["v"].shape)
    dht = r.standard_normal(p["initial_state"].shape)
    beta = np.zeros_like(p["beta"])
    sc = 0.6
    dq, dk, dv, db, dg, dh0 = token.bwd(p["q"], p["k"], p["v"], p["g"], beta, do, dht,
                                        scale=sc, initial_state=p["initial_state"])
    G = np.cumsum(p["g"][0, :, 0])
    S0 = p["initial_state"][0, 0]
    q = p["q"][0, :, 0]
    d = do[0, :, 0]
    exp_dh0 = sum(sc * np.exp(G[t]) * np.outer(q[t], d[t]) for t in range(7)) \
        + np.exp(G[-1]) * dht[0, 0]
    assert rel(dh0[0, 0], exp_dh0) < 1e-13
    for t in range(7):
        assert rel(dq[0, t, 0], sc * np.exp(G[t]) * S0 @ d[t]) < 1e-13
    assert np.abs(dv).max() == 0.0
    terms = [sc * np.exp(G[s]) * (S0.T @ q[s]) @ d[s] for s in range(7)]
    for t in range(7):
        exp = sum(terms[t:]) + np.exp(G[-1]) * np.sum(S0 * dht[0, 0])
        assert abs(dg[0, t, 0] - exp) <= 1e-12 * max(1.0, abs(exp))


def test_oracle_threads_do_not_change_results():
    p = problem(B=2, T=40, Hq=2, Hv=4, K=5, V=6, seed=22)
    a = token.fwd(p["q"], p["k"], p["v"], p["g"], p["beta"],
                  initial_state=p["initial_state"], threads=1)
    b = token.fwd(p["q"], p["k"], p["v"], p["g"], p["beta"],
                  initial_state=p["initial_state"], threads=4)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


def test_unit_mask_samples_units():
    p = problem(B=2, T=30, Hq=1, Hv=3, K=4, V=3, seed=23)
    full = token.fwd(p["q"], p["k"], p["v"], p["g"], p["beta"],
                     initial_state=p["initial_state"])
    mask = np.zeros((2, 3), dtype=bool)
    mask[1, 2] = True
    part = token.fwd(p["q"], p["k"], p["v"], p["g"], p["beta"],
                     initial_state=p["initial_state"], unit_mask=mask)
    assert np.array_equal(part[0][1, :, 2], full[0][1, :, 2])
    assert np.array_equal(part[1][1, 2], full[1][1, 2])
    assert np.abs(part[0][0]).max() == 0.0

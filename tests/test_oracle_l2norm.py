"""Pins of the oracle's optional in-kernel q/k L2 normalisation
(``oracle.l2norm``; used by ``token.fwd/bwd(..., qk_l2norm=True)``).

The forward is pinned by what characterises a per-row L2 normalisation: the
result does not change when a row is scaled (degree-0 homogeneity) and rows of
unit L2 norm pass through (up to the eps term), while rows of unit L1 norm do
not.  The reverse mode is pinned by finite differences of the whole forward
(normalisation + recurrence) with respect to the raw q and k."""
import numpy as np
import pytest

from oracle import l2norm, token
from tests.test_oracle_pins import problem, rel


def _fwd(p, **kw):
    return token.fwd(p["q"], p["k"], p["v"], p["g"], p["beta"], scale=0.9,
                     initial_state=p["initial_state"], cu_seqlens=p["cu_seqlens"], **kw)


def test_scaling_rows_changes_nothing():
    p = problem(B=1, T=10, Hq=2, Hv=4, K=4, V=3, seed=31, normalize=False)
    o, ht = _fwd(p, qk_l2norm=True)
    r = np.random.default_rng(32)
    cq = r.uniform(0.3, 5.0, size=p["q"].shape[:-1] + (1,))
    ck = r.uniform(0.3, 5.0, size=p["k"].shape[:-1] + (1,))
    p2 = dict(p, q=p["q"] * cq, k=p["k"] * ck)
    o2, ht2 = _fwd(p2, qk_l2norm=True)
    # only the eps term depends on the row scale
    assert rel(o2, o) < 1e-5 and rel(ht2, ht) < 1e-5
    # without the normalisation the same scaling does change the result
    o3, _ = _fwd(p2)
    assert rel(o3, _fwd(p)[0]) > 1e-2


def test_unit_l2_rows_pass_through_and_unit_l1_rows_do_not():
    p = problem(B=1, T=9, Hq=1, Hv=2, K=5, V=3, seed=33, normalize=True)
    o_n, _ = _fwd(p, qk_l2norm=True)
    o_p, _ = _fwd(p)
    assert rel(o_n, o_p) < 1e-5          # eps/2 relative at unit norm
    l1 = dict(p, q=p["q"] / np.sum(np.abs(p["q"]), -1, keepdims=True),
              k=p["k"] / np.sum(np.abs(p["k"]), -1, keepdims=True))
    assert rel(_fwd(l1, qk_l2norm=True)[0], _fwd(l1)[0]) > 1e-2
    xh = l2norm.fwd(p["q"] * 7.0)
    assert np.allclose(np.linalg.norm(xh, axis=-1), 1.0, atol=1e-7)


@pytest.mark.parametrize("kw", [dict(B=1, T=8, Hq=1, Hv=2, K=3, V=4),
                                dict(lengths=[5, 0, 4], Hq=2, Hv=4, K=4, V=2)])
def test_l2norm_backward_matches_finite_differences(kw):
    p = problem(seed=34, normalize=False, **kw)
    r = np.random.default_rng(35)
    o, ht = _fwd(p, qk_l2norm=True)
    do = r.standard_normal(o.shape)
    dht = r.standard_normal(ht.shape)
    dq, dk, dv, db, dg, dh0 = token.bwd(
        p["q"], p["k"], p["v"], p["g"], p["beta"], do, dht, scale=0.9,
        initial_state=p["initial_state"], cu_seqlens=p["cu_seqlens"], qk_l2norm=True)

    def loss(**over):
        pp = dict(p, **over)
        oo, hh = _fwd(pp, qk_l2norm=True)
        return float(np.sum(oo * do) + np.sum(hh * dht))

    h = 1e-6
    for name, gr in (("q", dq), ("k", dk), ("v", dv)):
        x = p[name]
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            fd[idx] = (loss(**{name: xp}) - loss(**{name: xm})) / (2 * h)
        assert rel(gr, fd) < 1e-6, name


def test_planted_mistakes_are_caught(monkeypatch):
    """Dropping the projection term of the reverse mode, or normalising by the
    squared norm, must fail the pins above."""
    p = problem(B=1, T=6, Hq=1, Hv=2, K=3, V=2, seed=36, normalize=False)
    good = token.bwd(p["q"], p["k"], p["v"], p["g"], p["beta"], np.ones((1, 6, 2, 2)),
                     np.zeros((1, 2, 3, 2)), scale=0.9, initial_state=p["initial_state"],
                     qk_l2norm=True)[0]
    monkeypatch.setattr(l2norm, "bwd", lambda x, dxh, eps=l2norm.EPS: dxh / np.sqrt(
        np.sum(np.asarray(x) ** 2, -1, keepdims=True) + eps))
    bad = token.bwd(p["q"], p["k"], p["v"], p["g"], p["beta"], np.ones((1, 6, 2, 2)),
                    np.zeros((1, 2, 3, 2)), scale=0.9, initial_state=p["initial_state"],
                    qk_l2norm=True)[0]
    assert rel(bad, good) > 1e-3
    monkeypatch.undo()
    monkeypatch.setattr(l2norm, "fwd", lambda x, eps=l2norm.EPS: np.asarray(x) / (
        np.sum(np.asarray(x) ** 2, -1, keepdims=True) + eps))
    with pytest.raises(AssertionError):
        test_scaling_rows_changes_nothing()

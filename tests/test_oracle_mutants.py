"""The oracle's pins have teeth: plausible mistakes planted in copies of the C
oracle (on the CPU, in a temporary directory) must each fail a pin.

Each mutant is one textual edit of gdn_oracle.c: a dropped term, a wrong sign,
a wrong index, an operand taken from the wrong step.  The pin battery is the
brute-force forward comparison, the GQA grouping check and the central
finite-difference gradient check used in test_oracle_pins.py.
"""
import os

import numpy as np
import pytest

from oracle import brute, token

SRC = os.path.join(os.path.dirname(token.__file__), "gdn_oracle.c")

MUTANTS = {
    "no_decay": ("      Si[j] *= a;\n", "\n"),
    "delta_sign": ("p[j] = beta * (v[j] - p[j]);", "p[j] = beta * (v[j] + p[j]);"),
    "no_beta": ("p[j] = beta * (v[j] - p[j]);", "p[j] = (v[j] - p[j]);"),
    "output_before_update": (
        "      Si[j] += ki * p[j];\n      if (o) o[j] += Si[j] * qi;",
        "      if (o) o[j] += Si[j] * qi;\n      Si[j] += ki * p[j];"),
    "no_scale": ("for (int j = 0; j < V; ++j) o[j] *= scale;", "for (int j = 0; j < V; ++j) o[j] *= 1.0;"),
    "gqa_modulo": ("const int n = u / Hv, h = u % Hv, hq = h / grp;\n      int64_t tok0, len;\n      unit_range(&d, n, &tok0, &len);\n      if (h0)\n        memcpy(S, h0 + (size_t)u * K * V",
                   "const int n = u / Hv, h = u % Hv, hq = h % Hq;\n      int64_t tok0, len;\n      unit_range(&d, n, &tok0, &len);\n      if (h0)\n        memcpy(S, h0 + (size_t)u * K * V"),
    "ignore_h0": ("      if (h0)\n        memcpy(S, h0 + (size_t)u * K * V, sizeof(double) * (size_t)K * V);",
                  "      if (0)\n        memcpy(S, h0 + (size_t)u * K * V, sizeof(double) * (size_t)K * V);"),
    "bwd_dg_sign": ("dga += dst * (a * Sr[j]);", "dga -= dst * (a * Sr[j]);"),
    "bwd_drop_dk_term": ("dkt[r] += a * acc;", "dkt[r] += 0.0 * acc;"),
    "bwd_dbeta_uses_v": ("db += dd[j] * (vt[j] - p[j]);", "db += dd[j] * vt[j];"),
    "bwd_dq_no_scale": ("dqt[r] = scale * acc;", "dqt[r] = acc;"),
    "bwd_no_state_decay": ("dSr[j] = a * dst;", "dSr[j] = dst;"),
    "bwd_dv_no_beta": ("dvt[j] = bt * dd[j];", "dvt[j] = dd[j];"),
    "bwd_dq_pre_state": ("const double *Sr = St + (size_t)r * V;\n            for (int j = 0; j < V; ++j) acc += Sr[j] * dot[j];",
                         "const double *Sr = Sp + (size_t)r * V;\n            for (int j = 0; j < V; ++j) acc += Sr[j] * dot[j];"),
}


def _problem(seed=3):
    rng = np.random.default_rng(seed)
    B, T, Hq, Hv, K, V = 1, 6, 1, 2, 3, 4
    q = rng.standard_normal((B, T, Hq, K))
    k = rng.standard_normal((B, T, Hq, K))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, Hv, V))
    g = -np.logaddexp(0, rng.standard_normal((B, T, Hv)))
    beta = 1 / (1 + np.exp(-rng.standard_normal((B, T, Hv))))
    S0 = rng.standard_normal((B, Hv, K, V))
    return q, k, v, g, beta, S0


def pins_pass(orc) -> bool:
    """True iff the oracle object passes every pin of the battery."""
    q, k, v, g, beta, S0 = _problem()
    sc = 0.7
    o, ht = orc.fwd(q, k, v, g, beta, scale=sc, initial_state=S0)
    ob, hb = brute.fwd(q, k, v, g, beta, scale=sc, initial_state=S0)
    if not (np.allclose(o, ob, rtol=1e-10, atol=1e-12)
            and np.allclose(ht, hb, rtol=1e-10, atol=1e-12)):
        return False
    # grouping: Hq = 1 < Hv = 2, so both v-heads read q/k head 0
    q2 = np.concatenate([q, q * 0.5], axis=2)
    k2 = np.concatenate([k, k[:, ::-1]], axis=2)
    v4 = np.concatenate([v, v], axis=2)
    g4 = np.concatenate([g, g], axis=2)
    b4 = np.concatenate([beta, beta], axis=2)
    S4 = np.concatenate([S0, S0], axis=1)
    o4, _ = orc.fwd(q2, k2, v4, g4, b4, scale=sc, initial_state=S4)
    o4r, _ = orc.fwd(np.repeat(q2, 2, axis=2), np.repeat(k2, 2, axis=2), v4, g4, b4,
                     scale=sc, initial_state=S4)
    if not np.array_equal(o4, o4r):
        return False
    rng = np.random.default_rng(4)
    do = rng.standard_normal(o.shape)
    dht = rng.standard_normal(ht.shape)
    grads = orc.bwd(q, k, v, g, beta, do, dht, scale=sc, initial_state=S0)

    def loss(**over):
        a = dict(q=q, k=k, v=v, g=g, beta=beta, S0=S0)
        a.update(over)
        oo, hh = brute.fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], scale=sc,
                           initial_state=a["S0"])
        return float(np.sum(oo * do) + np.sum(hh * dht))

    eps = 1e-6
    for name, gr in zip(["q", "k", "v", "beta", "g", "S0"], grads):
        x = dict(q=q, k=k, v=v, g=g, beta=beta, S0=S0)[name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy(); xp[idx] += eps
            xm = x.copy(); xm[idx] -= eps
            fd[idx] = (loss(**{name: xp}) - loss(**{name: xm})) / (2 * eps)
        if np.linalg.norm(gr - fd) > 1e-6 * max(np.linalg.norm(fd), 1e-12):
            return False
    return True


def test_unmutated_oracle_passes_battery():
    assert pins_pass(token.Oracle(token._LIB if os.path.exists(token._LIB) else token.build()))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) >= 1, f"mutation site for {name} not found"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new, 1))
    lib = token.build(force=True, src=str(src), out=str(tmp_path / "libmutant.so"))
    assert not pins_pass(token.Oracle(lib)), f"mutant {name} slipped through the pins"

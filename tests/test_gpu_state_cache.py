"""GPU: the backward with the forward's state cache.

The training-mode forward can leave the state entering every chunk in a
cache that the backward then takes instead of recomputing those states.  The
cache path must give the same gradients as the recompute path (the same
segment passes compute the same states in both) and stay within the oracle
tolerance, across the passes that write the cache: the main pass, the fix-up
pass of segments past the first (forced short segments), the serial residual
pass (gates that do not decay), packed sequences with empty ones, an initial
state, fp32 and the in-library q/k normalisation.
"""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import (BLOCK_TOL, BLOCK_TOL_CANCEL, TOL, announce, block_rel_max,
                            oracle_bwd, oracle_fwd, rel, to_dev, token_mask)

pytestmark = pytest.mark.gpu

NAMES = ["dq", "dk", "dv", "db", "dg", "dh0"]


@pytest.fixture(scope="module")
def gdn():
    import gated_deltanet_chunked_gdn_amd as g
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    g.lib()
    return g


def both(gdn, p, cp_mode, l2=False):
    d = to_dev(p)
    kw = dict(scale=d["scale"], initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"],
              cp_mode=cp_mode, use_qk_l2norm_in_kernel=l2)
    cache = gdn.state_cache_empty(d["q"], d["v"], cu_seqlens=d["cu_seqlens"], cp_mode=cp_mode,
                                  use_qk_l2norm_in_kernel=l2)
    cache.fill_(255)  # NaN in bf16 and fp32: every entry must be written by the forward
    _, A, _, _, _ = gdn.chunk_gated_delta_rule_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                                   state_cache=cache, **kw)
    with_cache = gdn.chunk_gated_delta_rule_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], A,
                                                d["do"], dht=d["dht"], state_cache=cache, **kw)
    recompute = gdn.chunk_gated_delta_rule_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], A,
                                               d["do"], dht=d["dht"], **kw)
    # with a cache the backward reads neither A nor anything the forward's
    # intermediates hold: an inference-mode forward plus the cache suffices
    cache2 = gdn.state_cache_empty(d["q"], d["v"], cu_seqlens=d["cu_seqlens"], cp_mode=cp_mode,
                                   use_qk_l2norm_in_kernel=l2)
    gdn.chunk_gated_delta_rule_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                   return_intermediates=False, state_cache=cache2, **kw)
    no_a = gdn.chunk_gated_delta_rule_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], None,
                                          d["do"], dht=d["dht"], state_cache=cache2, **kw)
    torch.cuda.synchronize()
    for n, x, y in zip(NAMES, no_a, with_cache):
        assert torch.equal(x, y), f"{n}: backward with the cache depends on A"
    # both parts of the cache written: the states, then (at the next 256-byte
    # boundary) the per-chunk T
    es = d["q"].element_size()
    B, T = d["q"].shape[:2]
    Hv, K, V = d["v"].shape[2], d["q"].shape[3], d["v"].shape[3]
    if d["cu_seqlens"] is not None:
        lens = (d["cu_seqlens"][1:] - d["cu_seqlens"][:-1]).tolist()
        nc = sum((n + 63) // 64 for n in lens)
    else:
        nc = B * ((T + 63) // 64)
    n_st = nc * Hv * K * V * es
    t_off = (n_st + 255) // 256 * 256
    states = cache[:n_st].view(d["q"].dtype)
    tm = cache[t_off:t_off + nc * Hv * 64 * 64 * es].view(d["q"].dtype)
    end = t_off + nc * Hv * 64 * 64 * es
    assert not torch.isnan(states).any(), "state cache: states left unwritten"
    assert not torch.isnan(tm).any(), "state cache: T left unwritten"
    if l2:
        # then the normalised q, k rows and their factors, each at the next
        # 256-byte boundary: every row of unit norm, every factor 1 / |x|
        rows = d["q"].shape[0] * d["q"].shape[1] * d["q"].shape[2]
        al = lambda x: (x + 255) // 256 * 256
        qn_off = al(end)
        kn_off = al(qn_off + rows * K * es)
        rq_off = al(kn_off + rows * K * es)
        rk_off = al(rq_off + rows * 4)
        end = rk_off + rows * 4
        for off, f_off, x in ((qn_off, rq_off, d["q"]), (kn_off, rk_off, d["k"])):
            xn = cache[off:off + rows * K * es].view(d["q"].dtype).float().view(-1, K)
            fr = cache[f_off:f_off + rows * 4].view(torch.float32)
            raw = x.float().reshape(-1, K)
            assert torch.allclose(xn.norm(dim=1), torch.ones_like(fr), atol=2e-2)
            assert torch.allclose(fr, torch.rsqrt((raw * raw).sum(1) + 1e-6), rtol=1e-5)
    assert cache.numel() == end
    return with_cache, recompute


CASES = [
    # label, builder, dtype, cp_mode, l2
    ("bf16 T=300 cp=1", lambda: synth.custom(2, 300, 2, 4, 128, 128, dtype="bf16", seed=5,
                                             gate="slow", h0=True, grads=True), "bf16", 1, False),
    ("bf16 nodecay cp=1", lambda: synth.custom(1, 600, 2, 4, 64, 128, dtype="bf16", seed=6,
                                               gate="nodecay", h0=True, grads=True), "bf16", 1,
     False),
    ("bf16 varlen+empty cp=2", lambda: synth.custom(1, 0, 2, 4, 128, 128, dtype="bf16", seed=7,
                                                    gate="default", lengths=[0, 1, 64, 330, 0,
                                                                             700, 63],
                                                    h0=True, grads=True), "bf16", 2, False),
    ("bf16 auto", lambda: synth.custom(1, 1000, 2, 4, 128, 128, dtype="bf16", seed=8,
                                       gate="default", h0=False, grads=True), "bf16", -1, False),
    ("f32 cp=1", lambda: synth.custom(1, 200, 1, 3, 64, 32, dtype="f32", seed=9, gate="slow",
                                      h0=True, grads=True), "f32", 1, False),
    ("bf16 l2norm cp=1", lambda: synth.custom(1, 260, 2, 4, 128, 128, dtype="bf16", seed=10,
                                              gate="slow", h0=True, grads=True,
                                              normalize_qk=False), "bf16", 1, True),
    ("bf16 l2norm varlen+empty cp=2", lambda: synth.custom(1, 0, 2, 4, 128, 128, dtype="bf16",
                                                           seed=11, gate="default",
                                                           lengths=[0, 1, 64, 330, 0, 700, 63],
                                                           h0=True, grads=True,
                                                           normalize_qk=False), "bf16", 2, True),
    ("bf16 l2norm 3 v-heads per q/k head", lambda: synth.custom(1, 200, 1, 3, 128, 128,
                                                                dtype="bf16", seed=12,
                                                                gate="slow", h0=True, grads=True,
                                                                normalize_qk=False),
     "bf16", -1, True),
    ("f32 l2norm cp=1", lambda: synth.custom(1, 200, 1, 2, 64, 64, dtype="f32", seed=13,
                                             gate="slow", h0=True, grads=True,
                                             normalize_qk=False), "f32", 1, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_cache_matches_recompute_and_oracle(gdn, case):
    label, build, dtype, cp, l2 = case
    announce(f"state cache {label}")
    p = build()
    got, rec = both(gdn, p, cp, l2)
    for n, x, y in zip(NAMES, got, rec):
        # the cached states come from the forward's pass 1 and the recomputed
        # ones from the backward's state pass: two kernels, one recurrence, so
        # the gradients agree to the rounding of the bf16 states
        assert rel(x.float().cpu().numpy(), y.float().cpu().numpy()) <= TOL[dtype], n
    ref = oracle_bwd(p, qk_l2norm=l2)
    errs = {n: rel(x, r) for n, x, r in zip(NAMES, got, ref)}
    bad = {n: e for n, e in errs.items() if not e <= TOL[dtype]}
    assert not bad, f"{label}: {bad} (all: {errs})"


@pytest.mark.parametrize("l2", [False, True], ids=["plain", "l2norm"])
def test_full_hv64_t8192_cached_step(gdn, l2):
    """The benchmark's own step at its full size and in its launch
    configuration: the training forward fills the cache (no A, no g_cum), the
    backward takes it with A = None.  o, the final state and every gradient
    are checked against the oracle on whole q/k groups: v-heads 0, 1 (q/k
    head 0), 40, 41 (q/k head 20) and 62, 63 (q/k head 31).  Also with raw q,
    k normalised inside the library (the benchmark's --qk-l2norm step)."""
    w = synth.WORKLOADS["hv64_t8192"]
    p = synth.make(w, with_grads=True, normalize_qk=not l2)
    announce(f"full hv64_t8192 cached fwd+bwd l2={l2}")
    d = to_dev(p)
    kw = dict(scale=d["scale"], initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"],
              use_qk_l2norm_in_kernel=l2)
    cache = gdn.state_cache_empty(d["q"], d["v"], use_qk_l2norm_in_kernel=l2)
    _, A, o, _, ht = gdn.chunk_gated_delta_rule_fwd(
        d["q"], d["k"], d["v"], d["g"], d["beta"], output_final_state=True,
        return_intermediates=False, return_states=False, state_cache=cache, **kw)
    assert A is None
    got = gdn.chunk_gated_delta_rule_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], None,
                                         d["do"], dht=d["dht"], state_cache=cache, **kw)
    torch.cuda.synchronize()
    heads = [0, 1, 40, 41, 62, 63]
    mask = np.zeros((w.B, w.Hv), dtype=bool)
    mask[:, heads] = True
    tm = token_mask(p, mask)
    ro, rht = oracle_fwd(p, unit_mask=mask, qk_l2norm=l2)
    o_np = o.double().cpu().numpy()
    errs = {"o": rel(o_np[tm], ro[tm]),
            "ht": rel(ht.double().cpu().numpy()[mask], rht[mask])}
    blocks = {"o": block_rel_max(o_np, ro, tm)}
    ref = oracle_bwd(p, unit_mask=mask, qk_l2norm=l2)
    grp = w.Hv // w.Hq
    qk_heads = sorted({h // grp for h in heads})
    for n, x, r in zip(NAMES, got, ref):
        x = x.double().cpu().numpy()
        assert np.isfinite(x).all(), n
        if n in ("dq", "dk"):
            errs[n] = rel(x[:, :, qk_heads], r[:, :, qk_heads])
            blocks[n] = block_rel_max(x[:, :, qk_heads], r[:, :, qk_heads])
        elif n == "dh0":
            errs[n] = rel(x[mask], r[mask])
        else:
            errs[n] = rel(x[tm], r[tm])
            blocks[n] = block_rel_max(x, r, tm)
    announce("  rel " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()) +
             " | worst block " + " ".join(f"{n}={e:.2e}" for n, e in blocks.items()))
    bad = {n: e for n, e in errs.items() if not e <= TOL[w.dtype]}
    assert not bad, f"{bad} (all {errs})"
    btol = {n: (BLOCK_TOL_CANCEL if n in ("db", "dg") else BLOCK_TOL)[w.dtype] for n in blocks}
    bad = {n: e for n, e in blocks.items() if not e <= btol[n]}
    assert not bad, f"worst 64-token block: {bad} (all {blocks})"

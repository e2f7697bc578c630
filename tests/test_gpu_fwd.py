"""GPU forward parity: the HIP path through the C ABI vs the fp64 oracle.

Tolerance (relative Frobenius error over a whole output): 1e-5 for fp32
inputs, 1e-2 for bf16 inputs.  Full-size workloads compare every output of a
sample of (sequence, v-head) units that the oracle computes one by one.
"""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import (BLOCK_TOL, TOL, announce, block_rel_max, oracle_bwd, oracle_fwd, rel,
                            to_dev, token_mask)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import gated_deltanet_chunked_gdn_amd as g
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    g.lib()
    return g


def run_fwd(gdn, p, cp_mode=-1, want_inter=False):
    d = to_dev(p)
    out = gdn.chunk_gated_delta_rule_fwd(
        d["q"], d["k"], d["v"], d["g"], d["beta"], scale=d["scale"],
        initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"],
        output_final_state=True, return_intermediates=want_inter, cp_mode=cp_mode)
    torch.cuda.synchronize()
    return out


def test_mfma_selftest(gdn):
    announce("selftest")
    gdn.selftest()


def check(gdn, p, dtype, cp_mode=-1, label=""):
    announce(f"fwd {label} cp={cp_mode}")
    _, _, o, _, ht = run_fwd(gdn, p, cp_mode)
    ro, rht = oracle_fwd(p)
    eo, eh = rel(o, ro), rel(ht, rht)
    assert eo <= TOL[dtype], f"o rel err {eo:.3e} ({label})"
    assert eh <= TOL[dtype], f"final_state rel err {eh:.3e} ({label})"
    return eo, eh


def test_tiny_f32_workload(gdn):
    p = synth.make(synth.WORKLOADS["tiny_f32"])
    check(gdn, p, "f32", label="tiny_f32")


@pytest.mark.parametrize("gate", ["default", "slow", "nodecay"])
@pytest.mark.parametrize("cp", [0, 1, 2])
def test_tiny_f32_gates_and_cp(gdn, gate, cp):
    p = synth.make(synth.WORKLOADS["tiny_f32"], gate=gate, with_h0=True)
    check(gdn, p, "f32", cp_mode=cp, label=f"tiny_f32 {gate}")


def test_fixup_stops_on_relative_decay(gdn):
    """Gates that decay by about e^-5 a chunk: the correction pass crosses the
    2^-30 relative stop a few chunks into each 8-chunk segment, so every
    segment after the first exits early; fp32 at its 1e-5 bound against the
    oracle, forward and backward."""
    p = synth.custom(1, 2048, 1, 2, 32, 32, dtype="f32", seed=21, gate="moderate", h0=True,
                     grads=True)
    check(gdn, p, "f32", cp_mode=8, label="moderate gates, 8-chunk segments")
    d = to_dev(p)
    got = gdn.chunk_gated_delta_rule_bwd(
        d["q"], d["k"], d["v"], d["g"], d["beta"], None, d["do"], dht=d["dht"],
        scale=d["scale"], initial_state=d["initial_state"], cp_mode=8)
    torch.cuda.synchronize()
    ref = oracle_bwd(p)
    errs = {n: rel(x, r) for n, x, r in zip(["dq", "dk", "dv", "db", "dg", "dh0"], got, ref)}
    bad = {n: e for n, e in errs.items() if not e <= TOL["f32"]}
    assert not bad, f"{bad} (all {errs})"


@pytest.mark.parametrize("T", [1, 63, 64, 65, 130, 257])
@pytest.mark.parametrize("kv", [(128, 128), (64, 64), (64, 128), (128, 64), (32, 32)])
def test_bf16_ragged_lengths(gdn, T, kv):
    K, V = kv
    p = synth.custom(2, T, 2, 4, K, V, dtype="bf16", seed=T, gate="slow", h0=True)
    check(gdn, p, "bf16", cp_mode=1, label=f"T={T} K={K} V={V}")


@pytest.mark.parametrize("kv", [(32, 32), (64, 64), (32, 64), (64, 32)])
def test_f32_shapes(gdn, kv):
    K, V = kv
    p = synth.custom(1, 150, 1, 3, K, V, dtype="f32", seed=3, gate="slow", h0=True)
    check(gdn, p, "f32", cp_mode=1, label=f"f32 K={K} V={V}")


@pytest.mark.parametrize("gate", ["default", "slow", "nodecay"])
def test_varlen_with_empty_and_short(gdn, gate):
    lengths = [0, 1, 64, 130, 0, 700, 63, 129]
    p = synth.custom(1, 0, 2, 4, 128, 128, dtype="bf16", seed=11, gate=gate,
                     lengths=lengths, h0=True)
    for cp in (0, 2, -1):
        check(gdn, p, "bf16", cp_mode=cp, label=f"varlen {gate}")


def test_gqa_grouping_matches_repeated_heads(gdn):
    p = synth.custom(1, 300, 2, 6, 64, 64, dtype="bf16", seed=4, gate="slow", h0=True)
    _, _, o1, _, h1 = run_fwd(gdn, p, cp_mode=2)
    p2 = dict(p)
    p2["q"] = p["q"].repeat_interleave(3, dim=2)
    p2["k"] = p["k"].repeat_interleave(3, dim=2)
    _, _, o2, _, h2 = run_fwd(gdn, p2, cp_mode=2)
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


def test_cp_split_agrees_with_unsplit_and_is_deterministic(gdn):
    p = synth.custom(1, 4096, 2, 4, 128, 128, dtype="bf16", seed=8, gate="slow", h0=True)
    _, _, o0, _, h0 = run_fwd(gdn, p, cp_mode=0)
    for cp in (1, 3, 16):
        _, _, o1, _, h1 = run_fwd(gdn, p, cp_mode=cp)
        assert rel(o1, o0.double().cpu().numpy()) <= 1e-2
        assert rel(h1, h0.double().cpu().numpy()) <= 1e-2
    _, _, oa, _, ha = run_fwd(gdn, p, cp_mode=3)
    _, _, ob, _, hb = run_fwd(gdn, p, cp_mode=3)
    assert torch.equal(oa, ob) and torch.equal(ha, hb)


@pytest.mark.parametrize("gate", ["default", "slow", "nodecay"])
def test_intermediates_gate_cumsum_and_inverse(gdn, gate):
    """g_cum, A and the per-chunk states h against the oracle's chunked
    intermediates (fp64).  With one chunk per segment (cp_mode=1) every h
    after the first passes through the fix-up and serial carry; the slow and
    no-decay gates keep those corrections large."""
    from oracle import chunked
    p = synth.custom(1, 150, 1, 2, 64, 64, dtype="f32", seed=2, gate=gate)
    g_cum, A, o, h, ht = run_fwd(gdn, p, cp_mode=1, want_inter=True)
    q, k, v, g, b = (p[n][0].double().numpy() for n in ("q", "k", "v", "g", "beta"))
    for hh in range(2):
        _, _, inter = chunked.chunk_forward_one(q[:, 0], k[:, 0], v[:, hh], g[:, hh],
                                                b[:, hh], p["scale"],
                                                np.zeros((64, 64)), 64)
        for c, it in enumerate(inter):
            s, n = 64 * c, len(it["gamma"])
            assert rel(g_cum[0, s:s + n, hh], it["gamma"]) < 1e-5
            assert rel(A[0, s:s + n, hh, :n], it["T"]) < 1e-5
            assert rel(h[c, hh], it["S_in"]) < 1e-5 or np.abs(it["S_in"]).max() == 0


# ------------------------------------------------------ full-size workloads

def _sampled(gdn, name, heads, gate="default", T=None, cp=-1):
    w = synth.WORKLOADS[name]
    p = synth.make(w, gate=gate, T=T)
    N = len(p["lengths"]) if "lengths" in p else w.B
    mask = np.zeros((N, w.Hv), dtype=bool)
    mask[:, heads] = True
    announce(f"full {name} gate={gate} T={T} cp={cp}")
    _, _, o, _, ht = run_fwd(gdn, p, cp_mode=cp)
    ro, rht = oracle_fwd(p, unit_mask=mask)
    tm = token_mask(p, mask)
    o_np = o.double().cpu().numpy()
    eo = rel(o_np[tm], ro[tm])
    eh = rel(ht.double().cpu().numpy()[mask], rht[mask])
    # per 64-token block of each sampled head, and per (sequence, head) state
    bo = block_rel_max(o_np, ro, tm)
    ht_np = ht.double().cpu().numpy()
    bh = max(rel(ht_np[n, hh], rht[n, hh]) for n, hh in zip(*np.nonzero(mask)))
    announce(f"  o rel {eo:.2e} (worst block {bo:.2e}), final {eh:.2e} (worst unit {bh:.2e})")
    assert eo <= TOL[w.dtype], f"{name} o rel err {eo:.3e}"
    assert eh <= TOL[w.dtype], f"{name} final rel err {eh:.3e}"
    assert bo <= BLOCK_TOL[w.dtype], f"{name} o worst 64-token block rel err {bo:.3e}"
    assert bh <= BLOCK_TOL[w.dtype], f"{name} worst final state rel err {bh:.3e}"
    assert np.isfinite(o_np).all()


def test_full_hv64_t8192(gdn):
    _sampled(gdn, "hv64_t8192", heads=[0, 1, 17, 40, 63])


def test_full_hv64_t8192_slow_decay(gdn):
    _sampled(gdn, "hv64_t8192", heads=[0, 1, 33, 62], gate="slow")


def test_full_hv8_t65536(gdn):
    _sampled(gdn, "hv8_t65536", heads=[0, 5])


def test_hv8_long_slow_decay_cp_fixup(gdn):
    # slow decay: the segment fix-ups run over whole segments
    _sampled(gdn, "hv8_t65536", heads=[3], gate="slow", T=16384)


def test_hv8_t65536_full_length_slow_decay(gdn):
    # the whole 65536-token sequence (1024 chunks, every segment boundary of
    # the automatic split) with a state that survives many chunks
    _sampled(gdn, "hv8_t65536", heads=[3], gate="slow")


def test_hv8_long_no_decay(gdn):
    _sampled(gdn, "hv8_t65536", heads=[2], gate="nodecay", T=8192)


def test_full_varlen16_hv32(gdn):
    _sampled(gdn, "varlen16_hv32", heads=[0, 31])


def test_full_varlen16_hv32_slow(gdn):
    _sampled(gdn, "varlen16_hv32", heads=[7], gate="slow")


@pytest.mark.parametrize("dtype,K,V,T,T1", [("bf16", 128, 128, 3000, 1234),
                                            ("bf16", 64, 64, 700, 64),
                                            ("f32", 32, 32, 400, 130)])
def test_resume_invariance(gdn, dtype, K, V, T, T1):
    """[0, T1) then [T1, T) with the first call's final state as the second
    call's initial state equals one call over [0, T)."""
    p = synth.custom(2, T, 2, 4, K, V, dtype=dtype, seed=31, gate="slow", h0=True)
    d = to_dev(p)
    announce(f"resume {dtype} K={K} V={V} T={T} T1={T1}")

    def fwd(sl, h0):
        q, k, v, g, b = (d[n][:, sl].contiguous() for n in ("q", "k", "v", "g", "beta"))
        return gdn.chunk_gated_delta_rule(q, k, v, g, b, scale=d["scale"], initial_state=h0,
                                          output_final_state=True)

    o, ht = fwd(slice(0, T), d["initial_state"])
    o1, h1 = fwd(slice(0, T1), d["initial_state"])
    o2, h2 = fwd(slice(T1, T), h1)
    torch.cuda.synchronize()
    o12 = torch.cat([o1, o2], dim=1).double().cpu().numpy()
    ref = o.double().cpu().numpy()
    assert rel(o12, ref) <= TOL[dtype]
    assert rel(h2, ht.double().cpu().numpy()) <= TOL[dtype]
    ro, rht = oracle_fwd(p)
    assert rel(o12, ro) <= TOL[dtype] and rel(h2, rht) <= TOL[dtype]

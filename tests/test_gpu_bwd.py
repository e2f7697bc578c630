"""GPU backward parity: dq, dk, dv, dbeta, dg, dh0 of the HIP path (through the
C ABI) against the fp64 oracle's reverse mode.

Tolerance (relative Frobenius error over a whole gradient): 1e-5 for fp32
inputs, 1e-2 for bf16 inputs.  dq and dk are summed over each q/k group, so
sampled full-size checks select whole groups.
"""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import (BLOCK_TOL, BLOCK_TOL_CANCEL, TOL, announce, block_rel_max,
                            oracle_bwd, rel, to_dev, token_mask)

pytestmark = pytest.mark.gpu

NAMES = ["dq", "dk", "dv", "db", "dg", "dh0"]


@pytest.fixture(scope="module")
def gdn():
    import gated_deltanet_chunked_gdn_amd as g
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    g.lib()
    return g


def run_bwd(gdn, p, cp_mode=-1, use_A=False):
    d = to_dev(p)
    A = None
    if use_A:
        _, A, _, _, _ = gdn.chunk_gated_delta_rule_fwd(
            d["q"], d["k"], d["v"], d["g"], d["beta"], scale=d["scale"],
            initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"], cp_mode=cp_mode)
    out = gdn.chunk_gated_delta_rule_bwd(
        d["q"], d["k"], d["v"], d["g"], d["beta"], A, d["do"], dht=d["dht"],
        scale=d["scale"], initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"],
        cp_mode=cp_mode)
    torch.cuda.synchronize()
    return out


def check(gdn, p, dtype, cp_mode=-1, label="", use_A=False):
    announce(f"bwd {label} cp={cp_mode} A={use_A}")
    got = run_bwd(gdn, p, cp_mode, use_A)
    ref = oracle_bwd(p)
    errs = {n: rel(x, r) for n, x, r in zip(NAMES, got, ref)}
    bad = {n: e for n, e in errs.items() if not e <= TOL[dtype]}
    assert not bad, f"{label}: {bad} (all: {errs})"
    return errs


@pytest.mark.parametrize("gate", ["default", "slow", "nodecay"])
def test_tiny_f32(gdn, gate):
    p = synth.make(synth.WORKLOADS["tiny_f32"], gate=gate, with_h0=True, with_grads=True)
    for cp in (0, 1, -1):
        check(gdn, p, "f32", cp_mode=cp, label=f"tiny_f32 {gate}")


@pytest.mark.parametrize("kv", [(32, 32), (64, 64), (32, 64), (64, 32)])
def test_f32_shapes(gdn, kv):
    K, V = kv
    p = synth.custom(1, 150, 1, 3, K, V, dtype="f32", seed=3, gate="slow", h0=True, grads=True)
    check(gdn, p, "f32", cp_mode=1, label=f"f32 K={K} V={V}")


@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
@pytest.mark.parametrize("kv", [(128, 128), (64, 64), (64, 128), (128, 64), (32, 32)])
def test_bf16_ragged(gdn, T, kv):
    K, V = kv
    p = synth.custom(2, T, 2, 4, K, V, dtype="bf16", seed=T + 7, gate="slow", h0=True,
                     grads=True)
    check(gdn, p, "bf16", cp_mode=1, label=f"T={T} K={K} V={V}")


@pytest.mark.parametrize("gate", ["default", "slow", "nodecay"])
def test_varlen_with_empty(gdn, gate):
    lengths = [0, 1, 64, 130, 0, 400, 63]
    p = synth.custom(1, 0, 2, 4, 128, 128, dtype="bf16", seed=21, gate=gate,
                     lengths=lengths, h0=True, grads=True)
    for cp in (0, 2, -1):
        check(gdn, p, "bf16", cp_mode=cp, label=f"varlen {gate}")


def test_given_A_matches_recomputed(gdn):
    p = synth.custom(1, 300, 2, 4, 64, 64, dtype="bf16", seed=5, gate="slow", h0=True,
                     grads=True)
    a = run_bwd(gdn, p, cp_mode=2, use_A=False)
    b = run_bwd(gdn, p, cp_mode=2, use_A=True)
    for n, x, y in zip(NAMES, a, b):
        assert rel(y, x.double().cpu().numpy()) < 1e-2, n
    check(gdn, p, "bf16", cp_mode=2, label="given A", use_A=True)


def test_bwd_deterministic_and_cp_invariant(gdn):
    p = synth.custom(1, 2048, 2, 4, 128, 128, dtype="bf16", seed=9, gate="slow", h0=True,
                     grads=True)
    a = run_bwd(gdn, p, cp_mode=4)
    b = run_bwd(gdn, p, cp_mode=4)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    c = run_bwd(gdn, p, cp_mode=0)
    for n, x, y in zip(NAMES, a, c):
        assert rel(x, y.double().cpu().numpy()) < 1e-2, n


def _sampled_bwd(gdn, heads, gate="default", T=None, cp=-1):
    w = synth.WORKLOADS["bwd_b2_t16384_hv16"]
    p = synth.make(w, gate=gate, T=T, with_h0=gate != "default")
    N = w.B
    mask = np.zeros((N, w.Hv), dtype=bool)
    mask[:, heads] = True
    announce(f"full bwd gate={gate} T={T} heads={heads}")
    got = run_bwd(gdn, p, cp_mode=cp)
    ref = oracle_bwd(p, unit_mask=mask)
    grp = w.Hv // w.Hq
    qk_heads = sorted({h // grp for h in heads})
    tm = token_mask(p, mask)
    errs, blocks = {}, {}
    for n, x, r in zip(NAMES, got, ref):
        x = x.double().cpu().numpy()
        if n in ("dq", "dk"):
            errs[n] = rel(x[:, :, qk_heads], r[:, :, qk_heads])
            blocks[n] = block_rel_max(x[:, :, qk_heads], r[:, :, qk_heads])
        elif n == "dh0":
            errs[n] = rel(x[mask], r[mask])
            blocks[n] = max(rel(x[b, hh], r[b, hh]) for b, hh in zip(*np.nonzero(mask)))
        else:
            errs[n] = rel(x[tm], r[tm])
            blocks[n] = block_rel_max(x, r, tm)
    announce("  rel " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()) +
             " | worst block " + " ".join(f"{n}={e:.2e}" for n, e in blocks.items()))
    bad = {n: e for n, e in errs.items() if not e <= TOL[w.dtype]}
    assert not bad, f"{bad} (all {errs})"
    btol = {n: (BLOCK_TOL_CANCEL if n in ("db", "dg") else BLOCK_TOL)[w.dtype] for n in NAMES}
    bad = {n: e for n, e in blocks.items() if not e <= btol[n]}
    assert not bad, f"worst 64-token block: {bad} (all {blocks})"


def test_full_bwd_b2_t16384_hv16(gdn):
    _sampled_bwd(gdn, heads=[2, 3, 14, 15])


def test_full_bwd_slow_decay(gdn):
    _sampled_bwd(gdn, heads=[4, 5], gate="slow", T=4096)

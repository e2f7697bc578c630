"""GPU parity of the in-library q/k L2 normalisation (use_qk_l2norm_in_kernel):
raw (unnormalised) q, k in; the oracle normalises in fp64 (oracle.l2norm) and
takes dq, dk back through the normalisation.  Tolerances as elsewhere
(relative Frobenius error 1e-5 fp32, 1e-2 bf16)."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import TOL, announce, rel, to_dev
from oracle import token

pytestmark = pytest.mark.gpu

NAMES = ["dq", "dk", "dv", "db", "dg", "dh0"]


@pytest.fixture(scope="module")
def gdn():
    import gated_deltanet_chunked_gdn_amd as g
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    g.lib()
    return g


def _cu(p):
    return None if p["cu_seqlens"] is None else p["cu_seqlens"].numpy()


def _check_fwd(gdn, p, dtype, cp, label):
    announce(f"l2norm fwd {label} cp={cp}")
    d = to_dev(p)
    _, _, o, _, ht = gdn.chunk_gated_delta_rule_fwd(
        d["q"], d["k"], d["v"], d["g"], d["beta"], scale=d["scale"],
        initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"], cp_mode=cp,
        use_qk_l2norm_in_kernel=True)
    torch.cuda.synchronize()
    ro, rht = token.fwd(p["q"], p["k"], p["v"], p["g"], p["beta"], scale=p["scale"],
                        initial_state=p["initial_state"], cu_seqlens=_cu(p), qk_l2norm=True)
    assert rel(o, ro) <= TOL[dtype], label
    assert rel(ht, rht) <= TOL[dtype], label


def _check_bwd(gdn, p, dtype, cp, label):
    announce(f"l2norm bwd {label} cp={cp}")
    d = to_dev(p)
    got = gdn.chunk_gated_delta_rule_bwd(
        d["q"], d["k"], d["v"], d["g"], d["beta"], None, d["do"], dht=d["dht"],
        scale=d["scale"], initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"],
        cp_mode=cp, use_qk_l2norm_in_kernel=True)
    torch.cuda.synchronize()
    ref = token.bwd(p["q"], p["k"], p["v"], p["g"], p["beta"], p["do"], p["dht"],
                    scale=p["scale"], initial_state=p["initial_state"], cu_seqlens=_cu(p),
                    qk_l2norm=True)
    errs = {n: rel(x, r) for n, x, r in zip(NAMES, got, ref)}
    bad = {n: e for n, e in errs.items() if not e <= TOL[dtype]}
    assert not bad, f"{label}: {bad} (all {errs})"


@pytest.mark.parametrize("kv", [(128, 128), (64, 64), (32, 32), (128, 64)])
def test_bf16(gdn, kv):
    K, V = kv
    p = synth.custom(2, 300, 2, 4, K, V, dtype="bf16", seed=41, gate="slow", h0=True,
                     grads=True, normalize_qk=False)
    _check_fwd(gdn, p, "bf16", -1, f"bf16 K={K} V={V}")
    _check_bwd(gdn, p, "bf16", 2, f"bf16 K={K} V={V}")


@pytest.mark.parametrize("kv", [(32, 32), (64, 64)])
def test_f32(gdn, kv):
    K, V = kv
    p = synth.custom(1, 200, 1, 2, K, V, dtype="f32", seed=42, gate="slow", h0=True,
                     grads=True, normalize_qk=False)
    _check_fwd(gdn, p, "f32", 1, f"f32 K={K} V={V}")
    _check_bwd(gdn, p, "f32", 1, f"f32 K={K} V={V}")


def test_varlen(gdn):
    p = synth.custom(1, 0, 2, 4, 128, 128, dtype="bf16", seed=43, gate="default",
                     lengths=[70, 0, 257, 1], h0=True, grads=True, normalize_qk=False)
    _check_fwd(gdn, p, "bf16", -1, "varlen")
    _check_bwd(gdn, p, "bf16", -1, "varlen")


def test_matches_prenormalised_inputs(gdn):
    """The fused path on raw rows and the plain path on rows normalised in
    fp32 by torch agree to bf16 rounding (the inputs are then the same up to
    one rounding of the normalised rows)."""
    p = synth.custom(1, 512, 4, 8, 128, 128, dtype="bf16", seed=44, normalize_qk=False)
    d = to_dev(p)
    o1, _ = gdn.chunk_gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                       scale=d["scale"], use_qk_l2norm_in_kernel=True)
    qn = (d["q"].float() * torch.rsqrt((d["q"].float() ** 2).sum(-1, keepdim=True) + 1e-6))
    kn = (d["k"].float() * torch.rsqrt((d["k"].float() ** 2).sum(-1, keepdim=True) + 1e-6))
    o2, _ = gdn.chunk_gated_delta_rule(qn.bfloat16(), kn.bfloat16(), d["v"], d["g"],
                                       d["beta"], scale=d["scale"])
    torch.cuda.synchronize()
    assert rel(o1, o2.double().cpu().numpy()) < 5e-3

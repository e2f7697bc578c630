"""GPU parity along the pages' head-count sweep (H_v in 64, 48, 32, 24, 16, 8
with H_q = H_v / 2), including the non-power-of-two counts 48 and 24: the
automatic context-parallel split and the workgroup mapping change with the
head count.  Sampled whole q/k groups are checked against the oracle."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import TOL, announce, oracle_bwd, oracle_fwd, rel, to_dev, token_mask

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import gated_deltanet_chunked_gdn_amd as g
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    g.lib()
    return g


def _groups(hv):
    # first and last q/k group (2 v-heads each)
    return [0, 1, hv - 2, hv - 1]


@pytest.mark.parametrize("hv", [48, 24, 16, 8])
@pytest.mark.parametrize("gate,T", [("default", 8192), ("slow", 4096)])
def test_sweep_forward(gdn, hv, gate, T):
    w = synth.sweep_workload(hv)
    p = synth.make(w, gate=gate, T=T, with_grads=False)
    heads = _groups(hv)
    mask = np.zeros((1, hv), dtype=bool)
    mask[:, heads] = True
    announce(f"sweep fwd hv={hv} gate={gate} T={T}")
    d = to_dev(p)
    o, ht = gdn.chunk_gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                       scale=d["scale"], output_final_state=True)
    torch.cuda.synchronize()
    ro, rht = oracle_fwd(p, unit_mask=mask)
    tm = token_mask(p, mask)
    assert rel(o.double().cpu().numpy()[tm], ro[tm]) <= TOL["bf16"]
    assert rel(ht.double().cpu().numpy()[mask], rht[mask]) <= TOL["bf16"]


@pytest.mark.parametrize("hv", [48, 24])
def test_sweep_backward(gdn, hv):
    w = synth.sweep_workload(hv)
    p = synth.make(w, gate="slow", T=2048, with_h0=True)
    heads = _groups(hv)
    mask = np.zeros((1, hv), dtype=bool)
    mask[:, heads] = True
    announce(f"sweep bwd hv={hv}")
    d = to_dev(p)
    got = gdn.chunk_gated_delta_rule_bwd(
        d["q"], d["k"], d["v"], d["g"], d["beta"], None, d["do"], dht=d["dht"],
        scale=d["scale"], initial_state=d["initial_state"])
    torch.cuda.synchronize()
    ref = oracle_bwd(p, unit_mask=mask)
    qk_heads = sorted({h // 2 for h in heads})
    tm = token_mask(p, mask)
    for n, x, r in zip(["dq", "dk", "dv", "db", "dg", "dh0"], got, ref):
        x = x.double().cpu().numpy()
        if n in ("dq", "dk"):
            e = rel(x[:, :, qk_heads], r[:, :, qk_heads])
        elif n == "dh0":
            e = rel(x[mask], r[mask])
        else:
            e = rel(x[tm], r[tm])
        assert e <= TOL["bf16"], (n, e)

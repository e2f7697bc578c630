"""The Python binding rejects malformed arguments before any launch.

Every check here raises from the argument checks of the binding, which run
before the library is asked to enqueue anything; the tensors are CPU tensors,
so a check that let one through would stop at the final device check instead
(and the message would say so).
"""
import pytest
import torch

import gated_deltanet_chunked_gdn_amd as gdn


def inputs(B=1, T=70, Hq=2, Hv=4, K=32, V=32, dt=torch.bfloat16):
    g = torch.Generator().manual_seed(0)
    q = torch.randn(B, T, Hq, K, generator=g).to(dt)
    k = torch.randn(B, T, Hq, K, generator=g).to(dt)
    v = torch.randn(B, T, Hv, V, generator=g).to(dt)
    gg = -torch.rand(B, T, Hv, generator=g)
    beta = torch.rand(B, T, Hv, generator=g).to(dt)
    do = torch.randn(B, T, Hv, V, generator=g).to(dt)
    return q, k, v, gg, beta, do


def bwd(**over):
    q, k, v, g, beta, do = inputs()
    args = dict(q=q, k=k, v=v, g=g, beta=beta, A=None, do=do, dht=None, initial_state=None)
    args.update(over)
    return gdn.chunk_gated_delta_rule_bwd(
        args["q"], args["k"], args["v"], args["g"], args["beta"], args["A"], args["do"],
        dht=args["dht"], initial_state=args["initial_state"])


def test_valid_arguments_reach_the_device_check():
    with pytest.raises(ValueError, match="on the GPU"):
        bwd()
    q, k, v, g, beta, _ = inputs()
    with pytest.raises(ValueError, match="on the GPU"):
        gdn.chunk_gated_delta_rule_fwd(q, k, v, g, beta)


@pytest.mark.parametrize("do,msg", [
    (torch.zeros(1, 70, 4, 32, dtype=torch.float32), "do must have"),   # wrong dtype
    (torch.zeros(1, 70, 4, 16, dtype=torch.bfloat16), "do must have"),  # wrong V
    (torch.zeros(1, 69, 4, 32, dtype=torch.bfloat16), "do must have"),  # wrong T
    (None, "do must have"),
])
def test_bwd_rejects_bad_do(do, msg):
    with pytest.raises(ValueError, match=msg):
        bwd(do=do)


@pytest.mark.parametrize("A", [
    torch.zeros(1, 70, 4, 64, dtype=torch.bfloat16),   # dtype
    torch.zeros(1, 70, 4, 32, dtype=torch.float32),    # last dimension is the chunk, 64
    torch.zeros(1, 70, 2, 64, dtype=torch.float32),    # H_q heads instead of H_v
])
def test_bwd_rejects_bad_A(A):
    with pytest.raises(ValueError, match="A must be float32"):
        bwd(A=A)


@pytest.mark.parametrize("name", ["dht", "initial_state"])
@pytest.mark.parametrize("x", [
    torch.zeros(2, 4, 32, 32, dtype=torch.float32),    # [B] given where N = 1 ... one too many
    torch.zeros(1, 4, 32, 32, dtype=torch.bfloat16),   # dtype
    torch.zeros(1, 2, 32, 32, dtype=torch.float32),    # H_q instead of H_v
])
def test_bwd_rejects_bad_states(name, x):
    with pytest.raises(ValueError, match=name):
        bwd(**{name: x})


def test_bwd_state_shape_follows_cu_seqlens():
    """With cu_seqlens the states are per sequence: a [B, ...] state with
    N != B sequences is rejected (a kernel would read past its end)."""
    q, k, v, g, beta, do = inputs(T=100)
    cu = torch.tensor([0, 30, 100], dtype=torch.int32)
    dht = torch.zeros(1, 4, 32, 32)
    with pytest.raises(ValueError, match="dht"):
        gdn.chunk_gated_delta_rule_bwd(q, k, v, g, beta, None, do, dht=dht, cu_seqlens=cu)
    with pytest.raises(ValueError, match="initial_state"):
        gdn.chunk_gated_delta_rule_fwd(q, k, v, g, beta, initial_state=dht, cu_seqlens=cu)


def test_fwd_rejects_mixed_dtypes():
    q, k, v, g, beta, _ = inputs()
    with pytest.raises(TypeError):
        gdn.chunk_gated_delta_rule_fwd(q.float(), k, v, g, beta)
    with pytest.raises(TypeError):
        gdn.chunk_gated_delta_rule_fwd(q, k, v, g.double(), beta)

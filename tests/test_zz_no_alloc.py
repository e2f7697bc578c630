"""The forward entry point that allocates nothing (gdn_chunk_fwd_noalloc):
its scratch is the library's fixed device array instead of a caller
workspace.  Through the C ABI it must give what gdn_chunk_fwd gives on the
same inputs (the same kernels, so bit for bit) and stay within the oracle's
tolerance, on two calls in a row, the second with a smaller problem (the
array keeps the first call's contents)."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import TOL, announce, oracle_fwd, rel, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import gated_deltanet_chunked_gdn_amd as g
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    L = g.lib()
    P = ctypes.c_void_p
    L.gdn_chunk_fwd_noalloc.argtypes = [ctypes.POINTER(g.GdnProblem)] + [P] * 13
    L.gdn_chunk_fwd_noalloc.restype = ctypes.c_int
    L.gdn_chunk_fwd_noalloc_max_bytes.restype = ctypes.c_size_t
    return g


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def both(gdn, p):
    """o and the final state from gdn_chunk_fwd (torch workspace) and from
    gdn_chunk_fwd_noalloc, on the same device inputs."""
    d = to_dev(p)
    L = gdn.lib()
    pr = gdn._Prepared(d["q"], d["v"], d["scale"], d["cu_seqlens"], -1)
    N, Hv, K, V = pr.N, d["v"].shape[2], d["q"].shape[3], d["v"].shape[3]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = []
    for noalloc in (False, True):
        o = torch.full_like(d["v"], float("nan"))
        ht = torch.full((N, Hv, K, V), float("nan"), device="cuda")
        args = [ctypes.byref(pr.prob), _ptr(d["q"]), _ptr(d["k"]), _ptr(d["v"]), _ptr(d["g"]),
                _ptr(d["beta"]), _ptr(d["initial_state"]), _ptr(o), _ptr(ht), None, None, None,
                None]
        if noalloc:
            rc = L.gdn_chunk_fwd_noalloc(*args, stream)
        else:
            n = L.gdn_chunk_fwd_workspace_size(ctypes.byref(pr.prob))
            assert n <= L.gdn_chunk_fwd_noalloc_max_bytes()
            ws = torch.empty(n, dtype=torch.uint8, device="cuda")
            rc = L.gdn_chunk_fwd(*args, _ptr(ws), n, stream)
        assert rc == 0, gdn.last_error()
        torch.cuda.synchronize()
        out.append((o, ht))
    return out


@pytest.mark.parametrize("case", [
    # (label, problem): the second is smaller than the first
    ("bf16 K=V=128 T=3000 h0 slow", dict(B=1, T=3000, Hq=2, Hv=4, K=128, V=128, dtype="bf16",
                                         gate="slow", h0=True, seed=41)),
    ("bf16 K=V=128 T=700 varlen", dict(B=1, T=0, Hq=2, Hv=4, K=128, V=128, dtype="bf16",
                                       gate="default", h0=True, seed=42,
                                       lengths=[300, 0, 65, 335])),
    ("f32 K=V=32 T=200", dict(B=2, T=200, Hq=1, Hv=2, K=32, V=32, dtype="f32", gate="slow",
                              h0=False, seed=43)),
])
def test_noalloc_matches_workspace_entry_point(gdn, case):
    label, kw = case
    announce(f"noalloc {label}")
    p = synth.custom(kw["B"], kw["T"], kw["Hq"], kw["Hv"], kw["K"], kw["V"], dtype=kw["dtype"],
                     seed=kw["seed"], gate=kw["gate"], h0=kw["h0"], lengths=kw.get("lengths"))
    (o1, h1), (o2, h2) = both(gdn, p)
    assert torch.equal(o1, o2), f"{label}: o differs from gdn_chunk_fwd"
    assert torch.equal(h1, h2), f"{label}: final state differs from gdn_chunk_fwd"
    ro, rht = oracle_fwd(p)
    tol = TOL[kw["dtype"]]
    assert rel(o2, ro) <= tol and rel(h2, rht) <= tol


def test_noalloc_rejects_a_problem_beyond_its_scratch(gdn):
    L = gdn.lib()
    big = gdn.GdnProblem(1, 1 << 20, 8, 16, 128, 128, 1, gdn.GDN_BF16, 0.088, None, None, -1, 0)
    assert L.gdn_chunk_fwd_workspace_size(ctypes.byref(big)) > L.gdn_chunk_fwd_noalloc_max_bytes()
    P = ctypes.c_void_p
    rc = L.gdn_chunk_fwd_noalloc(ctypes.byref(big), *([P(256)] * 6), P(256), None, None, None,
                                 None, None, None)
    assert rc == 4 and "scratch" in gdn.last_error()

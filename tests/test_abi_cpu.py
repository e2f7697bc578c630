"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad problems with the documented codes before
any HIP call."""
import ctypes
import os
import re

import pytest

import gated_deltanet_chunked_gdn_amd as gdn

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "gdn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = gdn.lib()
    names = declared_functions()
    assert len(names) >= 7
    for n in names:
        assert hasattr(lib, n), n


def prob(**kw):
    d = dict(B=1, T=256, Hq=2, Hv=4, K=128, V=128, N=1, dtype=gdn.GDN_BF16, scale=0.088,
             cu_seqlens=None, cu_seqlens_host=None, cp_mode=-1)
    d.update(kw)
    return gdn.GdnProblem(**d)


def ws(p):
    return gdn.lib().gdn_chunk_fwd_workspace_size(ctypes.byref(p))


def fwd_rc(p, ptr=16, wsb=1 << 30, workspace=1 << 20, o=None, cache=None):
    L = gdn.lib()
    P = ctypes.c_void_p
    return L.gdn_chunk_fwd(ctypes.byref(p), P(ptr), P(ptr), P(ptr), P(ptr), P(ptr), None,
                           P(ptr if o is None else o), None, None, None, None, cache,
                           P(workspace), wsb, None)


def test_valid_problem_sizes():
    p = prob()
    assert ws(p) > 0
    assert gdn.lib().gdn_chunk_bwd_workspace_size(ctypes.byref(p)) > ws(p)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), 1), (dict(Hq=0), 1), (dict(K=-1), 1),
    (dict(Hq=3, Hv=4), 2), (dict(K=96), 2), (dict(V=256), 2), (dict(dtype=7), 2),
    (dict(dtype=gdn.GDN_F32, K=128, V=128), 2),
    (dict(N=2), 1), (dict(cp_mode=-5), 1),
])
def test_invalid_problems(kw, code):
    p = prob(**kw)
    assert ws(p) == 0
    assert fwd_rc(p) == code
    assert gdn.last_error() != ""


def test_cu_seqlens_validation():
    import numpy as np
    good = np.array([0, 10, 10, 256], dtype=np.int32)
    host = good.ctypes.data_as(ctypes.c_void_p)
    p = prob(N=3, cu_seqlens=16, cu_seqlens_host=host.value)
    assert ws(p) > 0
    assert gdn.lib().gdn_plan_segments(ctypes.byref(p)) >= 2
    bad_cases = [np.array([1, 10, 20, 256], np.int32), np.array([0, 20, 10, 256], np.int32),
                 np.array([0, 10, 20, 255], np.int32)]
    for arr in bad_cases:
        h = arr.ctypes.data_as(ctypes.c_void_p)
        p = prob(N=3, cu_seqlens=16, cu_seqlens_host=h.value)
        assert ws(p) == 0 and fwd_rc(p) == 1
    # device pointer without host copy, B != 1, host copy without device pointer
    assert fwd_rc(prob(N=3, cu_seqlens=16)) == 1
    assert fwd_rc(prob(B=2, N=3, cu_seqlens=16, cu_seqlens_host=host.value)) == 1
    assert fwd_rc(prob(cu_seqlens_host=host.value)) == 1


def test_null_and_misaligned_pointers_and_workspace():
    p = prob()
    L = gdn.lib()
    P = ctypes.c_void_p
    rc = L.gdn_chunk_fwd(ctypes.byref(p), None, P(16), P(16), P(16), P(16), None, P(16),
                         None, None, None, None, None, P(1 << 20), 1 << 30, None)
    assert rc == 1
    assert fwd_rc(p, ptr=18) == 3                 # q not 16-byte aligned
    assert fwd_rc(p, o=20) == 3                   # o written with 8/16-byte stores
    assert fwd_rc(p, cache=ctypes.c_void_p(24)) == 3  # state cache moved 16 bytes a lane
    assert fwd_rc(p, wsb=16) == 4                  # workspace too small
    assert fwd_rc(p, workspace=0) == 4             # no workspace
    assert fwd_rc(p, workspace=(1 << 20) + 64) == 4  # workspace misaligned


def test_bwd_validation():
    p = prob(Hq=3)
    L = gdn.lib()
    P = ctypes.c_void_p
    rc = L.gdn_chunk_bwd(ctypes.byref(p), *([P(16)] * 16), P(1 << 20), 1 << 30, None)
    assert rc == 2
    p = prob()
    rc = L.gdn_chunk_bwd(ctypes.byref(p), P(16), P(16), P(16), P(16), P(16), None, None,
                         P(16), None, None, P(16), P(16), P(16), P(16), None, None,
                         P(1 << 20), 1 << 30, None)
    assert rc == 1  # dq missing


@pytest.mark.parametrize("slot", [10, 11, 12])  # dq, dk, dv
def test_bwd_gradient_outputs_need_16_byte_alignment(slot):
    """dq, dk and dv leave the kernels as 16-byte row pieces."""
    p = prob()
    L = gdn.lib()
    P = ctypes.c_void_p
    args = [P(16)] * 16
    args[5] = args[6] = args[8] = args[14] = args[15] = None  # A, h0, dht, dh0, cache
    args[slot - 1] = P(24)
    rc = L.gdn_chunk_bwd(ctypes.byref(p), *args, P(1 << 20), 1 << 30, None)
    assert rc == 3, gdn.last_error()
    assert "16-byte" in gdn.last_error()


def test_plan_segments_cp_modes():
    L = gdn.lib()
    p = prob(T=8192, Hv=64, Hq=32)
    assert L.gdn_plan_segments(ctypes.byref(prob(T=8192, Hv=64, Hq=32, cp_mode=0))) == 1
    assert L.gdn_plan_segments(ctypes.byref(prob(T=8192, Hv=64, Hq=32, cp_mode=16))) == 8
    auto = L.gdn_plan_segments(ctypes.byref(p))
    assert 2 <= auto <= 16
    assert L.gdn_plan_segments(ctypes.byref(prob(T=65536, Hv=8, Hq=4))) >= 16


def test_qk_l2norm_flag():
    base = ws(prob())
    assert ws(prob(qk_l2norm=1)) == base    # rows normalised as loaded: no extra room
    assert ws(prob(qk_l2norm=2)) == 0 and fwd_rc(prob(qk_l2norm=2)) == 1


def test_state_cache_size():
    L = gdn.lib()
    p = prob(T=8192, Hv=64, Hq=32)
    # states, then T at a 256-byte boundary
    assert L.gdn_state_cache_size(ctypes.byref(p)) == 128 * 64 * (128 * 128 + 64 * 64) * 2
    assert L.gdn_state_cache_size(ctypes.byref(prob(T=100))) == 2 * 4 * (128 * 128 + 64 * 64) * 2
    assert L.gdn_state_cache_size(ctypes.byref(prob(Hq=3))) == 0
    # with qk_l2norm: then the normalised q, k rows ([tokens][Hq][K], bf16)
    # and their fp32 factors ([tokens][Hq]), each at a 256-byte boundary
    base = 128 * 64 * (128 * 128 + 64 * 64) * 2
    rows = 8192 * 32
    al = lambda x: (x + 255) // 256 * 256
    want = al(al(al(base) + rows * 128 * 2) + rows * 128 * 2)
    want = al(want + rows * 4) + rows * 4
    assert L.gdn_state_cache_size(ctypes.byref(prob(T=8192, Hv=64, Hq=32, qk_l2norm=1))) == want


def test_empty_problem_is_valid():
    p = prob(T=0)
    assert ws(p) > 0


def test_noalloc_rejects_oversized_problems_before_any_device_call():
    """The fixed-scratch forward checks the problem's workspace against its
    array's size on the host, before it looks the array up on a device."""
    L = gdn.lib()
    L.gdn_chunk_fwd_noalloc_max_bytes.restype = ctypes.c_size_t
    cap = L.gdn_chunk_fwd_noalloc_max_bytes()
    assert cap == 128 << 20
    big = prob(T=1 << 20, Hq=8, Hv=16)
    assert ws(big) > cap
    assert ws(prob(T=8192, Hq=32, Hv=64)) <= cap  # the headline forward fits
    P = ctypes.c_void_p
    rc = L.gdn_chunk_fwd_noalloc(ctypes.byref(big), *([P(256)] * 6), P(256), None, None, None,
                                 None, None, None)
    assert rc == 4 and "scratch" in gdn.last_error()
    rc = L.gdn_chunk_fwd_noalloc(ctypes.byref(prob(Hq=3)), *([P(256)] * 6), P(256), None, None,
                                 None, None, None, None)
    assert rc == 2

"""MI355X (gfx950) gated delta rule chunked prefill: Python binding.

Thin ctypes layer over ``libgdn.so`` (include/gdn.h).  It only marshals
arguments: torch supplies device memory (outputs and workspace) and the
current HIP stream; every step of the computation runs in the library's HIP
kernels.  There is no CPU or PyTorch fallback: if the library is missing the
import of the entry points raises.

API (mirrors the FlashQLA article's "高级 API 示例" and "底层 API" sections):

  chunk_gated_delta_rule(q, k, v, g, beta, scale, initial_state,
                         output_final_state, cu_seqlens) -> (o, final_state)
  chunk_gated_delta_rule_fwd(q, k, v, g, beta, scale, initial_state,
                             cu_seqlens) -> (g, A, o, h, final_state)
  chunk_gated_delta_rule_bwd(q, k, v, g, beta, A, do, dht, scale,
                             initial_state, cu_seqlens)
      -> (dq, dk, dv, db, dg, dh0)

Shapes: q, k [B, T, Hq, K]; v [B, T, Hv, V]; g, beta [B, T, Hv];
initial/final state [N, Hv, K, V] fp32.  q, k, v, beta share one dtype
(bfloat16 or float32); g and states are float32.  v-head h reads q/k head
h // (Hv // Hq).  With cu_seqlens (int32 [N+1]) B must be 1.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_F32, GDN_BF16 = 0, 1
CHUNK = 64


class GdnProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("Hq", ctypes.c_int32),
                ("Hv", ctypes.c_int32), ("K", ctypes.c_int32), ("V", ctypes.c_int32),
                ("N", ctypes.c_int32), ("dtype", ctypes.c_int32), ("scale", ctypes.c_float),
                ("cu_seqlens", ctypes.c_void_p), ("cu_seqlens_host", ctypes.c_void_p),
                ("cp_mode", ctypes.c_int32), ("qk_l2norm", ctypes.c_int32)]


class GdnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"gdn error {code}: {msg}")
        self.code = code


_lib = None


def lib():
    """Load libgdn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} not found: build it with "
                "`python -m gated_deltanet_chunked_gdn_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        P, S = ctypes.c_void_p, ctypes.c_size_t
        pp = ctypes.POINTER(GdnProblem)
        L.gdn_chunk_fwd_workspace_size.argtypes = [pp]
        L.gdn_chunk_fwd_workspace_size.restype = S
        L.gdn_chunk_bwd_workspace_size.argtypes = [pp]
        L.gdn_chunk_bwd_workspace_size.restype = S
        L.gdn_plan_segments.argtypes = [pp]
        L.gdn_plan_segments.restype = ctypes.c_int64
        L.gdn_state_cache_size.argtypes = [pp]
        L.gdn_state_cache_size.restype = S
        L.gdn_chunk_fwd.argtypes = [pp] + [P] * 12 + [P, S, P]
        L.gdn_chunk_fwd.restype = ctypes.c_int
        L.gdn_chunk_bwd.argtypes = [pp] + [P] * 16 + [P, S, P]
        L.gdn_chunk_bwd.restype = ctypes.c_int
        L.gdn_timing_enable.argtypes = [ctypes.c_int]
        L.gdn_timing_enable.restype = ctypes.c_int
        L.gdn_timing_collect.argtypes = [ctypes.c_int, P, P, P]
        L.gdn_timing_collect.restype = ctypes.c_int
        L.gdn_last_error.restype = ctypes.c_char_p
        L.gdn_selftest.restype = ctypes.c_int
        _lib = L
    return _lib


def last_error() -> str:
    return lib().gdn_last_error().decode()


def _check(rc: int):
    if rc != 0:
        raise GdnError(rc, last_error())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def timing_enable(on: bool) -> bool:
    """Turn per-kernel HIP-event timing on/off for this thread (see gdn.h)."""
    return bool(lib().gdn_timing_enable(1 if on else 0))


def timing_collect(max_kernels: int = 64):
    """Wait for the recorded kernel events; returns {name: (launches, total_ms)}."""
    names = ctypes.create_string_buffer(32 * max_kernels)
    counts = (ctypes.c_int32 * max_kernels)()
    ms = (ctypes.c_double * max_kernels)()
    n = lib().gdn_timing_collect(max_kernels, names, counts, ms)
    if n < 0:
        raise GdnError(-n, last_error())
    out = {}
    for i in range(n):
        nm = names.raw[32 * i:32 * (i + 1)].split(b"\0", 1)[0].decode()
        out[nm] = (int(counts[i]), float(ms[i]))
    return out


def selftest() -> None:
    """MFMA lane-layout check on the current device (raises on mismatch)."""
    _check(lib().gdn_selftest())


class _Prepared:
    """Problem descriptor plus the tensors that must outlive the launch."""

    def __init__(self, q, v, scale, cu_seqlens, cp_mode, qk_l2norm=False):
        B, T, Hq, K = q.shape
        Hv, V = v.shape[2], v.shape[3]
        if q.dtype == torch.bfloat16:
            dt = GDN_BF16
        elif q.dtype == torch.float32:
            dt = GDN_F32
        else:
            raise TypeError(f"q/k/v/beta must be bfloat16 or float32, got {q.dtype}")
        self.cu_dev = self.cu_host = None
        if cu_seqlens is not None:
            cu = cu_seqlens
            self.cu_host = cu.detach().to("cpu", torch.int32).contiguous()
            self.cu_dev = cu.detach().to(q.device, torch.int32).contiguous()
            N = self.cu_host.numel() - 1
        else:
            N = B
        self.N = N
        self.prob = GdnProblem(B, T, Hq, Hv, K, V, N, dt,
                               float(K ** -0.5 if scale is None else scale),
                               None if self.cu_dev is None else self.cu_dev.data_ptr(),
                               None if self.cu_host is None else self.cu_host.data_ptr(),
                               int(cp_mode), int(bool(qk_l2norm)))

    def ref(self):
        return ctypes.byref(self.prob)


def _contig(x):
    return None if x is None else x.contiguous()


def plan_segments(q, k, v, cu_seqlens=None, cp_mode: int = -1) -> int:
    """Number of context-parallel segments the forward launches for this
    problem (host-side planning; q, k, v give the shapes only)."""
    pr = _Prepared(q, v, None, cu_seqlens, cp_mode)
    n = lib().gdn_plan_segments(pr.ref())
    if n <= 0:
        raise ValueError(last_error())
    return int(n)


def state_cache_empty(q, v, cu_seqlens=None, cp_mode: int = -1,
                      use_qk_l2norm_in_kernel: bool = False):
    """An uninitialised state cache for this problem (an opaque uint8 buffer):
    chunk_gated_delta_rule_fwd fills it with the state entering every chunk
    and every chunk's T, and chunk_gated_delta_rule_bwd then takes those
    instead of recomputing them (memory for compute: 40 KB per chunk and
    v-head at K = V = 128 in bf16).  For calls with use_qk_l2norm_in_kernel
    it also holds the normalised q, k rows and their factors, so pass the
    same flag here."""
    pr = _Prepared(q, v, None, cu_seqlens, cp_mode, use_qk_l2norm_in_kernel)
    n = lib().gdn_state_cache_size(pr.ref())
    if n == 0:
        raise ValueError(last_error())
    return torch.empty(n, device=q.device, dtype=torch.uint8)


def _check_cache(cache, pr, q):
    if cache is None:
        return None
    n = lib().gdn_state_cache_size(pr.ref())
    if (cache.dtype != torch.uint8 or cache.dim() != 1 or cache.numel() < n
            or not cache.is_contiguous() or cache.device != q.device):
        raise ValueError("state_cache must come from state_cache_empty for this problem")
    return cache


def _check_inputs(q, k, v, g, beta):
    """Shapes and dtypes of the forward inputs (the device is checked last,
    by _check_device, after every other argument)."""
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:2] != q.shape[:2]:
        raise ValueError("q, k must be [B,T,Hq,K] and v [B,T,Hv,V]")
    if g.shape != v.shape[:3] or beta.shape != v.shape[:3]:
        raise ValueError("g and beta must be [B,T,Hv]")
    if k.dtype != q.dtype or v.dtype != q.dtype or beta.dtype != q.dtype:
        raise TypeError("q, k, v and beta must share one dtype")
    if g.dtype != torch.float32:
        raise TypeError("g must be float32")


def _check_state(x, name, shape):
    """An optional fp32 state-shaped tensor ([N, Hv, K, V])."""
    if x is not None and (x.dtype != torch.float32 or tuple(x.shape) != tuple(shape)):
        raise ValueError(f"{name} must be float32 {list(shape)}, got "
                         f"{x.dtype} {list(x.shape)}")


def _check_device(q, *others):
    """Every tensor on the GPU that holds q (a kernel reads each of them)."""
    if not q.is_cuda:
        raise ValueError("inputs must be on the GPU")
    for x in others:
        if x is not None and x.device != q.device:
            raise ValueError(f"every tensor must be on {q.device}, got one on {x.device}")


def chunk_gated_delta_rule_fwd(q, k, v, g, beta, scale=None, initial_state=None,
                               cu_seqlens=None, output_final_state=True,
                               return_intermediates=True, cp_mode: int = -1,
                               return_states: bool = True,
                               use_qk_l2norm_in_kernel: bool = False,
                               state_cache=None):
    """Forward.  Returns (g_cum, A, o, h, final_state).

    g_cum is the gate cumsum inside each 64-token chunk [B,T,Hv]; A the
    per-chunk inverse T = (I + strict_lower(diag(beta) K K^T * decay))^-1,
    [B,T,Hv,64]; h the state entering every chunk [NC,Hv,K,V].  With
    return_intermediates=False those three are None (inference mode);
    return_states=False drops only h (the backward does not take it).
    use_qk_l2norm_in_kernel L2-normalises every q and k row in the library
    (x * (sum x^2 + 1e-6)^-1/2) before use.  state_cache (from
    state_cache_empty) is filled with the per-chunk states for the backward.
    """
    _check_inputs(q, k, v, g, beta)
    q, k, v, g, beta = (_contig(x) for x in (q, k, v, g, beta))
    pr = _Prepared(q, v, scale, cu_seqlens, cp_mode, use_qk_l2norm_in_kernel)
    B, T, Hq, K = q.shape
    Hv, V = v.shape[2], v.shape[3]
    dev = q.device
    h0 = _contig(initial_state)
    _check_state(h0, "initial_state", (pr.N, Hv, K, V))
    _check_device(q, k, v, g, beta, h0, state_cache)
    o = torch.empty_like(v)
    ht = torch.empty(pr.N, Hv, K, V, device=dev, dtype=torch.float32) if output_final_state else None
    g_cum = A = h = None
    if return_intermediates:
        if pr.cu_host is not None:
            lens = (pr.cu_host[1:] - pr.cu_host[:-1]).tolist()
            nc = sum((L + CHUNK - 1) // CHUNK for L in lens)
        else:
            nc = B * ((T + CHUNK - 1) // CHUNK)
        g_cum = torch.empty_like(g)
        A = torch.empty(B, T, Hv, CHUNK, device=dev, dtype=torch.float32)
        if return_states:
            h = torch.empty(nc, Hv, K, V, device=dev, dtype=torch.float32)
    L = lib()
    ws_bytes = L.gdn_chunk_fwd_workspace_size(pr.ref())
    if ws_bytes == 0:
        raise GdnError(1, last_error())
    ws = torch.empty(ws_bytes, device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream(dev).cuda_stream
    cache = _check_cache(state_cache, pr, q)
    _check(L.gdn_chunk_fwd(pr.ref(), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0),
                           _ptr(o), _ptr(ht), _ptr(g_cum), _ptr(A), _ptr(h), _ptr(cache),
                           _ptr(ws), ws_bytes, ctypes.c_void_p(stream)))
    return g_cum, A, o, h, ht


def chunk_gated_delta_rule(q, k, v, g, beta, scale=None, initial_state=None,
                           output_final_state=False, cu_seqlens=None, cp_mode: int = -1,
                           use_qk_l2norm_in_kernel: bool = False):
    """Inference forward: returns (o, final_state or None)."""
    _, _, o, _, ht = chunk_gated_delta_rule_fwd(
        q, k, v, g, beta, scale=scale, initial_state=initial_state, cu_seqlens=cu_seqlens,
        output_final_state=output_final_state, return_intermediates=False, cp_mode=cp_mode,
        use_qk_l2norm_in_kernel=use_qk_l2norm_in_kernel)
    return o, ht


def chunk_gated_delta_rule_bwd(q, k, v, g, beta, A, do, dht=None, scale=None,
                               initial_state=None, cu_seqlens=None, cp_mode: int = -1,
                               use_qk_l2norm_in_kernel: bool = False, state_cache=None):
    """Backward.  Returns (dq, dk, dv, db, dg, dh0); dg is w.r.t. the raw g.

    A is the forward's A output (or None to recompute it).  With
    use_qk_l2norm_in_kernel (as in the forward) dq, dk are with respect to
    the raw q, k.  state_cache: the cache the forward of the same inputs
    filled (the per-chunk states and T are then taken from it and A is not
    read), or None."""
    _check_inputs(q, k, v, g, beta)
    if do is None or do.shape != v.shape or do.dtype != v.dtype:
        raise ValueError(f"do must have v's shape {list(v.shape)} and dtype {v.dtype}")
    q, k, v, g, beta, do = (_contig(x) for x in (q, k, v, g, beta, do))
    A, dht, h0 = _contig(A), _contig(dht), _contig(initial_state)
    pr = _Prepared(q, v, scale, cu_seqlens, cp_mode, use_qk_l2norm_in_kernel)
    B, T, Hq, K = q.shape
    Hv, V = v.shape[2], v.shape[3]
    if A is not None and (A.dtype != torch.float32 or tuple(A.shape) != (B, T, Hv, CHUNK)):
        raise ValueError(f"A must be float32 [{B},{T},{Hv},{CHUNK}] (the forward's A), got "
                         f"{A.dtype} {list(A.shape)}")
    _check_state(dht, "dht", (pr.N, Hv, K, V))
    _check_state(h0, "initial_state", (pr.N, Hv, K, V))
    _check_device(q, k, v, g, beta, do, A, dht, h0, state_cache)
    dev = q.device
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    db = torch.empty_like(beta)
    dg = torch.empty_like(g)
    dh0 = torch.empty(pr.N, v.shape[2], q.shape[3], v.shape[3], device=dev,
                      dtype=torch.float32)
    L = lib()
    ws_bytes = L.gdn_chunk_bwd_workspace_size(pr.ref())
    if ws_bytes == 0:
        raise GdnError(1, last_error())
    ws = torch.empty(ws_bytes, device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream(dev).cuda_stream
    _check(L.gdn_chunk_bwd(pr.ref(), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(A),
                           _ptr(h0), _ptr(do), _ptr(dht), _ptr(dq), _ptr(dk), _ptr(dv),
                           _ptr(db), _ptr(dg), _ptr(dh0), _ptr(_check_cache(state_cache, pr, q)),
                           _ptr(ws), ws_bytes, ctypes.c_void_p(stream)))
    return dq, dk, dv, db, dg, dh0

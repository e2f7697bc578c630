"""ctypes front end of the fp64 token-recurrence oracle (``gdn_oracle.c``).

TEST INFRASTRUCTURE ONLY: the correctness reference for the HIP library.  Only
tests, the smoke check and the benchmark's CPU-baseline leg may import it.

The recurrence is the gated delta rule the FlashQLA article's API sections
("高级 API 示例", "底层 API") expose as ``chunk_gated_delta_rule`` /
``chunk_gated_delta_rule_fwd`` / ``chunk_gated_delta_rule_bwd``:
``S_t = exp(g_t)(I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T`` and
``o_t = scale * S_t^T q_t``; the backward is its reverse mode.  All arithmetic
is float64 on whatever (already rounded) values the caller passes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import l2norm

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile the C oracle with gcc (plain -O3, OpenMP, no fp contraction)."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        subprocess.check_call([
            "gcc", "-O3", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
            "-std=c99", src, "-o", tmp, "-lm"])
        os.replace(tmp, out)
    return out


class Oracle:
    """The C oracle loaded from one shared-library path."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.gdn_oracle_fwd.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P,
                                       ctypes.c_double, P, P, P, P, I]
        lib.gdn_oracle_fwd.restype = I
        lib.gdn_oracle_bwd.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P,
                                       ctypes.c_double, P, P, P, P, P, P, P, P,
                                       P, P, I]
        lib.gdn_oracle_bwd.restype = I
        lib.gdn_oracle_max_threads.restype = I
        self.lib = lib

    def fwd(self, *a, **kw):
        return fwd(*a, _lib=self.lib, **kw)

    def bwd(self, *a, **kw):
        return bwd(*a, _lib=self.lib, **kw)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = Oracle(_LIB).lib
    return _lib


def max_threads() -> int:
    return _load().gdn_oracle_max_threads()


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dims(q, v, cu_seqlens):
    B, T, Hq, K = q.shape
    Hv, V = v.shape[2], v.shape[3]
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        N = cu.shape[0] - 1
    else:
        cu = None
        N = B
    return B, T, Hq, Hv, K, V, N, cu


def _mask(unit_mask, N, Hv):
    if unit_mask is None:
        return None
    m = np.ascontiguousarray(np.asarray(unit_mask, dtype=np.uint8).reshape(N * Hv))
    return m


def fwd(q, k, v, g, beta, scale=None, initial_state=None, cu_seqlens=None,
        unit_mask=None, threads: int = 0, qk_l2norm: bool = False, _lib=None):
    """Forward: returns (o [B,T,Hv,V], final_state [N,Hv,K,V]) in float64.

    ``unit_mask`` ([N, Hv] bools) restricts the work to selected
    (sequence, v-head) units; other entries of the outputs are zero.
    ``qk_l2norm`` first L2-normalises every q and k row (``oracle.l2norm``).
    """
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    if qk_l2norm:
        q, k = l2norm.fwd(q), l2norm.fwd(k)
    h0 = _f64(initial_state)
    B, T, Hq, Hv, K, V, N, cu = _dims(q, v, cu_seqlens)
    if scale is None:
        scale = K ** -0.5
    o = np.zeros((B, T, Hv, V))
    ht = np.zeros((N, Hv, K, V))
    m = _mask(unit_mask, N, Hv)
    rc = (_lib or _load()).gdn_oracle_fwd(B, T, Hq, Hv, K, V, N, _ptr(cu), _ptr(q), _ptr(k),
                                _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(h0),
                                _ptr(o), _ptr(ht), _ptr(m), int(threads))
    if rc != 0:
        raise ValueError(f"oracle fwd rejected the problem (code {rc})")
    return o, ht


def bwd(q, k, v, g, beta, do, dht=None, scale=None, initial_state=None,
        cu_seqlens=None, unit_mask=None, threads: int = 0, qk_l2norm: bool = False,
        _lib=None):
    """Backward: returns (dq, dk, dv, dbeta, dg, dh0) in float64.

    dg is the gradient with respect to the raw log-gate g; dq/dk are summed
    over the v-heads of each q/k group.  With ``qk_l2norm`` the recurrence
    runs on the normalised rows and dq/dk are taken back through the
    normalisation (with respect to the raw q, k).
    """
    q, k, v, g, beta, do = (_f64(x) for x in (q, k, v, g, beta, do))
    q_raw, k_raw = q, k
    if qk_l2norm:
        q, k = l2norm.fwd(q), l2norm.fwd(k)
    h0 = _f64(initial_state)
    dht = _f64(dht)
    B, T, Hq, Hv, K, V, N, cu = _dims(q, v, cu_seqlens)
    if scale is None:
        scale = K ** -0.5
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    db = np.zeros_like(beta)
    dg = np.zeros_like(g)
    dh0 = np.zeros((N, Hv, K, V))
    m = _mask(unit_mask, N, Hv)
    rc = (_lib or _load()).gdn_oracle_bwd(B, T, Hq, Hv, K, V, N, _ptr(cu), _ptr(q), _ptr(k),
                                _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(h0),
                                _ptr(do), _ptr(dht), _ptr(dq), _ptr(dk), _ptr(dv),
                                _ptr(db), _ptr(dg), _ptr(dh0), _ptr(m), int(threads))
    if rc != 0:
        raise ValueError(f"oracle bwd rejected the problem (code {rc})")
    if qk_l2norm:
        dq, dk = l2norm.bwd(q_raw, dq), l2norm.bwd(k_raw, dk)
    return dq, dk, dv, db, dg, dh0

"""Helpers shared by the GPU parity tests (no tests here)."""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import token

TOL = {"bf16": 1e-2, "f32": 1e-5}


def rel(x, ref) -> float:
    """Relative Frobenius error ||x - ref|| / ||ref|| (absolute if ref == 0)."""
    if isinstance(x, torch.Tensor):
        x = x.detach().double().cpu().numpy()
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    nr = np.linalg.norm(ref)
    d = np.linalg.norm(x - ref)
    return float(d / nr) if nr > 0 else float(d)


def announce(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(p, dev="cuda:0"):
    out = {}
    for k_, v_ in p.items():
        out[k_] = v_.to(dev) if isinstance(v_, torch.Tensor) else v_
    return out


def oracle_fwd(p, unit_mask=None):
    cu = None if p["cu_seqlens"] is None else p["cu_seqlens"].numpy()
    return token.fwd(p["q"], p["k"], p["v"], p["g"], p["beta"], scale=p["scale"],
                     initial_state=p["initial_state"], cu_seqlens=cu, unit_mask=unit_mask)


def oracle_bwd(p, unit_mask=None):
    cu = None if p["cu_seqlens"] is None else p["cu_seqlens"].numpy()
    return token.bwd(p["q"], p["k"], p["v"], p["g"], p["beta"], p["do"], p["dht"],
                     scale=p["scale"], initial_state=p["initial_state"], cu_seqlens=cu,
                     unit_mask=unit_mask)


def token_mask(p, unit_mask):
    """[B, T, Hv] bool: tokens that belong to selected (sequence, v-head) units."""
    B, T, Hv = p["g"].shape
    m = np.zeros((B, T, Hv), dtype=bool)
    if p["cu_seqlens"] is None:
        for b in range(B):
            m[b, :, :] = unit_mask[b][None, :]
    else:
        cu = p["cu_seqlens"].numpy()
        for n in range(len(cu) - 1):
            m[0, cu[n]:cu[n + 1], :] = unit_mask[n][None, :]
    return m

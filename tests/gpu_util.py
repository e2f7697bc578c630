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


# Bound on the relative error of any one 64-token block of one head (the
# whole-tensor bound is TOL).  A block's error averages 64 rows only, so a
# fault confined to one row of a block (about 1/8 of the block's norm) or to
# part of a chunk cannot hide in it the way it hides in a whole-tensor norm
# over 10^5 rows.  The margin over TOL covers the spread of honest bf16
# rounding between blocks; dbeta and dg are sums with cancellation and get a
# wider one.
BLOCK_TOL = {"bf16": 2.5e-2, "f32": 1e-4}
BLOCK_TOL_CANCEL = {"bf16": 6e-2, "f32": 1e-4}


def block_rel_max(x, ref, sel=None, block=64):
    """Largest relative Frobenius error over blocks of `block` consecutive
    selected tokens of one head.

    x, ref: [B, T, H] or [B, T, H, D]; sel: [B, T, H] bool (the tokens of the
    selected units) or None (all).  Blocks whose reference norm is 0 use the
    absolute error."""
    if isinstance(x, torch.Tensor):
        x = x.detach().double().cpu().numpy()
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if x.ndim == 3:
        x, ref = x[..., None], ref[..., None]
    B, T, H = x.shape[:3]
    worst = 0.0
    for b in range(B):
        for h in range(H):
            rows = slice(None) if sel is None else sel[b, :, h]
            xs, rs = x[b, rows, h], ref[b, rows, h]
            n = xs.shape[0]
            if n == 0:
                continue
            nb = (n + block - 1) // block
            pad = nb * block - n
            xs = np.concatenate([xs, np.zeros((pad,) + xs.shape[1:])]).reshape(nb, -1)
            rs = np.concatenate([rs, np.zeros((pad,) + rs.shape[1:])]).reshape(nb, -1)
            d = np.linalg.norm(xs - rs, axis=1)
            nr = np.linalg.norm(rs, axis=1)
            e = np.where(nr > 0, d / np.where(nr > 0, nr, 1.0), d)
            worst = max(worst, float(e.max()))
    return worst


def announce(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(p, dev="cuda:0"):
    out = {}
    for k_, v_ in p.items():
        out[k_] = v_.to(dev) if isinstance(v_, torch.Tensor) else v_
    return out


def oracle_fwd(p, unit_mask=None, qk_l2norm=False):
    cu = None if p["cu_seqlens"] is None else p["cu_seqlens"].numpy()
    return token.fwd(p["q"], p["k"], p["v"], p["g"], p["beta"], scale=p["scale"],
                     initial_state=p["initial_state"], cu_seqlens=cu, unit_mask=unit_mask,
                     qk_l2norm=qk_l2norm)


def oracle_bwd(p, unit_mask=None, qk_l2norm=False):
    cu = None if p["cu_seqlens"] is None else p["cu_seqlens"].numpy()
    return token.bwd(p["q"], p["k"], p["v"], p["g"], p["beta"], p["do"], p["dht"],
                     scale=p["scale"], initial_state=p["initial_state"], cu_seqlens=cu,
                     unit_mask=unit_mask, qk_l2norm=qk_l2norm)


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

"""Seeded synthetic inputs for the GDN chunked prefill (forward and backward).

Shared by the tests, the smoke check and the benchmark; holds none of the
operator's arithmetic (only the input recipe).  The pages benchmark an
undisclosed-length head-count sweep (FlashQLA article, "性能基准测试": head
counts {64, 48, 32, 24, 16, 8}, i.e. TP1..TP8 of one model family) and publish
no dataset; these inputs stand in for it.

Recipe (one generator per workload, ``numpy.random.default_rng(seed)``; all
draws float32 standard normal, in this order):
  1. (varlen only) sequence lengths ~ U{lo..hi} -> cu_seqlens, B = 1
  2. q, then k, each L2-normalised over the key dimension in float32
  3. v
  4. g = -softplus(x)   (log-gate, kept float32)
  5. beta = sigmoid(x)
  6. initial state = 0.1 x  (float32; only when requested)
  7. do = x, then dht = 0.1 x (only when requested)
then q, k, v, beta, do are cast to the working dtype (bf16 rounding is
round-to-nearest-even, done by torch).  scale = K^-0.5.

Gate variants (same seed): "slow" divides g by 100, "moderate" by 10, "nodecay" sets g = 0.
These expose the carried state, which the default gates (about e^-52 per
64-token chunk) make numerically invisible after a chunk or two.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

SEED_BASE = 20260000


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    T: int
    Hq: int
    Hv: int
    K: int
    V: int
    dtype: str  # "f32" | "bf16"
    varlen: Optional[tuple] = None  # (n_seqs, lo, hi)
    h0: bool = False
    backward: bool = False
    seed: int = SEED_BASE


# The five workloads the operator is exercised on (sizes as named).
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 256, 2, 2, 32, 32, "f32", seed=SEED_BASE + 0),
    "hv64_t8192": Workload("hv64_t8192", 1, 8192, 32, 64, 128, 128, "bf16",
                           seed=SEED_BASE + 1),
    "hv8_t65536": Workload("hv8_t65536", 1, 65536, 4, 8, 128, 128, "bf16",
                           seed=SEED_BASE + 2),
    "varlen16_hv32": Workload("varlen16_hv32", 1, 0, 16, 32, 128, 128, "bf16",
                              varlen=(16, 256, 16384), h0=True, seed=SEED_BASE + 3),
    "bwd_b2_t16384_hv16": Workload("bwd_b2_t16384_hv16", 2, 16384, 8, 16, 128, 128,
                                   "bf16", backward=True, seed=SEED_BASE + 4),
}


# Head-count sweep of the pages' benchmark (FlashQLA article, "性能基准测试":
# head counts 64, 48, 32, 24, 16, 8 for TP1..TP8), at the headline length and
# the headline's q/k grouping (H_q = H_v / 2).
SWEEP_HV = (64, 48, 32, 24, 16, 8)


def sweep_workload(hv: int, T: int = 8192) -> Workload:
    return Workload(f"sweep_hv{hv}_t{T}", 1, T, hv // 2, hv, 128, 128, "bf16",
                    backward=True, seed=SEED_BASE + 100 + hv)


def _softplus(x):
    return np.logaddexp(0.0, x).astype(np.float32)


def _l2n(x):
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / np.maximum(n, np.float32(1e-6))).astype(np.float32)


def torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def make(w: Workload, gate: str = "default", T: Optional[int] = None,
         lengths=None, with_h0: Optional[bool] = None,
         with_grads: Optional[bool] = None, normalize_qk: bool = True):
    """Build one problem as a dict of CPU torch tensors.

    ``T`` overrides the sequence length (reduced-size variants); ``lengths``
    overrides the varlen draw; ``with_h0``/``with_grads`` override the
    workload's flags; ``normalize_qk=False`` keeps q, k as raw N(0, 1) draws
    (inputs for the in-library L2 normalisation).  Keys: q k v g beta scale cu_seqlens initial_state
    do dht, plus ``lengths`` for varlen problems.
    """
    rng = np.random.default_rng(w.seed)
    B, Hq, Hv, K, V = w.B, w.Hq, w.Hv, w.K, w.V
    cu = None
    if w.varlen is not None or lengths is not None:
        if lengths is None:
            n, lo, hi = w.varlen
            lengths = rng.integers(lo, hi, size=n, endpoint=True)
        lengths = np.asarray(lengths, dtype=np.int64)
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
        B, Ttot = 1, int(cu[-1])
        N = len(lengths)
    else:
        Ttot = w.T if T is None else T
        N = B
    sn = lambda *shape: rng.standard_normal(shape, dtype=np.float32)
    q = sn(B, Ttot, Hq, K)
    k = sn(B, Ttot, Hq, K)
    if normalize_qk:
        q, k = _l2n(q), _l2n(k)
    v = sn(B, Ttot, Hv, V)
    g = -_softplus(sn(B, Ttot, Hv))
    beta = (1.0 / (1.0 + np.exp(-sn(B, Ttot, Hv)))).astype(np.float32)
    if gate == "slow":
        g = (g / np.float32(100.0)).astype(np.float32)
    elif gate == "moderate":
        g = (g / np.float32(10.0)).astype(np.float32)
    elif gate == "nodecay":
        g = np.zeros_like(g)
    elif gate != "default":
        raise ValueError(gate)
    want_h0 = w.h0 if with_h0 is None else with_h0
    h0 = (np.float32(0.1) * sn(N, Hv, K, V)) if want_h0 else None
    want_g = w.backward if with_grads is None else with_grads
    do = dht = None
    if want_g:
        do = sn(B, Ttot, Hv, V)
        dht = np.float32(0.1) * sn(N, Hv, K, V)
    dt = torch_dtype(w.dtype)
    out = dict(
        q=torch.from_numpy(q).to(dt), k=torch.from_numpy(k).to(dt),
        v=torch.from_numpy(v).to(dt), g=torch.from_numpy(g),
        beta=torch.from_numpy(beta).to(dt), scale=float(K) ** -0.5,
        cu_seqlens=None if cu is None else torch.from_numpy(cu.astype(np.int32)),
        initial_state=None if h0 is None else torch.from_numpy(h0),
        do=None if do is None else torch.from_numpy(do).to(dt),
        dht=None if dht is None else torch.from_numpy(dht),
    )
    if cu is not None:
        out["lengths"] = [int(x) for x in lengths]
    return out


def custom(B, T, Hq, Hv, K, V, dtype="bf16", seed=1, gate="default",
           lengths=None, h0=False, grads=False, normalize_qk=True):
    """Arbitrary-shape problem with the same recipe (for edge-case tests)."""
    w = Workload("custom", B, T, Hq, Hv, K, V, dtype, h0=h0, backward=grads, seed=seed)
    return make(w, gate=gate, lengths=lengths, normalize_qk=normalize_qk)

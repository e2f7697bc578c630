"""Per-row L2 normalisation of q and k, forward and reverse mode, in float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages state no in-kernel normalisation (their inputs are whatever the
caller passes).  The plainest reading of an in-kernel "q/k L2 normalisation"
is taken here and in the library alike: for every token and q/k head, over
the key dimension,

    x_hat = x * r,   r = (sum_i x_i^2 + eps)^(-1/2),   eps = 1e-6.

Reverse mode (d x_hat given): with the Jacobian r (I - x_hat x_hat^T),

    dx = r * (d x_hat - x_hat * <x_hat, d x_hat>).
"""
from __future__ import annotations

import numpy as np

EPS = 1e-6


def _r(x, eps):
    return 1.0 / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def fwd(x, eps: float = EPS):
    """x_hat for rows along the last axis."""
    x = np.asarray(x, dtype=np.float64)
    return x * _r(x, eps)


def bwd(x, dxhat, eps: float = EPS):
    """Gradient with respect to x given the gradient with respect to x_hat."""
    x = np.asarray(x, dtype=np.float64)
    dxhat = np.asarray(dxhat, dtype=np.float64)
    r = _r(x, eps)
    xh = x * r
    return r * (dxhat - xh * np.sum(xh * dxhat, axis=-1, keepdims=True))

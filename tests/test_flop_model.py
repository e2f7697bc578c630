"""The FLOP model behind bench.py's TFLOP/s and %-of-peak figures.

bench.chunk_flops states the dense products of the chunked algorithm per
full 64-token chunk and v-head.  These tests count, with an ndarray subclass
that tallies every matrix product (2 m k n each), the products the oracle's
chunked form (oracle/chunked.py) actually performs on one full chunk, and
require the model to equal that count (the triangular inverse, done there
by a library routine, is the model's n^3/3 convention and is added
separately).
"""
import numpy as np
import pytest

import bench
from oracle import chunked

N = 64


class Counted(np.ndarray):
    flops = 0

    def __matmul__(self, other):
        a, b = np.asarray(self), np.asarray(other)
        Counted.flops += 2 * a.shape[0] * a.shape[-1] * b.shape[-1]
        return np.matmul(a, b).view(Counted)

    def __rmatmul__(self, other):
        return Counted.__matmul__(np.asarray(other).view(Counted), self)


def _inputs(K, V, seed):
    rng = np.random.default_rng(seed)
    arr = lambda *s: rng.standard_normal(s).view(Counted)  # noqa: E731
    q, k, v = arr(N, K), arr(N, K), arr(N, V)
    g = (-0.1 * np.abs(rng.standard_normal(N))).view(Counted)
    beta = rng.random(N).view(Counted)
    return q, k, v, g, beta, arr(K, V), arr(N, V), arr(K, V)


def _count(fn, *args):
    Counted.flops = 0
    fn(*args)
    return Counted.flops


@pytest.mark.parametrize("K,V", [(32, 16), (64, 64), (128, 128)])
def test_forward_model_equals_the_chunked_forms_products(K, V):
    q, k, v, g, beta, S0, _, _ = _inputs(K, V, 1)
    counted = _count(chunked.chunk_forward_one, q, k, v, g, beta, 0.5, S0, N)
    fwd, _ = bench.chunk_flops(K, V)
    assert counted + N ** 3 / 3 == fwd


@pytest.mark.parametrize("K,V", [(32, 16), (64, 64), (128, 128)])
def test_backward_model_equals_the_chunked_forms_products(K, V):
    q, k, v, g, beta, S0, do, dST = _inputs(K, V, 2)
    # the oracle's backward first replays the forward to keep each chunk's
    # entering state: that replay is not part of the backward's count
    replay = _count(chunked.chunk_forward_one, q, k, v, g, beta, 0.5, S0, N)
    total = _count(chunked.chunk_backward_one, q, k, v, g, beta, 0.5, S0, do, dST, N)
    _, bwd = bench.chunk_flops(K, V)
    assert total - replay + N ** 3 / 3 == bwd


def test_kernel_split_of_the_forward_and_min_bytes():
    """The per-kernel FLOPs of the forward's two kernels add up to the
    forward's chunked-algorithm count, and the minimum bytes of the headline
    forward are the inputs read once plus o and the final state (410 MB)."""
    import synth
    w = synth.WORKLOADS["hv64_t8192"]
    nch = 128
    fwd, _ = bench.chunk_flops(w.K, w.V)
    split = bench.kernel_flops("prep", w, nch) + bench.kernel_flops("fwd_main", w, nch)
    assert abs(split - fwd * nch * w.Hv) < 1e-6 * split
    assert bench.kernel_flops("fwd_fix", w, nch) is None
    mb = bench.min_bytes(w, 8192, 1, "fwd", 2)
    assert abs(mb - 409.8e6) < 0.5e6
    # the backward adds do and dht to the reads, every gradient to the writes
    # and, in the pages' dataflow, the saved A (fp32, 64 per token and v-head)
    with_a = bench.min_bytes(w, 8192, 1, "bwd", 2, with_A=True)
    assert with_a - bench.min_bytes(w, 8192, 1, "bwd", 2) == 8192 * 64 * 64 * 4

"""The per-block error measure the full-size parity tests use finds what a
whole-tensor norm hides."""
import numpy as np

from tests.gpu_util import block_rel_max, rel


def test_one_wrong_row_is_found():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((1, 65536, 2, 128))
    x = ref * (1 + 1e-3 * rng.standard_normal(ref.shape))
    x[0, 40000, 1] = 0.0                       # one row lost
    assert rel(x, ref) < 1e-2                  # invisible in the whole tensor
    assert block_rel_max(x, ref) > 0.1         # about 1/8 of its block


def test_selection_and_clean_blocks():
    rng = np.random.default_rng(1)
    ref = rng.standard_normal((2, 300, 3))
    x = ref.copy()
    sel = np.zeros((2, 300, 3), dtype=bool)
    sel[1, :, 2] = True
    x[0, 5, 0] += 10.0                         # outside the selection
    assert block_rel_max(x, ref, sel) == 0.0
    x[1, 299, 2] += 1.0                        # last, partial block of the selection
    assert block_rel_max(x, ref, sel) > 0.0

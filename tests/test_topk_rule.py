"""The rule by which the persistent decode's top-K is compared with the
oracle's, in the GPU tests and in bench.py's parity check before timing:
equal, except that distinct logits closer than the 36-bit hand-off rounding
resolves (2^-35 relative to the largest) may swap ranks; exact ties keep the
lower-index rule and must match."""
import numpy as np
import pytest

import bench
from tests.gpu_util import topk_matches

L = np.array([1.0, 0.5, 0.5, 0.3, 0.3 + 1e-12, 0.1, 0.3 - 1e-9])

CASES = [
    ([0, 1, 2], [0, 1, 2], True),          # equal
    ([0, 2, 1], [0, 1, 2], False),         # an exact tie in the other order
    ([0, 1, 3, 4], [0, 1, 4, 3], True),    # a 1e-12 near-tie swapped
    ([0, 1, 4], [0, 1, 3], True),          # across the boundary, same near-tie
    ([0, 1, 6], [0, 1, 3], False),         # 1e-9 apart: far wider than the rounding
    ([0, 1, 5], [0, 1, 2], False),         # another expert
    ([0, 0, 1], [0, 1, 2], False),         # a duplicate
    ([0, 1, -1], [0, 1, 2], False),        # no expert
    ([0, 1, 7], [0, 1, 2], False),         # out of range
]


@pytest.mark.parametrize("rule", [topk_matches, bench.topk_matches], ids=["tests", "bench"])
@pytest.mark.parametrize("idx,ref,want", CASES)
def test_topk_rule(rule, idx, ref, want):
    assert rule(idx, ref, L) is want

"""Host-side helpers of bench.py that report on the weight quantization
(no GPU): the count of codes on which dividing by the mean and multiplying by
its reciprocal disagree (hand-worked cases and an exact-reciprocal
invariant), and the fp64 absmean."""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def _f32(bits: int) -> np.float32:
    return np.array([bits], np.uint32).view(np.float32)[0]


def test_divide_and_reciprocal_disagree_next_to_a_tie():
    """m = 0x3cbe3acc (0.023221396), W = 0x3c3e3acd, one ulp above m / 2:
    W / m rounds to 0.50000006 (code 1), W * fl(1/m) to 0.5 (code 0, half to
    even).  -W disagrees the same way; m / 2 itself and values far from the
    boundary agree."""
    m, w = _f32(0x3cbe3acc), _f32(0x3c3e3acd)
    assert w / m == np.float32(0.50000006) and w * (np.float32(1.0) / m) == np.float32(0.5)
    W = np.array([w, -w, np.float32(m * np.float32(0.5)), np.float32(0.2), np.float32(0.0)], np.float32)
    assert bench.q1_disagreement_count(W, m) == 2


def test_power_of_two_mean_never_disagrees():
    """1/m is exact for a power of two, so both readings give the same codes."""
    W = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    for m in (0.25, 1.0, 8.0):
        assert bench.q1_disagreement_count(W, np.float32(m)) == 0


def test_absmean_floor_and_value():
    assert bench.absmean_f32(np.zeros(16, np.float32)) == np.float32(1e-5)
    assert bench.absmean_f32(np.array([1, -2, 3, -6], np.float32)) == np.float32(3.0)

"""The GPU tests' check of flagged (near-tied) routing answers: the selected
set must be a valid top-K within the tolerance and the slots in descending
score order within it.  CPU only."""
import numpy as np
import pytest

tests_harness = pytest.importorskip("tests.gpu_harness")


def test_order_within_tolerance():
    score = np.array([0.5, 0.3, 0.3 - 5e-5, 0.1, 0.0])
    check = tests_harness._valid_topk
    assert check(score, [0, 1, 2], 3, ordered=True)
    assert check(score, [0, 2, 1], 3, ordered=True)  # the tied pair either way
    assert not check(score, [1, 0, 2], 3, ordered=True)  # 0.3 ahead of 0.5
    assert check(score, [1, 0, 2], 3)  # the set alone is valid
    assert not check(score, [0, 1, 3], 3, ordered=True)  # 0.1 selected over 0.3 - 5e-5

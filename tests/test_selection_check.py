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


def test_order_consistency_with_logit_intervals():
    """The unflagged tokens' slot-order check: an order is accepted when some
    scores inside the per-expert intervals are in that descending order."""
    check = tests_harness._order_consistent
    lo = np.array([1.0, 0.5, 0.5 - 1e-6, 0.1])
    hi = lo + 2e-6
    assert check(lo, hi, [0, 1, 2])
    assert check(lo, hi, [0, 2, 1])  # the pair within the intervals, either way
    assert not check(lo, hi, [1, 0, 2])  # 0.5 cannot rank above 1.0
    assert not check(lo, hi, [0, 3, 1])  # 0.1 cannot rank above 0.5
    # an interval overlapping only its neighbour: a swap two places away is not
    lo = np.array([0.3, 0.3 - 1.5e-6, 0.3 - 3e-6])
    hi = lo + 2e-6
    assert check(lo, hi, [1, 0, 2]) and check(lo, hi, [0, 2, 1])
    assert not check(lo, hi, [2, 1, 0])


def test_logit_error_bound_scales_with_the_sum_of_magnitudes():
    import dataclasses
    from synth import WORKLOADS
    spec = dataclasses.replace(WORKLOADS["qwen_decode"], n_tokens=2)
    x = np.array([[1.0] * 2048, [0.5] * 2048])
    w = np.full((3, 2048), 2.0 ** -6)
    b = tests_harness.logit_error_bound(spec, x, w)
    # d = 2048/32 + 40 = 104 roundings of 2u each, times sum |w x| = 32 and 16
    np.testing.assert_allclose(b[:, 0], 2 * 104 * 2.0 ** -24 * np.array([32.0, 16.0]))
    f32 = dataclasses.replace(WORKLOADS["tiny_f32"], n_tokens=2, d_model=64)
    np.testing.assert_allclose(tests_harness.logit_error_bound(f32, np.ones((1, 64)), np.ones((1, 64))),
                               [[2 * 64 * 2.0 ** -24 * 64]])

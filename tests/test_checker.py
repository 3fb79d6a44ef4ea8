"""The parity checker accepts what the rules allow and rejects real misses (CPU)."""
import numpy as np
import pytest

from oracle.check import check_scores, check_topk_row


def test_accepts_exact_and_padded():
    o = np.array([0.5, 0.9, 0.1, 0.7])
    check_topk_row([1, 3, -1, -1][:2] + [-1] * 0, None, o, 4, 2)
    check_topk_row([1, 0, 3, 2, -1, -1], None, o, 4, 6)


def test_accepts_near_tie_swap_rejects_real_miss():
    o = np.array([1.0, 0.50000, 0.50003, 0.2, 0.1])
    check_topk_row([0, 1], None, o, 5, 2)          # oracle picks 2, 1 is within tol of tau
    with pytest.raises(AssertionError):
        check_topk_row([0, 3], None, o, 5, 2)      # 3 is far below tau


def test_rejects_padding_duplicates_and_range():
    o = np.arange(10, dtype=float)
    with pytest.raises(AssertionError):
        check_topk_row([9, 8, 8], None, o, 10, 3)
    with pytest.raises(AssertionError):
        check_topk_row([9, 8, 10], None, o, 10, 3)
    with pytest.raises(AssertionError):
        check_topk_row([2, 1, 0, 5], None, o, 3, 4)  # slot 3 must be -1


def test_score_rule():
    check_scores(np.array([1.0005, 5e-5, -np.inf]), np.array([1.0, 0.0, -np.inf]))
    with pytest.raises(AssertionError):
        check_scores(np.array([1.002]), np.array([1.0]))
    with pytest.raises(AssertionError):
        check_scores(np.array([0.0]), np.array([-np.inf]))


def test_signed_weights_swap_uses_each_positions_tolerance():
    """With magnitude sums given, a position whose tolerance is wide (large
    M) may fall below a precisely scored one; the returned set is accepted
    iff some scores within each position's own tolerance rank it first."""
    o = np.array([1.0, 0.00424, 0.00405, 0.00318, 0.001])
    wide = np.array([1.0, 14.4, 0.004, 0.0154, 0.001])   # position 1: tol 0.0144
    check_topk_row([0, 2, 3], None, o, 5, 3, mag_row=wide)
    narrow = np.array([1.0, 0.004, 0.004, 0.0154, 0.001])  # every tol 1e-4
    with pytest.raises(AssertionError):
        check_topk_row([0, 2, 3], None, o, 5, 3, mag_row=narrow)
    # a wide tolerance elsewhere does not excuse a returned position far
    # below a precisely scored one that was left out
    with pytest.raises(AssertionError):
        check_topk_row([0, 1, 4], None, o, 5, 3, mag_row=wide)

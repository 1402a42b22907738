"""Pins of the sampling oracle to facts outside it: interval lengths against
SciPy's softmax, the zero- and high-temperature limits, the boundary
convention, shift invariance and a brute-force count over a grid of u."""
import numpy as np
import pytest
from scipy.special import softmax as scipy_softmax

from oracle import interval_of, sample_probs, sample_token


def test_probs_match_library_softmax():
    # catches a missing or inverted temperature scale
    z = np.array([0.3, -1.2, 2.0, 0.0, 0.7])
    for T in (0.25, 1.0, 3.0):
        assert np.allclose(sample_probs(z, T), scipy_softmax(z / T), rtol=1e-14, atol=0)


def test_grid_counts_equal_probabilities():
    # brute force: M evenly spaced u draw token i about M * p_i times
    # (a reversed cumulative sum or an off-by-one index fails this)
    z = np.array([1.0, -0.5, 0.25, 2.0, -3.0, 0.0, 0.5])
    T, M = 0.8, 20000
    p = scipy_softmax(z / T)
    counts = np.bincount([sample_token(z, T, (k + 0.5) / M) for k in range(M)], minlength=len(z))
    assert np.all(np.abs(counts - M * p) <= 1.0), (counts, M * p)


def test_intervals_tile_unit_range_in_index_order():
    z = np.array([0.1, 0.4, -0.2, 0.9])
    T = 0.5
    lo_prev = 0.0
    for i in range(len(z)):
        lo, hi = interval_of(z, T, i)
        assert lo == pytest.approx(lo_prev, abs=1e-15)
        assert hi - lo == pytest.approx(scipy_softmax(z / T)[i], rel=1e-12)
        # the interval's ends draw this token and its successor
        assert sample_token(z, T, lo + 1e-12) == i
        lo_prev = hi
    assert lo_prev == pytest.approx(1.0, abs=1e-15)


def test_boundary_belongs_to_next_token():
    # [c_{i-1}, c_i): u equal to c_0 = 0.5 draws token 1, u just below draws 0
    z = np.zeros(2)
    assert sample_token(z, 1.0, 0.5) == 1
    assert sample_token(z, 1.0, 0.5 - 1e-12) == 0
    assert sample_token(z, 1.0, 0.0) == 0


def test_low_temperature_is_greedy():
    rng = np.random.default_rng(5)
    for _ in range(20):
        z = rng.normal(size=50)
        z[int(np.argmax(z))] += 1.0  # a clear winner, 1000 temperatures ahead
        for u in (0.0, 0.3, 0.999999):
            assert sample_token(z, 1e-3, u) == int(np.argmax(z))


def test_high_temperature_is_uniform():
    # T -> infinity: p_i -> 1/V, so u in the middle of [i/V, (i+1)/V) draws i
    z = np.array([0.5, -0.25, 0.125, 0.0, 1.0])
    V = len(z)
    for i in range(V):
        assert sample_token(z, 1e9, (i + 0.5) / V) == i


def test_shift_invariance_and_zero_probability_tokens():
    z = np.array([0.0, 2.0, -1.0, 1.5])
    for u in np.linspace(0, 0.999, 37):
        assert sample_token(z, 0.7, u) == sample_token(z + 100.0, 0.7, u)
    # a token 2000 temperatures below the top has probability 0 in float64 and is never drawn
    z = np.array([0.0, -2000.0, 0.0])
    assert {sample_token(z, 1.0, u) for u in np.linspace(0, 0.999, 101)} == {0, 2}


def test_argument_checks():
    with pytest.raises(ValueError):
        sample_token(np.zeros(3), 0.0, 0.5)
    with pytest.raises(ValueError):
        sample_token(np.zeros(3), 1.0, 1.0)

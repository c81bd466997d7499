"""Pins of the oracle's top-k selection (oracle/select.py)."""
import numpy as np
import pytest

from oracle.forward import argmax_first
from oracle.select import top_k


def test_k1_is_the_first_argmax():
    rng = np.random.default_rng(1)
    y = rng.normal(size=(20, 300))
    y[3, [7, 50, 299]] = 10.0  # a three-way tie at the top
    v, i = top_k(y, 1)
    assert np.array_equal(i[:, 0], argmax_first(y)) and i[3, 0] == 7


def test_brute_force_small_rows():
    rng = np.random.default_rng(2)
    y = rng.integers(-3, 4, size=(30, 11)).astype(np.float64)  # many ties
    for K in (1, 4, 11):
        v, i = top_k(y, K)
        for m in range(30):
            order = sorted(range(11), key=lambda c: (-y[m, c], c))[:K]
            assert list(i[m]) == order
            assert list(v[m]) == [y[m, c] for c in order]


def test_hand_built_ties_and_signed_zero():
    y = np.array([[0.0, -0.0, 1.0, 1.0, -5.0, 0.0]])
    v, i = top_k(y, 5)
    assert list(i[0]) == [2, 3, 0, 1, 5]
    assert np.array_equal(v[0], np.array([1.0, 1.0, 0.0, -0.0, 0.0]))
    v, i = top_k(np.zeros((2, 40)), 16)
    assert np.array_equal(i, np.tile(np.arange(16), (2, 1)))


def test_rejects_bad_k():
    with pytest.raises(ValueError):
        top_k(np.zeros((2, 5)), 6)
    with pytest.raises(ValueError):
        top_k(np.zeros((2, 5)), 0)

"""Pins of the oracle's top-k selection (oracle/select.py)."""
import numpy as np
import pytest

from oracle.forward import argmax_first
from oracle.select import sample_top_k, top_k


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


def test_sampling_closed_forms():
    idx = np.tile(np.arange(100, 116), (5, 1))
    u = np.array([0.0, 0.1, 0.5, 0.93, 0.999])
    # K = 1: always the only candidate
    assert np.array_equal(sample_top_k(np.zeros((5, 1)), idx[:, :1], 0.7, u), np.full(5, 100))
    # equal values: uniform over the K, j = floor(u K)
    got = sample_top_k(np.full((5, 16), 2.5), idx, 1.3, u)
    assert np.array_equal(got, 100 + np.floor(u * 16).astype(int))
    # two candidates a > b: the second is drawn iff u >= 1 / (1 + exp((b - a) / tau))
    a, b, tau = 1.0, 0.2, 0.5
    p0 = 1 / (1 + np.exp((b - a) / tau))
    uu = np.array([p0 - 1e-9, p0 + 1e-9, 0.0, 0.999])
    got = sample_top_k(np.tile([a, b], (4, 1)), np.tile([7, 9], (4, 1)), tau, uu)
    assert list(got) == [7, 9, 7, 9]
    # tau -> 0: greedy (the largest) for every u < 1
    v = np.tile(np.linspace(3, 0, 16), (5, 1))
    assert np.array_equal(sample_top_k(v, idx, 1e-3, u), np.full(5, 100))
    with pytest.raises(ValueError):
        sample_top_k(v, idx, 0.0, u)

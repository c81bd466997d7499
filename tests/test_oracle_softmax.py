"""Pins of the oracle's log-normaliser and cross-entropy (oracle/softmax.py).

Each check is fixed by mathematics, not by re-typing the oracle: closed
forms, invariances, brute force with exact summation on tiny rows, and a
library routine.  Non-square [M, V] inputs catch a transposed target index.
"""
import math

import numpy as np
import pytest
from scipy.special import logsumexp

from oracle.softmax import cross_entropy, log_sum_exp, perplexity


def test_equal_logits_closed_form():
    # V equal logits c: lse = c + ln V; every target has nll = ln V; ppl = V
    for V, c in [(1, 0.0), (7, -3.5), (151936, 12.25), (5, 700.0)]:
        x = np.full((3, V), c)
        assert np.allclose(log_sum_exp(x), c + math.log(V), rtol=0, atol=1e-12 * max(1, abs(c)))
        nll = cross_entropy(x, np.array([0, V // 2, V - 1]))
        assert np.allclose(nll, math.log(V), rtol=0, atol=1e-9)
        assert perplexity(nll) == pytest.approx(V, rel=1e-9)


def test_single_row_vocabulary():
    x = np.array([[-2.0], [0.0], [3.25]])
    assert np.array_equal(log_sum_exp(x), x[:, 0])
    assert np.array_equal(cross_entropy(x, np.zeros(3, dtype=np.int64)), np.zeros(3))


def test_two_way_softplus():
    # lse(a, b) = a + ln(1 + e^(b - a)); nll of target 0 = softplus(b - a)
    rng = np.random.default_rng(3)
    a, b = rng.normal(0, 5, 50), rng.normal(0, 5, 50)
    x = np.stack([a, b], axis=1)
    sp = np.array([math.log1p(math.exp(bi - ai)) if bi < ai else (bi - ai) + math.log1p(math.exp(ai - bi))
                   for ai, bi in zip(a, b)])
    assert np.allclose(log_sum_exp(x), a + sp, rtol=0, atol=1e-12)
    assert np.allclose(cross_entropy(x, np.zeros(50, dtype=np.int64)), sp, rtol=0, atol=1e-12)
    assert np.allclose(cross_entropy(x, np.ones(50, dtype=np.int64)), sp - (b - a), rtol=0, atol=1e-12)


def test_shift_invariance_and_normalisation():
    rng = np.random.default_rng(4)
    x = rng.normal(0, 4, (6, 333))
    t = rng.integers(0, 333, 6)
    c = rng.normal(0, 100, 6)
    assert np.allclose(log_sum_exp(x + c[:, None]), log_sum_exp(x) + c, rtol=0, atol=1e-10)
    assert np.allclose(cross_entropy(x + c[:, None], t), cross_entropy(x, t), rtol=0, atol=1e-10)
    # the softmax it defines sums to one, and every nll is >= 0
    p = np.exp(x - log_sum_exp(x)[:, None])
    assert np.allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert (cross_entropy(x, t) >= 0).all()


def test_brute_force_tiny_rows():
    # M = 3 rows of V = 5: math.fsum over math.exp, target picked by hand
    x = np.array([[0.5, -1.0, 2.0, 0.0, 1.5],
                  [-3.0, -3.0, 4.0, 1.0, 0.25],
                  [10.0, 9.5, -2.0, 3.0, 0.0]])
    t = np.array([2, 0, 4])
    for m in range(3):
        lse = math.log(math.fsum(math.exp(v) for v in x[m]))
        assert log_sum_exp(x)[m] == pytest.approx(lse, rel=0, abs=1e-13)
        assert cross_entropy(x, t)[m] == pytest.approx(lse - x[m, t[m]], rel=0, abs=1e-13)


def test_against_scipy_logsumexp_large_values():
    # magnitudes where exp overflows without the max shift
    rng = np.random.default_rng(5)
    x = rng.normal(800, 30, (4, 2049))
    assert np.allclose(log_sum_exp(x), logsumexp(x, axis=1), rtol=1e-15, atol=1e-10)


def test_targets_outside_the_vocabulary_give_nan():
    x = np.zeros((4, 9))
    nll = cross_entropy(x, np.array([-1, 9, 3, 1 << 40]))
    assert np.isnan(nll[[0, 1, 3]]).all() and nll[2] == pytest.approx(math.log(9))


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        log_sum_exp(np.zeros((2, 0)))
    with pytest.raises(ValueError):
        cross_entropy(np.zeros((2, 3)), np.zeros(3, dtype=np.int64))

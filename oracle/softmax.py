"""Log-normaliser and cross-entropy of the head's logits -- TEST INFRASTRUCTURE.

The ARCHead paper ("Activation-Metric Residual Correction for LLM Output
Heads", abstract and section 1) notes that the head's logits go straight
into the softmax, and judges the packed head by the cross-entropy it adds
and by relative perplexity.  The pages print neither formula, so the oracle
takes the textbook definitions, in natural logarithms:

  lse[m] = log sum_v exp(logits[m, v])
  nll[m] = lse[m] - logits[m, targets[m]]      (= -log softmax(logits[m])[t])

and perplexity = exp(mean_m nll[m]).  A target outside [0, V) has no
defined cross-entropy: nll is NaN there.

Written out in fp64.  Subtracting the row maximum before exponentiating is
an identity in real arithmetic (log sum exp(x) = max x + log sum exp(x -
max x)); it only keeps exp from overflowing.  Parity pins live in
tests/test_oracle_softmax.py: closed forms (equal logits, V = 1, two-way
logits), shift invariance, sum_v exp(logits - lse) = 1, brute force with
math.fsum on tiny rows, and scipy's logsumexp.
"""
from __future__ import annotations

import numpy as np


def log_sum_exp(logits: np.ndarray) -> np.ndarray:
    """lse[m] = log sum_v exp(logits[m, v]) in fp64 for an [M, V] array."""
    x = np.asarray(logits, dtype=np.float64)
    if x.ndim != 2 or x.shape[1] == 0:
        raise ValueError("logits must be [M, V] with V >= 1")
    mx = x.max(axis=1)
    return mx + np.log(np.exp(x - mx[:, None]).sum(axis=1))


def cross_entropy(logits: np.ndarray, targets: np.ndarray) -> np.ndarray:
    """nll[m] = lse[m] - logits[m, targets[m]]; NaN where the target is not a row index."""
    x = np.asarray(logits, dtype=np.float64)
    t = np.asarray(targets, dtype=np.int64)
    if t.shape != (x.shape[0],):
        raise ValueError("targets must hold one index per row")
    lse = log_sum_exp(x)
    ok = (t >= 0) & (t < x.shape[1])
    picked = np.full(x.shape[0], np.nan)
    picked[ok] = x[np.arange(x.shape[0])[ok], t[ok]]
    return lse - picked


def perplexity(nll: np.ndarray) -> float:
    """exp of the mean cross-entropy over positions."""
    return float(np.exp(np.mean(np.asarray(nll, dtype=np.float64))))

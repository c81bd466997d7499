"""Top-k selection of the logits -- TEST INFRASTRUCTURE.

The ARCHead pages report how often the packed head keeps the dense head's
top-1 token (ARCHead paper, section 1; the results paragraphs); top-k
sampling draws from the same order widened to K candidates.  The plain
definition: the K vocabulary rows with the largest logits, larger value
first, equal values by lower index (the tie rule of the argmax, where -0 and
+0 are equal).  Pins in tests/test_oracle_select.py: K = 1 against the
oracle's pinned first-index argmax, brute force with Python's sort on small
rows, and hand-built ties.

Top-k sampling with temperature tau draws candidate j of the K with
probability proportional to exp((values[j] - values[0]) / tau) (the softmax
of the K logits at temperature tau; subtracting the largest changes nothing).
The uniform number u in [0, 1) is an input: the draw is the first j whose
cumulative weight exceeds u times the total.  Pins: K = 1, equal values
(j = floor(u K)), the two-way closed form, u = 0, and tau -> 0 (greedy).
"""
from __future__ import annotations

import numpy as np


def top_k(logits: np.ndarray, K: int) -> tuple[np.ndarray, np.ndarray]:
    """(values [M, K], indices [M, K]) of the K largest logits of each row."""
    y = np.asarray(logits)
    if y.ndim != 2 or not 1 <= K <= y.shape[1]:
        raise ValueError("logits must be [M, V] and 1 <= K <= V")
    # a stable sort of the negated values keeps lower indices first among equals
    idx = np.argsort(-y, axis=1, kind="stable")[:, :K]
    return np.take_along_axis(y, idx, axis=1), idx


def sample_top_k(values: np.ndarray, indices: np.ndarray, temperature: float,
                 u: np.ndarray) -> np.ndarray:
    """The vocabulary index drawn for each row from its top-k candidates."""
    v = np.asarray(values, dtype=np.float64)
    if temperature <= 0:
        raise ValueError("temperature must be positive")
    w = np.exp((v - v[:, :1]) / temperature)
    c = np.cumsum(w, axis=1)
    t = np.asarray(u, dtype=np.float64) * c[:, -1]
    j = np.array([np.searchsorted(c[m], t[m], side="right") for m in range(v.shape[0])])
    j = np.minimum(j, v.shape[1] - 1)
    return np.asarray(indices)[np.arange(v.shape[0]), j]

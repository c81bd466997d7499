"""Top-k selection of the logits -- TEST INFRASTRUCTURE.

The ARCHead pages report how often the packed head keeps the dense head's
top-1 token (ARCHead paper, section 1; the results paragraphs); top-k
sampling draws from the same order widened to K candidates.  The plain
definition: the K vocabulary rows with the largest logits, larger value
first, equal values by lower index (the tie rule of the argmax, where -0 and
+0 are equal).  Pins in tests/test_oracle_select.py: K = 1 against the
oracle's pinned first-index argmax, brute force with Python's sort on small
rows, and hand-built ties.
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

"""Dense fp64 forward of the packed ARCHead head (the plain definition).

ARCHead paper, section 3.2:
  eq 3  W_d   = Q5(A_c) Q8(B_c) + Q_SC4(W - A_c B_c)
  eq 6  W_hat = W_d + A_w B_w
  eq 7  Y_hat = H W_d^T + (H B_w^T) A_w^T
with both correction factors stored as row/group INT8 (text after eq 7).  In
terms of the stored fields (canonical layout, see oracle.layout):

  W_hat[v, j] = sA[v] sum_i A5[v,i] sB[i] B8[i,j]
              + sR[v, j // g] R4[v, j]
              + sC[v] sum_i C8[v,i] sD[i, j // g] D8[i, j]
  logits      = X W_hat^T

The oracle does not factor: it unpacks every field, forms the dense W_hat in
fp64 (a block of vocabulary rows at a time, purely to bound memory) and does
one plain matrix product per block.  Eq 7 and this product agree exactly in
real arithmetic; the factored order is the GPU's business.
"""
from __future__ import annotations

import numpy as np

from .layout import bf16_bits_to_f64, f16_bits_to_f64, unpack_r4


def dense_rows(f: dict, rows: np.ndarray) -> np.ndarray:
    """W_hat[rows, :] in fp64 (eq 6 with W_d from eq 3), from the packed fields."""
    d, g = f["d"], f["g"]
    rows = np.asarray(rows, dtype=np.int64)
    A = f["A5"][rows].astype(np.float64) * f16_bits_to_f64(f["sA"][rows])[:, None]
    B = f["B8"].astype(np.float64) * f16_bits_to_f64(f["sB"])[:, None]
    core = A @ B                                                     # (sA o A5)(sB o B8)
    R = unpack_r4(f["R4"][rows], d).astype(np.float64)
    sR = np.repeat(f16_bits_to_f64(f["sR"][rows]), g, axis=1)       # per (row, g-group)
    resid = sR * R                                                   # sR o R4
    C = f["C8"][rows].astype(np.float64) * f16_bits_to_f64(f["sC"][rows])[:, None]
    D = f["D8"].astype(np.float64) * np.repeat(f16_bits_to_f64(f["sD"]), g, axis=1)
    corr = C @ D                                                     # (sC o C8)(sD o D8)
    return core + resid + corr


def forward(f: dict, X_bits: np.ndarray, rows: np.ndarray | None = None,
            block: int = 8192) -> np.ndarray:
    """logits[m, v] = sum_j X[m, j] W_hat[v, j] (eq 7), fp64, for v in rows.

    X_bits holds bf16 bit patterns (M x d), widened exactly.  rows=None means
    every vocabulary row.
    """
    X = bf16_bits_to_f64(X_bits)
    if rows is None:
        rows = np.arange(f["V"], dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((X.shape[0], rows.shape[0]), dtype=np.float64)
    for s in range(0, rows.shape[0], block):
        Wb = dense_rows(f, rows[s:s + block])
        out[:, s:s + block] = X @ Wb.T
    return out


def argmax_first(logits: np.ndarray) -> np.ndarray:
    """Top-1 index per row; among equal maxima the lowest index wins."""
    return np.argmax(logits, axis=1).astype(np.int64)


def row_rms(logits: np.ndarray) -> np.ndarray:
    """sqrt(mean_v logits[m, v]^2) per row m (the tolerance's yardstick)."""
    return np.sqrt(np.mean(np.square(logits), axis=1))

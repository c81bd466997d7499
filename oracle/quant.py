"""Symmetric b-bit quantiser with fp16 scales.

ARCHead paper, section 3.2, eq 3: Q_b is b-bit group quantisation (Q5 for the
left core factor, Q8 for the right one, SC4 for the packed signed INT4
residual, whose group scales are stored quantised); the text after eq 7 stores both
correction factors with row/group INT8 quantisation; section 3.3 lists the
scales as FP16/BF16.  The paper does not spell the quantiser out.  Reading
taken here (each point listed in the design notes):

* symmetric, no zero point;
* scale s = fp16(absmax(group) / qmax) with qmax = 2**(b-1) - 1;
* q = clamp(round_half_even(x / s), -2**(b-1), 2**(b-1) - 1), dividing by
  the fp16-rounded scale in fp64;
* an all-zero group gets s = 0 and q = 0.
"""
from __future__ import annotations

import numpy as np


def qrange(bits: int) -> tuple[int, int]:
    return -(1 << (bits - 1)), (1 << (bits - 1)) - 1


def quantize_groups(x: np.ndarray, bits: int, group: int | None) -> tuple[np.ndarray, np.ndarray]:
    """Quantise the rows of x (R x C) in contiguous column groups.

    group=None means one group per row (row-wise scales).  Returns
    (q int8 R x C, scale fp16 bits R x C/group) -- the scale array is 1-D
    (R,) for row-wise quantisation.
    """
    x = np.asarray(x, dtype=np.float64)
    R, C = x.shape
    gsize = C if group is None else group
    if C % gsize:
        raise ValueError("group size must divide the row length")
    G = C // gsize
    lo, hi = qrange(bits)
    qmax = float(hi)
    xg = x.reshape(R, G, gsize)
    absmax = np.abs(xg).max(axis=2)
    s16 = (absmax / qmax).astype(np.float16)          # round to fp16 (nearest even)
    s = s16.astype(np.float64)
    q = np.zeros_like(xg)
    nz = s > 0
    q[nz] = np.rint(xg[nz] / s[nz][:, None])           # round half to even
    q = np.clip(q, lo, hi).astype(np.int8).reshape(R, C)
    sbits = s16.view(np.uint16)
    if group is None:
        sbits = sbits.reshape(R)
    return q, sbits


def dequantize_groups(q: np.ndarray, sbits: np.ndarray, group: int | None) -> np.ndarray:
    """s * q per group, in fp64."""
    q = np.asarray(q, dtype=np.float64)
    R, C = q.shape
    s = np.asarray(sbits, dtype=np.uint16).view(np.float16).astype(np.float64)
    if group is None:
        return q * s.reshape(R, 1)
    return (q.reshape(R, C // group, group) * s.reshape(R, C // group, 1)).reshape(R, C)

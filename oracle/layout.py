"""Canonical byte layout of the packed head, decoded the slow and plain way.

ARCHead paper, section 3.3 ("packed representation and integration" and the
"state-dict accounting" paragraph): the packed module registers only the SC4
INT4 residual with its FP16/BF16 scales, the 5-bit left and 8-bit right core
factors with their scales, the row/group INT8 correction factors, and shape
metadata.  The paper prints no byte layout, so the canonical host layout is
this package's own convention (shared with the C ABI as a contract, not as
code):

* all arrays row-major;
* R4: V x d/2 bytes; byte [v, c] holds column 2c in the low nibble and
  column 2c+1 in the high nibble, both 4-bit two's complement;
* A5: int8 per value (the device stores it at 5 bits; the host form is wide);
* B8, C8, D8: int8;
* every scale: IEEE binary16 bit pattern in a uint16;
* X: bf16 bit pattern in a uint16.
"""
from __future__ import annotations

import numpy as np


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns -> float64 (exact widening)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact widening: bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def unpack_r4(packed: np.ndarray, d: int) -> np.ndarray:
    """V x d/2 packed bytes -> V x d int8 values in [-8, 7].

    Column 2c is the low nibble of byte c, column 2c+1 the high nibble; a
    nibble n >= 8 stands for n - 16 (4-bit two's complement).
    """
    packed = np.asarray(packed, dtype=np.uint8)
    V = packed.shape[0]
    assert packed.shape == (V, d // 2)
    lo = (packed & 0x0F).astype(np.int16)
    hi = (packed >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty((V, d), dtype=np.int8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def pack_r4(values: np.ndarray) -> np.ndarray:
    """V x d int values in [-8, 7] -> V x d/2 packed bytes (inverse of unpack_r4)."""
    v = np.asarray(values, dtype=np.int16)
    if v.min(initial=0) < -8 or v.max(initial=0) > 7:
        raise ValueError("R4 values must lie in [-8, 7]")
    nib = (v & 0x0F).astype(np.uint8)
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


# --- state-dict byte accounting, ARCHead paper eq 10 -------------------------

def field_shapes(V: int, d: int, k: int, r: int, g: int) -> dict:
    """(numel, bits per element) of every registered buffer of the packed head.

    A5 is counted at 5 bits per value (the "5-bit left core factor" of the
    state-dict accounting paragraph), R4 at 4 bits, int8 fields at 8 bits and
    every scale at 16 bits.  A head without a core (k = 0) registers no core
    row scales, and one without a correction (r = 0) none for the correction.
    """
    G = d // g
    return {
        "R4": (V * d, 4), "sR": (V * G, 16),
        "A5": (V * k, 5), "sA": (V if k > 0 else 0, 16),
        "B8": (k * d, 8), "sB": (k, 16),
        "C8": (V * r, 8), "sC": (V if r > 0 else 0, 16),
        "D8": (r * d, 8), "sD": (r * G, 16),
    }


def packed_bytes(V: int, d: int, k: int, r: int, g: int) -> int:
    """Eq 10: sum over registered buffers of numel x element size, in bytes.

    Each buffer is rounded up to whole bytes on its own.
    """
    total = 0
    for numel, bits in field_shapes(V, d, k, r, g).values():
        total += (numel * bits + 7) // 8
    return total


def dense_bf16_bytes(V: int, d: int) -> int:
    """Bytes of the dense BF16 head the packed head replaces (V x d x 2)."""
    return V * d * 2

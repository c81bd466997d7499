"""ctypes loader for naive.c (the oracle's independent C triple loop).

TEST INFRASTRUCTURE ONLY.  build() compiles oracle/naive.c with gcc into
oracle/_naive.so; forward() calls it on canonical-layout numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "naive.c")
_LIB = os.path.join(_HERE, "_naive.so")
_lib = None


def build() -> str:
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-shared", "-fPIC", _SRC, "-o", _LIB, "-lm"])
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.naive_forward.restype = ctypes.c_int
        lib.naive_forward.argtypes = [ctypes.c_int64] * 6 + [ctypes.c_void_p] * 12
        _lib = lib
    return _lib


def forward(f: dict, X_bits: np.ndarray) -> np.ndarray:
    """fp64 logits (M x V) from the C triple loop."""
    lib = _load()
    arrs = {}
    for name, dt in [("A5", np.int8), ("sA", np.uint16), ("B8", np.int8), ("sB", np.uint16),
                     ("R4", np.uint8), ("sR", np.uint16), ("C8", np.int8), ("sC", np.uint16),
                     ("D8", np.int8), ("sD", np.uint16)]:
        arrs[name] = np.ascontiguousarray(f[name], dtype=dt)
    X = np.ascontiguousarray(X_bits, dtype=np.uint16)
    M = X.shape[0]
    out = np.empty((M, f["V"]), dtype=np.float64)
    rc = lib.naive_forward(f["V"], f["d"], f["k"], f["r"], f["g"], M,
                           *[arrs[n].ctypes.data for n in
                             ["A5", "sA", "B8", "sB", "R4", "sR", "C8", "sC", "D8", "sD"]],
                           X.ctypes.data, out.ctypes.data)
    if rc:
        raise ValueError("naive_forward rejected the shape")
    return out

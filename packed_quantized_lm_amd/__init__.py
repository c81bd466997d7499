"""Packed ARCHead LM-head forward for MI355X (gfx950).

The forward of the ARCHead packed output head (logits = X W_hat^T with
W_hat = (sA o A5)(sB o B8) + sR o R4 + (sC o C8)(sD o D8), factored so that
W_hat is never materialised) runs in hand-written HIP kernels behind the C
ABI in include/archead.h.  `binding.PackedHead` is the Python face of that
ABI; `binding.build_head` constructs a packed head on the GPU from a dense
head and calibration states; `synth` draws seeded synthetic inputs.
"""
from .binding import PackedHead, build_head, load_library, quantize, x_tensor_from_bits  # noqa: F401

__all__ = ["PackedHead", "build_head", "load_library", "quantize", "x_tensor_from_bits"]

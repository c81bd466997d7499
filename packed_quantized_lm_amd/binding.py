"""Thin Python binding of libarchead.so (the C ABI in include/archead.h).

Argument marshalling only: numpy arrays in the canonical host layout go to
archead_pack_load; torch CUDA tensors provide device memory for X, logits and
argmax, and torch's current stream is passed down as the hipStream_t.  Every
step of the forward runs in the library's HIP kernels.  There is no other
implementation behind this module: if the library is missing it raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libarchead.so")

OK, EINVAL, ESHAPE, ERANGE, ENOMEM, EHIP = range(6)
PATH_AUTO, PATH_GEMV, PATH_SKINNY, PATH_LDS = range(4)
PATHS = {"auto": PATH_AUTO, "gemv": PATH_GEMV, "skinny": PATH_SKINNY, "lds": PATH_LDS}

# exported symbol -> (restype, argtypes)
_VP = ctypes.c_void_p
_I64 = ctypes.c_int64
SIGNATURES = {
    "archead_pack_load": (ctypes.c_int, [_I64] * 5 + [_VP] * 10 + [_VP, ctypes.POINTER(_VP)]),
    "archead_reserve": (ctypes.c_int, [_VP, _I64, _VP]),
    "archead_forward": (ctypes.c_int, [_VP, _I64, _VP, _VP, _VP]),
    "archead_forward_argmax": (ctypes.c_int, [_VP, _I64, _VP, _VP, _VP, _VP]),
    "archead_forward_path": (ctypes.c_int, [_VP, _I64, _VP, _VP, _VP, ctypes.c_int, _VP]),
    "archead_forward_argmax_noalloc": (ctypes.c_int, [_VP, _I64, _VP, _VP, _VP, _VP]),
    "archead_forward_timed": (ctypes.c_int, [_VP, _I64, _VP, _VP, _VP, ctypes.c_int, _VP, _VP, _VP]),
    "archead_forward_ce": (ctypes.c_int, [_VP, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    "archead_forward_topk": (ctypes.c_int, [_VP, _I64, _VP, ctypes.c_int32, _VP, _VP, _VP, _VP]),
    "archead_forward_topk_path": (ctypes.c_int, [_VP, _I64, _VP, ctypes.c_int32, _VP, _VP, _VP, ctypes.c_int,
                                                 _VP]),
    "archead_forward_sample": (ctypes.c_int, [_VP, _I64, _VP, ctypes.c_int32, ctypes.c_float, _VP, _VP, _VP, _VP,
                                              _VP, _VP]),
    "archead_forward_ce_path": (ctypes.c_int, [_VP, _I64, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_int, _VP]),
    "archead_build": (ctypes.c_int, [_I64] * 6 + [_VP, _VP, ctypes.c_double, ctypes.c_double, ctypes.c_int,
                                                    ctypes.c_int, ctypes.c_uint64] + [_VP] * 10 + [_VP]),
    "archead_quantize": (ctypes.c_int, [_VP, _I64, _I64, ctypes.c_int, _I64, _VP, _VP, _VP]),
    "archead_packed_bytes": (ctypes.c_int, [_VP, ctypes.POINTER(ctypes.c_uint64)]),
    "archead_device_bytes": (ctypes.c_int, [_VP, ctypes.POINTER(ctypes.c_uint64)]),
    "archead_free": (ctypes.c_int, [_VP]),
    "archead_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "archead_last_error": (ctypes.c_char_p, []),
}

_lib = None


class ArcheadError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


def load_library(path: str = LIB_PATH):
    """Load libarchead.so (built by packed_quantized_lm_amd.build); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m packed_quantized_lm_amd.build`")
    # torch first: its HIP runtime is then the one the library binds to (same
    # soname), so torch's streams and allocations are valid inside the library
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != OK:
        lib = load_library()
        detail = lib.archead_last_error().decode() or lib.archead_status_string(status).decode()
        raise ArcheadError(status, where, detail)


def _np_ptr(a):
    return None if a is None else a.ctypes.data


def _stream_handle(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtypes, shape, device):
    """Raise before any launch unless t is a contiguous device tensor of one of
    dtypes, of the given shape, on device (the library takes raw pointers: a
    host tensor or a wrong element type would be read as garbage or fault)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda" or t.device != device:
        raise ValueError(f"{name} must live on {device}, not {t.device}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must have dtype {' or '.join(str(d) for d in dtypes)}, not {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_FIELD_DTYPES = [("A5", np.int8), ("sA", np.uint16), ("B8", np.int8), ("sB", np.uint16),
                 ("R4", np.uint8), ("sR", np.uint16), ("C8", np.int8), ("sC", np.uint16),
                 ("D8", np.int8), ("sD", np.uint16)]


class PackedHead:
    """A packed ARCHead head resident on the current HIP device."""

    def __init__(self, fields: dict, stream=None):
        lib = load_library()
        self.V, self.d, self.k, self.r, self.g = (int(fields[n]) for n in ("V", "d", "k", "r", "g"))
        arrs = {}
        for name, dt in _FIELD_DTYPES:
            a = fields.get(name)
            arrs[name] = None if a is None else np.ascontiguousarray(a, dtype=dt)
        handle = ctypes.c_void_p()
        st = lib.archead_pack_load(self.V, self.d, self.k, self.r, self.g,
                                   *[_np_ptr(arrs[n]) for n, _ in _FIELD_DTYPES],
                                   _stream_handle(stream), ctypes.byref(handle))
        _check(st, "archead_pack_load")
        self._h = handle

    @property
    def handle(self):
        if self._h is None:
            raise ValueError("head was freed")
        return self._h

    def reserve(self, M_max: int, stream=None):
        _check(load_library().archead_reserve(self.handle, int(M_max), _stream_handle(stream)),
               "archead_reserve")

    def packed_bytes(self) -> int:
        out = ctypes.c_uint64()
        _check(load_library().archead_packed_bytes(self.handle, ctypes.byref(out)), "archead_packed_bytes")
        return out.value

    def device_bytes(self) -> int:
        out = ctypes.c_uint64()
        _check(load_library().archead_device_bytes(self.handle, ctypes.byref(out)), "archead_device_bytes")
        return out.value

    def _check_x(self, X):
        """X: a contiguous bf16 (or 16-bit bit-pattern) M x d device tensor; returns M."""
        import torch
        if not isinstance(X, torch.Tensor) or X.dim() != 2:
            raise ValueError(f"X must be an M x {self.d} tensor")
        if X.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
            raise TypeError("X must hold bf16 values")
        _need(X, "X", (X.dtype,), (X.shape[0], self.d), X.device)
        return int(X.shape[0])

    def _check_out(self, X, logits=None, argmax=None):
        import torch
        M = self._check_x(X)
        if logits is not None:
            _need(logits, "logits", (torch.float32,), (M, self.V), X.device)
        if argmax is not None:
            _need(argmax, "argmax", (torch.int32,), (M,), X.device)
        return M

    def forward_into(self, X, logits, argmax, path: str | int = "auto", stream=None):
        """Enqueue the forward writing into preallocated torch tensors (either
        of logits / argmax may be None).  X: bf16 (or int16 bit patterns) M x d."""
        p = PATHS[path] if isinstance(path, str) else int(path)
        M = self._check_out(X, logits, argmax)
        st = load_library().archead_forward_path(
            self.handle, M, ctypes.c_void_p(X.data_ptr()),
            None if logits is None else ctypes.c_void_p(logits.data_ptr()),
            None if argmax is None else ctypes.c_void_p(argmax.data_ptr()),
            p, _stream_handle(stream))
        _check(st, "archead_forward_path")

    def forward_argmax_noalloc_into(self, X, logits, argmax, stream=None):
        """Enqueue archead_forward_argmax_noalloc: the forward and its argmax
        into preallocated tensors (logits may be None), on the library's fixed
        per-GPU workspace -- nothing is allocated."""
        M = self._check_out(X, logits, argmax)
        if argmax is None:
            raise ValueError("argmax is required")
        st = load_library().archead_forward_argmax_noalloc(
            self.handle, M, ctypes.c_void_p(X.data_ptr()),
            None if logits is None else ctypes.c_void_p(logits.data_ptr()),
            ctypes.c_void_p(argmax.data_ptr()), _stream_handle(stream))
        _check(st, "archead_forward_argmax_noalloc")

    def forward_timed(self, X, logits, argmax, ev_before, ev_after, path: str | int = "auto",
                      stream=None):
        """forward_into that also records the torch.cuda.Event pair around the
        vocabulary-tile kernel on the same stream."""
        p = PATHS[path] if isinstance(path, str) else int(path)
        M = self._check_out(X, logits, argmax)
        st = load_library().archead_forward_timed(
            self.handle, M, ctypes.c_void_p(X.data_ptr()),
            None if logits is None else ctypes.c_void_p(logits.data_ptr()),
            None if argmax is None else ctypes.c_void_p(argmax.data_ptr()),
            p, _stream_handle(stream), ctypes.c_void_p(ev_before.cuda_event),
            ctypes.c_void_p(ev_after.cuda_event))
        _check(st, "archead_forward_timed")

    def forward_ce_into(self, X, targets, logits, argmax, lse, nll, path: str | int = "auto",
                        stream=None):
        """Enqueue the forward with the log-normaliser lse (and, with int32
        targets, the cross-entropy nll) into preallocated torch tensors;
        targets / nll, logits and argmax may be None."""
        import torch
        p = PATHS[path] if isinstance(path, str) else int(path)
        M = self._check_out(X, logits, argmax)
        for t, name, dt in ((targets, "targets", torch.int32), (lse, "lse", torch.float32),
                            (nll, "nll", torch.float32)):
            if t is not None:
                _need(t, name, (dt,), (M,), X.device)

        def ptr(t):
            return None if t is None else ctypes.c_void_p(t.data_ptr())
        st = load_library().archead_forward_ce_path(
            self.handle, M, ctypes.c_void_p(X.data_ptr()), ptr(targets), ptr(logits),
            ptr(argmax), ptr(lse), ptr(nll), p, _stream_handle(stream))
        _check(st, "archead_forward_ce_path")

    def forward_ce(self, X, targets=None, want_logits: bool = False, want_argmax: bool = False,
                   path: str | int = "auto", stream=None):
        """Returns (lse fp32 M, nll fp32 M or None, logits or None, argmax or None)."""
        import torch
        if X.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
            raise TypeError("X must hold bf16 values")
        if X.dim() != 2 or X.shape[1] != self.d or not X.is_contiguous():
            raise ValueError(f"X must be a contiguous M x {self.d} tensor")
        M = X.shape[0]
        if targets is not None and (targets.dtype != torch.int32 or targets.shape != (M,)
                                    or not targets.is_contiguous()):
            raise ValueError("targets must be a contiguous int32 tensor of M entries")
        dev = X.device
        lse = torch.empty((M,), dtype=torch.float32, device=dev)
        nll = torch.empty((M,), dtype=torch.float32, device=dev) if targets is not None else None
        logits = torch.empty((M, self.V), dtype=torch.float32, device=dev) if want_logits else None
        argmax = torch.empty((M,), dtype=torch.int32, device=dev) if want_argmax else None
        self.forward_ce_into(X, targets, logits, argmax, lse, nll, path=path, stream=stream)
        return lse, nll, logits, argmax

    def forward_topk_into(self, X, K: int, logits, values, indices, path: str | int = "auto", stream=None):
        """Enqueue the forward plus the K largest logits per row into preallocated
        torch tensors (logits M x V, values M x K fp32, indices M x K int32)."""
        import torch
        p = PATHS[path] if isinstance(path, str) else int(path)
        M = self._check_out(X, logits)
        if logits is None:
            raise ValueError("logits is required")
        _need(values, "values", (torch.float32,), (M, int(K)), X.device)
        _need(indices, "indices", (torch.int32,), (M, int(K)), X.device)
        st = load_library().archead_forward_topk_path(
            self.handle, M, ctypes.c_void_p(X.data_ptr()), int(K),
            ctypes.c_void_p(logits.data_ptr()), ctypes.c_void_p(values.data_ptr()),
            ctypes.c_void_p(indices.data_ptr()), p, _stream_handle(stream))
        _check(st, "archead_forward_topk_path")

    def forward_topk(self, X, K: int, path: str | int = "auto", stream=None):
        """Returns (values fp32 M x K, indices int32 M x K, logits fp32 M x V)."""
        import torch
        M = X.shape[0]
        logits = torch.empty((M, self.V), dtype=torch.float32, device=X.device)
        values = torch.empty((M, K), dtype=torch.float32, device=X.device)
        indices = torch.empty((M, K), dtype=torch.int32, device=X.device)
        self.forward_topk_into(X, K, logits, values, indices, path=path, stream=stream)
        return values, indices, logits

    def forward_sample_into(self, X, K: int, temperature: float, u, logits, values, indices, samples,
                            stream=None):
        """Enqueue the forward, the top K and one draw per row at the given
        temperature from the uniform numbers u (fp32 M, in [0, 1))."""
        import torch
        M = self._check_out(X, logits)
        if logits is None:
            raise ValueError("logits is required")
        _need(values, "values", (torch.float32,), (M, int(K)), X.device)
        _need(indices, "indices", (torch.int32,), (M, int(K)), X.device)
        _need(u, "u", (torch.float32,), (M,), X.device)
        _need(samples, "samples", (torch.int32,), (M,), X.device)
        ptr = lambda t: ctypes.c_void_p(t.data_ptr())
        st = load_library().archead_forward_sample(
            self.handle, M, ptr(X), int(K), float(temperature), ptr(u), ptr(logits),
            ptr(values), ptr(indices), ptr(samples), _stream_handle(stream))
        _check(st, "archead_forward_sample")

    def forward_sample(self, X, K: int, temperature: float, u, stream=None):
        """Returns (samples int32 M, values M x K, indices M x K, logits M x V)."""
        import torch
        M = X.shape[0]
        dev = X.device
        logits = torch.empty((M, self.V), dtype=torch.float32, device=dev)
        values = torch.empty((M, K), dtype=torch.float32, device=dev)
        indices = torch.empty((M, K), dtype=torch.int32, device=dev)
        samples = torch.empty((M,), dtype=torch.int32, device=dev)
        self.forward_sample_into(X, K, temperature, u, logits, values, indices, samples, stream=stream)
        return samples, values, indices, logits

    def forward(self, X, want_logits: bool = True, want_argmax: bool = False,
                path: str | int = "auto", stream=None):
        """Returns (logits fp32 M x V or None, argmax int32 M or None) as torch tensors."""
        import torch
        if X.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
            raise TypeError("X must hold bf16 values")
        if X.dim() != 2 or X.shape[1] != self.d or not X.is_contiguous():
            raise ValueError(f"X must be a contiguous M x {self.d} tensor")
        M = X.shape[0]
        logits = torch.empty((M, self.V), dtype=torch.float32, device=X.device) if want_logits else None
        argmax = torch.empty((M,), dtype=torch.int32, device=X.device) if want_argmax else None
        self.forward_into(X, logits, argmax, path=path, stream=stream)
        return logits, argmax

    def close(self):
        if self._h is not None:
            _check(load_library().archead_free(self._h), "archead_free")
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def quantize(x, bits: int, group: int | None = None, stream=None):
    """archead_quantize on a DEVICE fp64 rows x cols tensor: (codes int8,
    fp16 scale bits as int16) torch tensors; group=None means one group per row."""
    import torch
    rows, cols = (int(n) for n in x.shape)
    group = cols if group is None else int(group)
    if cols % group:
        raise ValueError("group must divide the row length")
    _need(x, "x", (torch.float64,), (rows, cols), x.device)
    q = torch.empty((rows, cols), dtype=torch.int8, device=x.device)
    s = torch.empty((rows, cols // group), dtype=torch.int16, device=x.device)
    _check(load_library().archead_quantize(ctypes.c_void_p(x.data_ptr()), rows, cols, int(bits), group,
                                           ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(s.data_ptr()),
                                           _stream_handle(stream)), "archead_quantize")
    return q, s


def build_head(W, H, k: int, r: int, g: int, p: float = 0.75, lam: float = 1e-2, power_iters: int = 2,
               oversample: int = 16, seed: int = 0, stream=None) -> dict:
    """archead_build on DEVICE fp64 tensors W (V x d) and H (N x d); returns the
    packed fields in the canonical host layout (numpy), as archead_pack_load takes them."""
    import torch
    V, d = (int(n) for n in W.shape)
    N = int(H.shape[0])
    _need(W, "W", (torch.float64,), (V, d), W.device)
    _need(H, "H", (torch.float64,), (N, d), W.device)
    dev = W.device
    G = d // g if g and d % g == 0 else 0
    out = {
        "A5": torch.empty((V, k), dtype=torch.int8, device=dev), "sA": torch.empty((V,), dtype=torch.int16, device=dev),
        "B8": torch.empty((k, d), dtype=torch.int8, device=dev), "sB": torch.empty((k,), dtype=torch.int16, device=dev),
        "R4": torch.empty((V, d // 2), dtype=torch.uint8, device=dev),
        "sR": torch.empty((V, G), dtype=torch.int16, device=dev),
        "C8": torch.empty((V, r), dtype=torch.int8, device=dev), "sC": torch.empty((V,), dtype=torch.int16, device=dev),
        "D8": torch.empty((r, d), dtype=torch.int8, device=dev),
        "sD": torch.empty((r, G), dtype=torch.int16, device=dev),
    }
    order = ["A5", "sA", "B8", "sB", "R4", "sR", "C8", "sC", "D8", "sD"]
    ptrs = [ctypes.c_void_p(out[n].data_ptr()) if out[n].numel() else None for n in order]
    _check(load_library().archead_build(V, d, int(k), int(r), int(g), N, ctypes.c_void_p(W.data_ptr()),
                                        ctypes.c_void_p(H.data_ptr()), float(p), float(lam), int(power_iters),
                                        int(oversample), int(seed) & (2 ** 64 - 1), *ptrs, _stream_handle(stream)),
           "archead_build")
    fields = {"V": V, "d": d, "k": int(k), "r": int(r), "g": int(g)}
    for n in order:
        a = out[n].cpu().numpy()
        fields[n] = a.view(np.uint16) if n.startswith("s") else a
    return fields


def x_tensor_from_bits(bits: np.ndarray, device="cuda"):
    """bf16 bit patterns (uint16 numpy) -> torch.bfloat16 device tensor (bitwise)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.to(device).view(torch.bfloat16)

"""The C-ABI library without a GPU: it loads, exports every symbol that
include/archead.h declares, and rejects bad arguments before touching the
device (no compute call is made here)."""
import ctypes
import os
import re

import numpy as np
import pytest

from packed_quantized_lm_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "archead.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from packed_quantized_lm_amd import build
        build.build()
    return binding.load_library()


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(archead_\w+)\s*\(", text)))


def test_header_declares_the_documented_entry_points():
    syms = declared_symbols()
    for name in ["archead_pack_load", "archead_forward", "archead_forward_argmax",
                 "archead_forward_path", "archead_forward_timed", "archead_forward_ce",
                 "archead_forward_ce_path", "archead_forward_topk", "archead_forward_topk_path",
                 "archead_forward_sample",
                 "archead_reserve", "archead_packed_bytes",
                 "archead_device_bytes", "archead_free", "archead_status_string",
                 "archead_last_error"]:
        assert name in syms
    assert set(syms) == set(binding.SIGNATURES)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(6):
        assert lib.archead_status_string(code).decode().startswith("ARCHEAD")


def _fields(V=32, d=128, k=8, r=4, g=32):
    from packed_quantized_lm_amd.synth import random_head
    return random_head(V, d, k, r, g, seed=1)


def _load(lib, f, **over):
    f = dict(f, **over)
    h = ctypes.c_void_p()
    ptr = lambda n, dt: None if f.get(n) is None else np.ascontiguousarray(f[n], dtype=dt).ctypes.data
    arrs = [ptr("A5", np.int8), ptr("sA", np.uint16), ptr("B8", np.int8), ptr("sB", np.uint16),
            ptr("R4", np.uint8), ptr("sR", np.uint16), ptr("C8", np.int8), ptr("sC", np.uint16),
            ptr("D8", np.int8), ptr("sD", np.uint16)]
    st = lib.archead_pack_load(f["V"], f["d"], f["k"], f["r"], f["g"], *arrs, None, ctypes.byref(h))
    return st, h


@pytest.mark.parametrize("over,status", [
    (dict(V=0), binding.ESHAPE),
    (dict(d=96), binding.ESHAPE),
    (dict(d=200), binding.ESHAPE),
    (dict(g=48), binding.ESHAPE),
    (dict(g=256), binding.ESHAPE),       # does not divide d = 128
    (dict(k=5000), binding.ESHAPE),
    (dict(r=-1), binding.ESHAPE),
    (dict(R4=None), binding.EINVAL),
    (dict(sR=None), binding.EINVAL),
    (dict(A5=None), binding.EINVAL),
    (dict(D8=None), binding.EINVAL),
])
def test_pack_load_rejects_bad_arguments_before_any_device_work(lib, over, status):
    st, h = _load(lib, _fields(), **over)
    assert st == status
    assert h.value is None
    assert lib.archead_last_error().decode() != ""


def test_pack_load_rejects_out_of_range_core_codes(lib):
    f = _fields()
    a5 = f["A5"].copy()
    a5[3, 2] = 16
    st, h = _load(lib, f, A5=a5)
    assert st == binding.ERANGE
    assert b"[-16, 15]" in lib.archead_last_error()


def test_calls_on_null_or_unknown_handles(lib):
    out = ctypes.c_uint64()
    assert lib.archead_packed_bytes(None, ctypes.byref(out)) == binding.EINVAL
    assert lib.archead_forward(None, 1, None, None, None) == binding.EINVAL
    assert lib.archead_forward_path(None, 1, None, None, None, 0, None) == binding.EINVAL
    assert lib.archead_reserve(None, 4, None) == binding.EINVAL
    assert lib.archead_free(None) == binding.OK
    bogus = ctypes.c_void_p(0x1234560)
    assert lib.archead_free(bogus) == binding.EINVAL
    assert lib.archead_forward(bogus, 1, None, None, None) == binding.EINVAL


def test_binding_raises_without_the_library(tmp_path):
    with pytest.raises(ImportError):
        binding._lib_backup = binding._lib
        try:
            binding._lib = None
            binding.load_library(str(tmp_path / "missing.so"))
        finally:
            binding._lib = binding._lib_backup


def test_forward_ce_rejects_missing_outputs_and_bad_handles(lib):
    buf = ctypes.c_void_p(16)  # never dereferenced: every call fails its checks first
    # lse is required
    assert lib.archead_forward_ce(None, 1, buf, None, None, None, None, None, None) == binding.EINVAL
    assert "lse" in lib.archead_last_error().decode()
    # a handle that is not live
    assert lib.archead_forward_ce(None, 1, buf, None, None, None, buf, None, None) == binding.EINVAL
    assert lib.archead_forward_ce_path(ctypes.c_void_p(12345), 1, buf, None, None, None, buf, None, 0,
                                       None) == binding.EINVAL


def test_forward_topk_rejects_missing_buffers_and_bad_handles(lib):
    buf = ctypes.c_void_p(16)  # never dereferenced: every call fails its checks first
    assert lib.archead_forward_topk(None, 1, buf, 4, None, buf, buf, None) == binding.EINVAL
    assert lib.archead_forward_topk(None, 1, buf, 4, buf, None, buf, None) == binding.EINVAL
    assert lib.archead_forward_topk(None, 1, buf, 4, buf, buf, buf, None) == binding.EINVAL
    assert "handle" in lib.archead_last_error().decode()


def test_forward_sample_rejects_bad_temperature_and_missing_buffers(lib):
    buf = ctypes.c_void_p(16)  # never dereferenced: every call fails its checks first
    for tau in (0.0, -1.0, float("inf"), float("nan")):
        assert lib.archead_forward_sample(None, 1, buf, 4, tau, buf, buf, buf, buf, buf, None) == binding.EINVAL
    assert lib.archead_forward_sample(None, 1, buf, 4, 1.0, None, buf, buf, buf, buf, None) == binding.EINVAL
    assert lib.archead_forward_sample(None, 1, buf, 4, 1.0, buf, buf, buf, buf, buf, None) == binding.EINVAL


def test_pack_load_reports_enomem_under_the_allocation_limit(lib, monkeypatch):
    """ARCHEAD_TEST_ALLOC_LIMIT refuses the packed head's device block before
    any HIP call: a status, never an abort, and no handle."""
    monkeypatch.setenv("ARCHEAD_TEST_ALLOC_LIMIT", "4096")
    st, h = _load(lib, _fields())
    assert st == binding.ENOMEM
    assert h.value is None
    assert b"ARCHEAD_TEST_ALLOC_LIMIT" in lib.archead_last_error()


def test_build_reports_enomem_under_the_allocation_limit(lib, monkeypatch):
    """The construction's first device allocation (the d x d metric) is refused
    under the limit; the call returns ENOMEM without touching W or H."""
    monkeypatch.setenv("ARCHEAD_TEST_ALLOC_LIMIT", "0")
    V, d, k, r, g, N = 64, 128, 8, 4, 32, 16
    dummy = np.zeros(8, dtype=np.float64)
    bufs = {n: np.zeros(16, dtype=np.int8) for n in ["A5", "sA", "B8", "sB", "R4", "sR", "C8", "sC", "D8", "sD"]}
    p = lambda n: bufs[n].ctypes.data
    st = lib.archead_build(V, d, k, r, g, N, dummy.ctypes.data, dummy.ctypes.data, 0.75, 1e-2, 2, 16, 7,
                           p("A5"), p("sA"), p("B8"), p("sB"), p("R4"), p("sR"), p("C8"), p("sC"), p("D8"),
                           p("sD"), None)
    assert st == binding.ENOMEM
    assert b"device allocation" in lib.archead_last_error()
    monkeypatch.setenv("ARCHEAD_TEST_ALLOC_LIMIT", "")
    st = lib.archead_quantize(dummy.ctypes.data, 0, 8, 4, 8, p("A5"), p("sA"), None)
    assert st == binding.OK or st == binding.EHIP  # no limit: the hook is off (rows = 0 launches nothing)

"""GPU parity of the baseline heads the pages compare against, at the Qwen
head's full shape and on the same kernels: a plain group-INT4 head (k = r = 0,
g = 32, the storage-matched group size) and SVD8 + INT4 (a rank-256 INT8 pair,
no correction).  Every logit against the fp64 oracle at M = 1 on every path
that takes the shape; sampled vocabulary rows at M = 2048."""
import numpy as np
import pytest

from gpu_util import TOL, assert_argmax_ok, assert_logits_close, gpu_forward, row_rms, say
from oracle import forward as oracle_forward
from oracle.layout import packed_bytes
from packed_quantized_lm_amd.synth import make_config

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from packed_quantized_lm_amd import load_library
    load_library()


def load(fields):
    from packed_quantized_lm_amd import PackedHead
    return PackedHead(fields)


@pytest.mark.parametrize("name,paths", [("int4_g32_m1", ["auto", "gemv", "skinny"]),
                                        ("svd8_int4_m1", ["auto", "gemv", "skinny"])])
def test_baseline_decode_full_oracle(name, paths):
    say(f"baseline {name}: generating + loading")
    c = make_config(name)
    h = load(c)
    assert h.packed_bytes() == packed_bytes(c["V"], c["d"], c["k"], c["r"], c["g"])
    say(f"baseline {name}: oracle")
    ref = oracle_forward.forward(c, c["X"])
    for path in paths:
        say(f"baseline {name}: GPU path={path}")
        y, a = gpu_forward(h, c["X"], path=path)
        ratio = assert_logits_close(y, ref, what=f"{name} {path}")
        assert_argmax_ok(a, y, ref, what=f"{name} {path}")
        say(f"baseline {name} {path}: worst |d|/(2e-3 rms) = {ratio:.3g}")
    h.close()


@pytest.mark.parametrize("name", ["int4_g32_m2048", "svd8_int4_m2048"])
def test_baseline_prefill_sampled(name):
    say(f"baseline {name}: generating + loading")
    c = make_config(name)
    h = load(c)
    say(f"baseline {name}: GPU forward M={c['M']}")
    y, a = gpu_forward(h, c["X"])
    assert np.array_equal(a, np.argmax(y, axis=1))
    rng = np.random.default_rng(2)
    rows = np.unique(np.concatenate([np.arange(32), np.arange(c["V"] - 32, c["V"]),
                                     rng.choice(c["V"], 448, replace=False)]))
    say(f"baseline {name}: oracle on {rows.size} sampled rows")
    ref = oracle_forward.forward(c, c["X"], rows=rows)
    ratio = assert_logits_close(y[:, rows], ref, rms=row_rms(ref), what=name)
    say(f"baseline {name}: worst sampled |d|/(2e-3 rms) = {ratio:.3g}")
    h.close()

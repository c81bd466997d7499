"""GPU parity of the HIP path against the CPU oracle (called through the C ABI).

Small cases compare every logit; the full-size workloads compare the full
oracle where it finishes in seconds (M <= 32) and sampled vocabulary rows
otherwise (plus properties that hold at any size).
"""
import numpy as np
import pytest

from gpu_util import TOL, assert_argmax_ok, assert_logits_close, gpu_forward, row_rms, say
from oracle import forward as oracle_forward
from packed_quantized_lm_amd.synth import make_config, random_small_head, to_bf16_bits, to_f16_bits

pytestmark = pytest.mark.gpu

PATHS = ["skinny", "lds"]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from packed_quantized_lm_amd import load_library
    load_library()
    return torch.device("cuda:0")


def load(fields):
    from packed_quantized_lm_amd import PackedHead
    return PackedHead(fields)


# --- tiny head packed by the oracle's construction -----------------------------

@pytest.fixture(scope="module")
def tiny():
    from oracle import packer
    c = make_config("tiny")
    f, _ = packer.pack(c["W"], c["H"], c["k"], c["r"], c["g"], p=0.75, lam=1e-2)
    return f, c["X"]


@pytest.mark.parametrize("path", ["auto"] + PATHS)
def test_tiny_config(tiny, path):
    f, X = tiny
    say(f"tiny V=2048 d=256 k=16 r=4 g=32 M=4 path={path}")
    h = load(f)
    ref = oracle_forward.forward(f, X)
    y, a = gpu_forward(h, X, path=path)
    assert_logits_close(y, ref, what="tiny")
    assert_argmax_ok(a, y, ref, what="tiny")
    h.close()


# --- ragged shapes ----------------------------------------------------------------

SHAPES = [
    # V,     d,   k,  r,   g,  M
    (1, 128, 1, 1, 32, 1),
    (15, 128, 8, 4, 32, 2),
    (17, 256, 16, 4, 64, 3),
    (1000, 384, 33, 7, 128, 5),
    (1000, 384, 33, 7, 96, 17),
    (4099, 640, 64, 48, 128, 31),
    (777, 512, 0, 16, 256, 8),     # no core term
    (777, 512, 40, 0, 512, 33),    # no correction term
    (300, 1024, 256, 64, 128, 64),
    (2500, 256, 16, 4, 32, 1),
    (3001, 512, 40, 20, 128, 2),   # two-chunk decode pipeline
    (5000, 1024, 96, 33, 128, 5),  # two-chunk decode pipeline
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "V{}_d{}_k{}_r{}_g{}_M{}".format(*s))
@pytest.mark.parametrize("path", PATHS)
def test_ragged_shapes(shape, path):
    V, d, k, r, g, M = shape
    say(f"ragged {shape} path={path}")
    f = random_small_head(V, d, k, r, g, M, seed=V * 7 + d + M, n_outliers=2, outlier_factor=20.0)
    h = load(f)
    ref = oracle_forward.forward(f, f["X"])
    y, a = gpu_forward(h, f["X"], path=path)
    assert_logits_close(y, ref, what=str(shape))
    assert_argmax_ok(a, y, ref, what=str(shape))
    h.close()


# --- the persistent batched-decode kernel (2 <= M <= 32, g = 128, d a multiple of 512):
# one and two m-tiles, ragged last v-blocks and wave ranges, missing terms ----------

BATCHED_SHAPES = [
    # V,     d,    k,   r,   g,  M
    (1, 512, 1, 1, 128, 2),
    (33, 512, 8, 4, 128, 3),
    (4099, 512, 40, 20, 128, 7),
    (2050, 1536, 96, 33, 128, 16),
    (2050, 1536, 96, 33, 128, 17),
    (9001, 1024, 64, 16, 128, 31),
    (6000, 2560, 192, 48, 128, 32),
    (777, 512, 0, 16, 128, 12),    # no core term
    (777, 1024, 40, 0, 128, 20),   # no correction term
    (500, 512, 0, 0, 128, 25),     # residual only
    (40000, 512, 16, 8, 128, 9),   # several v-blocks per wave
]


@pytest.mark.parametrize("shape", BATCHED_SHAPES, ids=lambda s: "V{}_d{}_k{}_r{}_g{}_M{}".format(*s))
def test_batched_decode_shapes(shape):
    V, d, k, r, g, M = shape
    say(f"batched decode {shape}")
    f = random_small_head(V, d, k, r, g, M, seed=V * 11 + d + M, n_outliers=2, outlier_factor=20.0)
    h = load(f)
    ref = oracle_forward.forward(f, f["X"])
    y, a = gpu_forward(h, f["X"], path="skinny")
    assert_logits_close(y, ref, what=str(shape))
    assert_argmax_ok(a, y, ref, what=str(shape))
    # argmax alone and logits alone give the same results
    _, a2 = gpu_forward(h, f["X"], path="skinny", want_logits=False)
    y3, _ = gpu_forward(h, f["X"], path="skinny", want_argmax=False)
    assert np.array_equal(a, a2)
    assert np.array_equal(y, y3)
    h.close()


# --- several m-tiles and v-ranges of the large-M kernel, ragged in both -------------

LDS_SHAPES = [
    # V,     d,   k,  r,   g,   M
    (1500, 512, 64, 16, 128, 300),
    (600, 256, 16, 4, 32, 257),
    (1100, 384, 33, 7, 96, 129),
    (520, 640, 0, 20, 128, 200),
]


@pytest.mark.parametrize("shape", LDS_SHAPES, ids=lambda s: "V{}_d{}_k{}_r{}_g{}_M{}".format(*s))
@pytest.mark.parametrize("path", PATHS)
def test_multi_tile_shapes(shape, path):
    V, d, k, r, g, M = shape
    say(f"multi-tile {shape} path={path}")
    f = random_small_head(V, d, k, r, g, M, seed=V + d * 3 + M, n_outliers=3, outlier_factor=30.0)
    h = load(f)
    ref = oracle_forward.forward(f, f["X"])
    y, a = gpu_forward(h, f["X"], path=path)
    assert_logits_close(y, ref, what=str(shape))
    assert_argmax_ok(a, y, ref, what=str(shape))
    h.close()


# --- residual group scales spread over a wide range -----------------------------------

@pytest.mark.parametrize("path", PATHS)
def test_wide_residual_scale_spread(path):
    """Residual group scales of each row spread over 2^-12 .. 1 times 1e-2,
    with some groups zero.  On the large-M path the residual operand
    q sR 2^(e_r - 10) then runs from normal fp16 deep into the subnormal
    range, where its absolute error stays at most 2^-25; the logits must
    still meet the tolerance (ARCHead paper, eq 7 with the residual of eq 3)."""
    V, d, k, r, g, M = 700, 512, 32, 8, 32, 150
    say(f"wide residual scale spread path={path}")
    f = random_small_head(V, d, k, r, g, M, seed=4242, n_outliers=2, outlier_factor=20.0)
    rng = np.random.default_rng(4243)
    G = d // g
    sr = 1e-2 * np.exp2(-rng.uniform(0.0, 12.0, size=(V, G)))
    sr[rng.random((V, G)) < 0.05] = 0.0
    f["sR"] = to_f16_bits(sr)
    h = load(f)
    ref = oracle_forward.forward(f, f["X"])
    y, a = gpu_forward(h, f["X"], path=path)
    assert_logits_close(y, ref, what=f"wide sR spread, {path}")
    assert_argmax_ok(a, y, ref, what=f"wide sR spread, {path}")
    h.close()


# --- degenerate rows, a zero hidden state and extreme codes -----------------------------

@pytest.mark.parametrize("path,M", [("gemv", 1), ("gemv", 2), ("skinny", 1), ("skinny", 20), ("skinny", 40),
                                    ("lds", 130)])
def test_zero_scales_zero_state_and_extreme_codes(path, M):
    """Rows whose sA or sC is zero (the large-M path masks their codes and
    keeps a unit divisor), rows with every scale zero (logits exactly zero,
    a block of equal maxima for the lowest-index rule), rows at the extreme
    codes (A5 = -16, R4 = -8, C8 = -128), and a hidden state of zeros (its
    logits are exactly zero): ARCHead paper, eq 7 with eq 3."""
    V, d, k, r, g = 1000, 512, 40, 12, 128
    say(f"degenerate rows path={path} M={M}")
    f = random_small_head(V, d, k, r, g, M, seed=515 + M, n_outliers=2, outlier_factor=20.0)
    sa = f["sA"].copy()
    sc = f["sC"].copy()
    sr = f["sR"].copy()
    sa[::7] = 0
    sc[::5] = 0
    sa[100:116] = 0
    sc[100:116] = 0
    sr[100:116] = 0
    f["sA"], f["sC"], f["sR"] = sa, sc, sr
    f["A5"][200:216] = -16
    f["R4"][200:216] = 0x88
    f["C8"][200:216] = -128
    if M > 1: # (at M = 1 the one hidden state stays random)
        X = f["X"].copy()
        X[0] = 0
        f["X"] = X
    h = load(f)
    ref = oracle_forward.forward(f, f["X"])
    y, a = gpu_forward(h, f["X"], path=path)
    if M > 1:
        assert np.all(y[0] == 0.0), "a zero hidden state gives exactly zero logits"
        assert a[0] == 0, "all-equal logits resolve to the lowest index"
    assert np.all(y[:, 100:116] == 0.0), "rows with every scale zero give exactly zero logits"
    assert_logits_close(y, ref, what=f"degenerate rows, {path}, M={M}")
    assert_argmax_ok(a, y, ref, what=f"degenerate rows, {path}, M={M}")
    h.close()


# --- integer fields read back exactly through the kernels ------------------------------

def _onehot(d, cols):
    x = np.zeros((len(cols), d))
    x[np.arange(len(cols)), cols] = 1.0
    return to_bf16_bits(x)


@pytest.mark.parametrize("path", PATHS)
def test_one_hot_probes_are_bit_exact(path):
    say(f"one-hot probes path={path}")
    rng = np.random.default_rng(3)
    V, d, k, r, g = 200, 256, 40, 12, 64
    G = d // g
    one, zero = to_f16_bits(1.0), to_f16_bits(0.0)
    base = {"V": V, "d": d, "k": k, "r": r, "g": g,
            "A5": np.zeros((V, k), np.int8), "sA": np.full(V, zero, np.uint16),
            "B8": np.zeros((k, d), np.int8), "sB": np.full(k, one, np.uint16),
            "R4": np.zeros((V, d // 2), np.uint8), "sR": np.full((V, G), zero, np.uint16),
            "C8": np.zeros((V, r), np.int8), "sC": np.full(V, zero, np.uint16),
            "D8": np.zeros((r, d), np.int8), "sD": np.full((r, G), one, np.uint16)}
    cols = [0, 1, 31, 32, 100, 255]
    X = _onehot(d, cols)
    # R4: logits[m, v] = R4[v, col_m]
    r4 = rng.integers(-8, 8, size=(V, d))
    nib = (r4 & 0xF).astype(np.uint8)
    f = dict(base, R4=(nib[:, 0::2] | (nib[:, 1::2] << 4)), sR=np.full((V, G), one, np.uint16))
    h = load(f)
    y, _ = gpu_forward(h, X, path=path, want_argmax=False)
    h.close()
    assert np.array_equal(y, r4[:, cols].T.astype(np.float32))
    # A5 through B8 = [I | 0]
    a5 = rng.integers(-16, 16, size=(V, k)).astype(np.int8)
    eye = np.zeros((k, d), np.int8)
    eye[np.arange(k), np.arange(k)] = 1
    h = load(dict(base, A5=a5, B8=eye, sA=np.full(V, one, np.uint16)))
    kc = [0, 1, 17, 39]
    y, _ = gpu_forward(h, _onehot(d, kc), path=path, want_argmax=False)
    h.close()
    assert np.array_equal(y, a5[:, kc].T.astype(np.float32))
    # B8 through A5 = delta
    b8 = rng.integers(-128, 128, size=(k, d)).astype(np.int8)
    a5d = np.zeros((V, k), np.int8)
    a5d[np.arange(k), np.arange(k)] = 1
    h = load(dict(base, A5=a5d, B8=b8, sA=np.full(V, one, np.uint16)))
    y, _ = gpu_forward(h, X, path=path, want_argmax=False)
    h.close()
    assert np.array_equal(y[:, :k], b8[:, cols].T.astype(np.float32))
    assert np.all(y[:, k:] == 0)
    # C8 through D8 = [I | 0]
    c8 = rng.integers(-128, 128, size=(V, r)).astype(np.int8)
    eye = np.zeros((r, d), np.int8)
    eye[np.arange(r), np.arange(r)] = 1
    h = load(dict(base, C8=c8, D8=eye, sC=np.full(V, one, np.uint16)))
    rc = [0, 5, 11]
    y, _ = gpu_forward(h, _onehot(d, rc), path=path, want_argmax=False)
    h.close()
    assert np.array_equal(y, c8[:, rc].T.astype(np.float32))
    # D8 through C8 = delta
    d8 = rng.integers(-128, 128, size=(r, d)).astype(np.int8)
    c8d = np.zeros((V, r), np.int8)
    c8d[np.arange(r), np.arange(r)] = 1
    h = load(dict(base, C8=c8d, D8=d8, sC=np.full(V, one, np.uint16)))
    y, _ = gpu_forward(h, X, path=path, want_argmax=False)
    h.close()
    assert np.array_equal(y[:, :r], d8[:, cols].T.astype(np.float32))


# --- determinism, argmax-only, M = 0, workspace growth -------------------------------

def test_repeat_is_bitwise_identical_and_argmax_only_matches():
    say("determinism")
    f = random_small_head(3000, 512, 64, 16, 128, 9, seed=12)
    h = load(f)
    y1, a1 = gpu_forward(h, f["X"])
    y2, a2 = gpu_forward(h, f["X"])
    _, a3 = gpu_forward(h, f["X"], want_logits=False)
    h.close()
    assert np.array_equal(y1, y2)
    assert np.array_equal(a1, a2) and np.array_equal(a1, a3)
    assert np.array_equal(a1, np.argmax(y1, axis=1))


def test_argmax_ties_resolve_to_the_lowest_index():
    say("argmax ties")
    V, d = 100, 128
    f = random_small_head(V, d, 8, 4, 32, 2, seed=5)
    # rows 10, 40, 77 identical -> identical logits
    for name in ["A5", "R4", "C8", "sA", "sR", "sC"]:
        f[name][40] = f[name][10]
        f[name][77] = f[name][10]
    h = load(f)
    ref = oracle_forward.forward(f, f["X"])
    y, a = gpu_forward(h, f["X"])
    h.close()
    assert y[0, 10] == y[0, 40] == y[0, 77]
    assert np.array_equal(a, np.argmax(y, axis=1))
    assert_logits_close(y, ref)


def test_zero_rows_and_workspace_growth():
    import torch
    from packed_quantized_lm_amd import x_tensor_from_bits
    say("M=0 and workspace growth")
    f = random_small_head(500, 256, 16, 8, 64, 70, seed=8)
    h = load(f)
    X = x_tensor_from_bits(f["X"])
    logits = torch.empty((0, 500), dtype=torch.float32, device="cuda")
    h.forward_into(X[:0], logits, None)
    ref = oracle_forward.forward(f, f["X"])
    for M in (1, 70, 3, 40):
        y, a = gpu_forward(h, f["X"][:M])
        assert_logits_close(y, ref[:M], what=f"M={M}")
        assert_argmax_ok(a, y, ref[:M])
    h.reserve(100)
    y, _ = gpu_forward(h, f["X"][:5])
    assert_logits_close(y, ref[:5])
    assert h.packed_bytes() > 0 and h.device_bytes() >= h.packed_bytes()
    h.close()


def test_packed_bytes_match_eq10():
    from oracle.layout import packed_bytes
    f = random_small_head(1001, 384, 33, 7, 96, 1, seed=1)
    h = load(f)
    assert h.packed_bytes() == packed_bytes(1001, 384, 33, 7, 96)
    h.close()


# --- full-size workloads ------------------------------------------------------------

_HEADS = {}


def _head(name):
    if name not in _HEADS:
        _HEADS.clear()
        c = make_config(name)
        _HEADS[name] = (c, load(c))
    return _HEADS[name]


def _sample_rows(V, n, seed):
    rng = np.random.default_rng(seed)
    rows = np.concatenate([np.arange(0, 64), np.arange(V - 64, V),
                           rng.choice(np.arange(64, V - 64), size=n, replace=False)])
    return np.unique(rows)


@pytest.mark.parametrize("name", ["qwen_m1", "qwen_m32", "large_m8"])
def test_full_size_workload_full_oracle(name):
    say(f"full size {name}: generating + loading")
    c, h = _head(name)
    say(f"full size {name}: GPU forward M={c['M']}")
    y, a = gpu_forward(h, c["X"])
    say(f"full size {name}: oracle")
    ref = oracle_forward.forward(c, c["X"])
    ratio = assert_logits_close(y, ref, what=name)
    assert_argmax_ok(a, y, ref, what=name)
    say(f"full size {name}: worst |d|/(2e-3 rms) = {ratio:.3g}")


def test_prefill_workload_sampled():
    name = "qwen_m2048"
    say(f"full size {name}: generating + loading")
    c, h = _head(name)
    say(f"full size {name}: GPU forward M={c['M']}")
    y, a = gpu_forward(h, c["X"])
    rows = _sample_rows(c["V"], 2048, seed=1)
    say(f"full size {name}: oracle on {rows.size} sampled rows")
    ref = oracle_forward.forward(c, c["X"], rows=rows)
    rms = row_rms(ref)
    ratio = assert_logits_close(y[:, rows], ref, rms=rms, what=name)
    # properties at full size: argmax is the first argmax of the GPU logits, and
    # the GPU's top-1 row is at least as large (within tolerance) as every sampled row
    assert np.array_equal(a, np.argmax(y, axis=1))
    top = oracle_forward.forward(c, c["X"][:64], rows=np.unique(a[:64]))
    idx = {v: i for i, v in enumerate(np.unique(a[:64]))}
    for m in range(64):
        v = a[m]
        assert top[m, idx[v]] >= ref[m].max() - TOL * rms[m]
    say(f"full size {name}: worst sampled |d|/(2e-3 rms) = {ratio:.3g}")


# --- HIP graph capture of a step -------------------------------------------------------

@pytest.mark.parametrize("path", ["skinny", "lds"])
def test_graph_replays_match_eager(path):
    import torch
    from packed_quantized_lm_amd import x_tensor_from_bits
    say(f"graph replay path={path}")
    f = random_small_head(1500, 512, 64, 16, 128, 40, seed=77)
    h = load(f)
    X = x_tensor_from_bits(f["X"])
    logits = torch.empty((40, 1500), dtype=torch.float32, device="cuda")
    arg = torch.empty((40,), dtype=torch.int32, device="cuda")
    h.forward_into(X, logits, arg, path=path)
    torch.cuda.synchronize()
    y0, a0 = logits.clone(), arg.clone()
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        h.forward_into(X, logits, arg, path=path)
    for rep in range(4):
        logits.fill_(float("nan"))
        arg.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(logits, y0), f"replay {rep}: logits differ"
        assert torch.equal(arg, a0), f"replay {rep}: argmax differs"
        h.forward_into(X, logits, arg, path=path)  # eager work between replays
        torch.cuda.synchronize()
    del g
    h.close()


def test_argmax_partials_fit_for_every_plan():
    """The decode plan at M = 1 writes fewer argmax partials per row than the
    plan at M = 30; a workspace sized for M = 30 must hold the larger count."""
    say("argmax partials sizing")
    f = random_small_head(5000, 512, 32, 16, 128, 30, seed=21)
    h = load(f)
    h.reserve(30)
    ref = oracle_forward.forward(f, f["X"])
    for M in (30, 1, 17):
        y, a = gpu_forward(h, f["X"][:M])
        assert_logits_close(y, ref[:M], what=f"M={M}")
        assert_argmax_ok(a, y, ref[:M], what=f"M={M}")
    h.close()

"""GPU parity of the fused log-normaliser / cross-entropy (archead_forward_ce)
against the CPU oracle (oracle/softmax.py over oracle/forward.py logits).

Tolerances follow from the logits' acceptance bound |dy| <= 2e-3 rms(row):
lse is 1-Lipschitz in the max norm, so |d lse| <= 2e-3 rms; nll = lse - y_t
adds the target logit's own error, so |d nll| <= 4e-3 rms.  Separately, lse
and nll must match the fp64 log-normaliser of the GPU's own logits to fp32
rounding of the exponentials and sums (EPS_ABS + EPS_REL |lse|), which
isolates the epilogue from the logits' rounding.
"""
import numpy as np
import pytest

from gpu_util import TOL, assert_logits_close, row_rms, say
from oracle import forward as oracle_forward
from oracle import softmax as oracle_softmax
from packed_quantized_lm_amd.synth import make_config, random_small_head

pytestmark = pytest.mark.gpu

EPS_ABS, EPS_REL = 2e-5, 2e-6


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


def gpu_ce(head, X_bits, targets, path="auto", want_logits=True, want_argmax=True):
    import torch
    from packed_quantized_lm_amd import x_tensor_from_bits
    X = x_tensor_from_bits(X_bits)
    t = None if targets is None else torch.from_numpy(np.asarray(targets, dtype=np.int32)).cuda()
    lse, nll, logits, arg = head.forward_ce(X, t, want_logits=want_logits, want_argmax=want_argmax, path=path)
    torch.cuda.synchronize()
    cpu = lambda x: None if x is None else x.cpu().numpy()
    return cpu(lse), cpu(nll), cpu(logits), cpu(arg)


def check_self_consistent(lse, nll, logits, targets, what):
    """lse / nll against the fp64 log-normaliser of the GPU's own logits."""
    ref = oracle_softmax.log_sum_exp(logits)
    err = np.abs(lse.astype(np.float64) - ref)
    bound = EPS_ABS + EPS_REL * np.abs(ref)
    assert np.all(err <= bound), f"{what}: lse vs own logits, worst {np.max(err / bound):.3g} x bound"
    if nll is not None:
        ref_nll = oracle_softmax.cross_entropy(logits, targets)
        ok = np.isfinite(ref_nll)
        assert np.array_equal(np.isnan(nll), ~ok), f"{what}: NaN pattern of nll"
        e2 = np.abs(nll[ok].astype(np.float64) - ref_nll[ok])
        assert np.all(e2 <= bound[ok]), f"{what}: nll vs own logits, worst {np.max(e2 / bound[ok]):.3g} x bound"


def check_oracle(lse, nll, ref_logits, targets, what, rms=None):
    rms = row_rms(ref_logits) if rms is None else rms
    ref = oracle_softmax.log_sum_exp(ref_logits)
    r1 = np.abs(lse - ref) / (TOL * rms)
    assert np.all(r1 <= 1.0), f"{what}: |d lse| / (2e-3 rms) = {r1.max():.3g}"
    if nll is not None:
        ref_nll = oracle_softmax.cross_entropy(ref_logits, targets)
        ok = np.isfinite(ref_nll)
        r2 = np.abs(nll[ok] - ref_nll[ok]) / (2 * TOL * rms[ok])
        assert np.all(r2 <= 1.0), f"{what}: |d nll| / (4e-3 rms) = {r2.max():.3g}"
        return max(float(r1.max()), float(r2.max(initial=0)))
    return float(r1.max())


# --- small shapes on every path -------------------------------------------------

CASES = [
    # path,    V,    d,   k,  r,   g,  M
    ("gemv", 1, 512, 8, 4, 128, 1),
    ("gemv", 1000, 1024, 33, 7, 128, 2),
    ("gemv", 4099, 1536, 64, 48, 128, 1),
    ("skinny", 15, 128, 8, 4, 32, 2),
    ("skinny", 2500, 512, 64, 16, 128, 1),   # single launch (matrix-core decode)
    ("skinny", 1000, 384, 33, 7, 96, 17),
    ("skinny", 4099, 640, 64, 48, 128, 33),
    ("skinny", 777, 512, 0, 16, 256, 8),      # no core term
    ("skinny", 3001, 1024, 40, 20, 128, 9),   # persistent batched-decode kernel, one m-tile
    ("skinny", 2050, 1536, 96, 33, 128, 32),  # the same, two m-tiles
    ("lds", 17, 256, 16, 4, 64, 3),
    ("lds", 1500, 512, 64, 16, 128, 130),     # several tiles, ragged tails in V and M
    ("lds", 600, 256, 16, 4, 32, 257),
    ("lds", 777, 512, 40, 0, 512, 129),       # no correction term
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "{}-V{}_d{}_k{}_r{}_g{}_M{}".format(*c))
def test_ce_matches_oracle(case):
    path, V, d, k, r, g, M = case
    say(f"ce {case}")
    f = random_small_head(V, d, k, r, g, M, seed=V + 3 * d + M, n_outliers=2, outlier_factor=20.0)
    rng = np.random.default_rng(V * 31 + M)
    targets = rng.integers(0, V, M).astype(np.int32)
    h = load(f)
    lse, nll, y, a = gpu_ce(h, f["X"], targets, path=path)
    ref = oracle_forward.forward(f, f["X"])
    assert_logits_close(y, ref, what=str(case))
    assert np.array_equal(a, np.argmax(y, axis=1))
    check_self_consistent(lse, nll, y, targets, str(case))
    worst = check_oracle(lse, nll, ref, targets, str(case))
    # the log-normaliser bounds: max y <= lse <= max y + ln V
    assert np.all(lse >= y.max(axis=1)) and np.all(lse <= y.max(axis=1) + np.log(V) + 1e-5)
    # without logits, argmax or targets the summaries are the same (bitwise)
    lse2, nll2, _, _ = gpu_ce(h, f["X"], targets, path=path, want_logits=False, want_argmax=False)
    lse3, nll3, _, _ = gpu_ce(h, f["X"], None, path=path, want_logits=False, want_argmax=True)
    assert np.array_equal(lse2, lse) and np.array_equal(nll2, nll) and np.array_equal(lse3, lse)
    assert nll3 is None
    say(f"ce {case}: worst |d|/bound vs oracle = {worst:.3g}")
    h.close()


@pytest.mark.parametrize("path,M", [("gemv", 2), ("skinny", 1), ("skinny", 20), ("lds", 130)])
def test_ce_targets_at_the_edges(path, M):
    """Targets at rows 0 and V-1, at the argmax (nll = lse - max), and outside
    [0, V) (NaN, not an error)."""
    V = 1000
    say(f"ce edges path={path} M={M}")
    f = random_small_head(V, 512, 32, 8, 128, M, seed=91 + M)
    h = load(f)
    _, _, y, a = gpu_ce(h, f["X"], None, path=path)
    t = np.empty(M, dtype=np.int32)
    pattern = [0, V - 1, -1, V, int(np.iinfo(np.int32).min), int(np.iinfo(np.int32).max)]
    for m in range(M):
        t[m] = a[m] if m % 7 == 6 else pattern[m % len(pattern)]
    lse, nll, y2, _ = gpu_ce(h, f["X"], t, path=path)
    assert np.array_equal(y2, y)
    bad = (t < 0) | (t >= V)
    assert np.isnan(nll[bad]).all() and np.isfinite(nll[~bad]).all()
    check_self_consistent(lse, nll, y, t, f"edges {path}")
    top = np.arange(M) % 7 == 6
    assert np.allclose(nll[top], lse[top] - y.max(axis=1)[top], rtol=0, atol=1e-5)
    h.close()


def test_ce_degenerate_rows():
    """All-zero hidden states (every logit 0: lse = ln V, nll = ln V) and a head
    whose scales are all zero, on every path."""
    V, d = 2000, 512
    for path, M in [("gemv", 1), ("skinny", 5), ("lds", 130)]:
        say(f"ce degenerate path={path} M={M}")
        f = random_small_head(V, d, 32, 8, 128, M, seed=5)
        f["X"][:] = 0
        h = load(f)
        t = (np.arange(M) * 37 % V).astype(np.int32)
        lse, nll, y, _ = gpu_ce(h, f["X"], t, path=path)
        assert np.array_equal(y, np.zeros_like(y))
        assert np.allclose(lse, np.log(V), rtol=0, atol=1e-5)
        assert np.allclose(nll, np.log(V), rtol=0, atol=1e-5)
        h.close()


def test_ce_graph_replays_match_eager():
    import torch
    from packed_quantized_lm_amd import x_tensor_from_bits
    say("ce graph replay")
    M, V = 40, 1500
    f = random_small_head(V, 512, 64, 16, 128, M, seed=78)
    h = load(f)
    X = x_tensor_from_bits(f["X"])
    t = torch.from_numpy(np.arange(M, dtype=np.int32) * 13 % V).cuda()
    lse = torch.empty((M,), dtype=torch.float32, device="cuda")
    nll = torch.empty_like(lse)
    h.forward_ce_into(X, t, None, None, lse, nll)
    torch.cuda.synchronize()
    l0, n0 = lse.clone(), nll.clone()
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        h.forward_ce_into(X, t, None, None, lse, nll)
    for rep in range(3):
        lse.fill_(float("nan"))
        nll.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(lse, l0) and torch.equal(nll, n0), f"replay {rep}"
    h.close()


# --- full-size workloads ----------------------------------------------------------

@pytest.mark.parametrize("name", ["qwen_m1", "qwen_m32", "large_m8", "qwen_m2048"])
def test_ce_full_size(name):
    say(f"ce full size {name}: generating + loading")
    c = make_config(name)
    h = load(c)
    M, V = c["M"], c["V"]
    targets = np.random.default_rng(17).integers(0, V, M).astype(np.int32)
    say(f"ce full size {name}: GPU forward_ce M={M}")
    lse, nll, y, a = gpu_ce(h, c["X"], targets)
    assert np.array_equal(a, np.argmax(y, axis=1))
    for m0 in range(0, M, 256):  # bounded host memory at M = 2048
        sl = slice(m0, min(M, m0 + 256))
        check_self_consistent(lse[sl], nll[sl], y[sl], targets[sl], f"{name} rows {m0}..")
    # against the oracle: every row up to M = 32, four rows of the prefill
    rows = np.arange(M) if M <= 32 else np.array([0, 1, M // 2, M - 1])
    say(f"ce full size {name}: oracle over the full vocabulary for {rows.size} hidden states")
    ref = oracle_forward.forward(c, c["X"][rows])
    worst = check_oracle(lse[rows], nll[rows], ref, targets[rows], name)
    say(f"ce full size {name}: worst |d|/bound vs oracle = {worst:.3g}")
    h.close()

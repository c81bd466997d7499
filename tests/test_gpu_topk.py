"""GPU parity of the top-k selection (archead_forward_topk) against the CPU
oracle.  The selection is exact on the logits it reads, so the GPU's indices
and values must equal oracle/select.py applied to the GPU's own logits,
bit for bit.  Against the oracle's fp64 logits the chosen rows must be the
oracle's top K up to near-ties: every chosen row's oracle logit is within the
logits' tolerance (2e-3 rms) of the oracle's K-th largest, and every row the
oracle ranks above its K-th largest by more than that is chosen."""
import numpy as np
import pytest

from gpu_util import TOL, assert_logits_close, row_rms, say
from oracle import forward as oracle_forward
from oracle.select import top_k
from packed_quantized_lm_amd.synth import make_config, random_small_head

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


def gpu_topk(head, X_bits, K, path="auto"):
    import torch
    from packed_quantized_lm_amd import x_tensor_from_bits
    v, i, y = head.forward_topk(x_tensor_from_bits(X_bits), K, path=path)
    torch.cuda.synchronize()
    return v.cpu().numpy(), i.cpu().numpy().astype(np.int64), y.cpu().numpy()


def check_exact(v, i, y, K, what):
    rv, ri = top_k(y, K)
    assert np.array_equal(i, ri), f"{what}: indices differ from the top-k of the GPU's own logits"
    assert np.array_equal(v, rv), f"{what}: values differ"


def check_oracle(i, ref, K, what, rms=None):
    rms = row_rms(ref) if rms is None else rms
    kth = np.sort(ref, axis=1)[:, -K]
    for m in range(ref.shape[0]):
        chosen = set(i[m].tolist())
        assert np.all(ref[m, i[m]] >= kth[m] - TOL * rms[m]), f"{what}: row {m} chose a row far below the K-th"
        must = np.nonzero(ref[m] > kth[m] + TOL * rms[m])[0]
        assert set(must.tolist()) <= chosen, f"{what}: row {m} missed a clear top-{K} row"


CASES = [
    # path,     V,    d,   k,  r,   g,  M,  K
    ("gemv", 1000, 512, 16, 4, 128, 1, 16),
    ("gemv", 3000, 1024, 33, 7, 128, 2, 5),
    ("skinny", 2500, 512, 64, 16, 128, 1, 8),    # single launch (matrix cores)
    ("skinny", 1025, 384, 33, 7, 96, 17, 16),    # one logit in the last slice
    ("skinny", 17, 256, 16, 4, 64, 3, 16),       # V barely above K
    ("lds", 1500, 512, 64, 16, 128, 130, 16),
    ("lds", 5000, 256, 16, 4, 32, 129, 1),
    ("skinny", 300000, 128, 1, 1, 32, 2, 16),   # merge over more keys than registers hold (LDS)
    ("skinny", 400000, 128, 1, 1, 32, 1, 16),   # ... and than LDS holds (read each round)
    # selection inside the single launch (M <= 2, d a multiple of 512): one
    # workgroup, a few, and more waves than the selecting workgroup has
    # threads (5, 6 and 9 wave keys per thread at V = 90000 and 140000)
    ("gemv", 20, 512, 8, 4, 128, 1, 16),
    ("gemv", 20, 512, 8, 4, 128, 2, 16),
    ("skinny", 1, 512, 1, 1, 128, 1, 1),
    ("skinny", 6001, 1024, 40, 20, 128, 1, 16),
    ("gemv", 6001, 1024, 40, 20, 128, 2, 3),
    ("skinny", 90000, 512, 16, 8, 128, 1, 16),
    ("gemv", 90000, 512, 16, 8, 128, 2, 16),
    ("gemv", 90000, 512, 16, 8, 32, 1, 11),
    ("gemv", 140000, 512, 16, 8, 128, 2, 16),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "{}-V{}_d{}_k{}_r{}_g{}_M{}_K{}".format(*c))
def test_topk_matches_oracle(case):
    path, V, d, k, r, g, M, K = case
    say(f"topk {case}")
    f = random_small_head(V, d, k, r, g, M, seed=V + d + 5 * M, n_outliers=2, outlier_factor=20.0)
    h = load(f)
    v, i, y = gpu_topk(h, f["X"], K, path=path)
    ref = oracle_forward.forward(f, f["X"])
    assert_logits_close(y, ref, what=str(case))
    check_exact(v, i, y, K, str(case))
    check_oracle(i, ref, K, str(case))
    h.close()


def test_topk_ties_resolve_to_lower_indices():
    # all-zero hidden states: every logit is 0 and the top K are rows 0 .. K-1
    # (inside the single launch: more than 256 candidate rows reach the
    # K-th largest wave key)
    for path, M, V in [("gemv", 1, 3000), ("gemv", 2, 3000), ("skinny", 1, 3000), ("skinny", 5, 3000),
                       ("lds", 130, 3000), ("gemv", 1, 90000), ("gemv", 2, 140000)]:
        say(f"topk ties path={path} M={M} V={V}")
        f = random_small_head(V, 512, 32, 8, 128, M, seed=4)
        f["X"][:] = 0
        h = load(f)
        v, i, y = gpu_topk(h, f["X"], 16, path=path)
        assert np.array_equal(i, np.tile(np.arange(16), (M, 1))) and not v.any()
        h.close()


def test_topk_first_entry_is_the_argmax_and_bad_k_is_rejected():
    import torch
    from packed_quantized_lm_amd import x_tensor_from_bits
    from packed_quantized_lm_amd.binding import ArcheadError
    f = random_small_head(1500, 512, 32, 8, 128, 40, seed=6)
    h = load(f)
    _, i, y = gpu_topk(h, f["X"], 1)
    y2, a = h.forward(x_tensor_from_bits(f["X"]), want_logits=True, want_argmax=True)
    torch.cuda.synchronize()
    assert np.array_equal(i[:, 0], a.cpu().numpy())
    for K in (0, 17):
        with pytest.raises(ArcheadError):
            h.forward_topk(x_tensor_from_bits(f["X"]), K)
    h.close()
    small = random_small_head(5, 128, 1, 1, 32, 1, seed=7)
    hs = load(small)
    with pytest.raises(ArcheadError):
        hs.forward_topk(x_tensor_from_bits(small["X"]), 6)  # K > V
    v, i, y = gpu_topk(hs, small["X"], 5)
    check_exact(v, i, y, 5, "V = K = 5")
    hs.close()


@pytest.mark.parametrize("name", ["qwen_m1", "qwen_m32", "large_m8", "qwen_m2048"])
def test_topk_full_size(name):
    say(f"topk full size {name}")
    c = make_config(name)
    h = load(c)
    v, i, y = gpu_topk(h, c["X"], 16)
    for m0 in range(0, c["M"], 256):
        sl = slice(m0, m0 + 256)
        check_exact(v[sl], i[sl], y[sl], 16, f"{name} rows {m0}..")
    rows = np.arange(c["M"]) if c["M"] <= 32 else np.array([0, 1, c["M"] // 2, c["M"] - 1])
    say(f"topk full size {name}: oracle for {rows.size} hidden states")
    ref = oracle_forward.forward(c, c["X"][rows])
    check_oracle(i[rows], ref, 16, name)
    h.close()


def check_draw(s, v, i, u, tau, what):
    """The draw against oracle/select.py's over the GPU's own top-k (exact
    inputs): equal, except where u lands within float rounding of a
    cumulative boundary (the kernel sums in fp32)."""
    from oracle.select import sample_top_k
    ref = sample_top_k(v, i, tau, u)
    w = np.exp((v.astype(np.float64) - v[:, :1]) / tau)
    c = np.cumsum(w, axis=1)
    t = u * c[:, -1]
    for m in range(s.shape[0]):
        if s[m] != ref[m]:
            near = np.min(np.abs(c[m] - t[m])) <= 1e-5 * c[m, -1]
            assert near, f"{what}: row {m}: drew {s[m]}, oracle {ref[m]}"


# forward_sample takes the automatic path: M = 1 runs the single launch, M = 40
# the streaming kernel, M = 130 the large-M kernel
@pytest.mark.parametrize("M", [1, 40, 130])
@pytest.mark.parametrize("tau", [0.7, 5.0, 1e-4])
def test_topk_sampling_matches_oracle(M, tau):
    """archead_forward_sample against the oracle's draw; at tau -> 0 the draw
    is the argmax; u = 0 always gives it."""
    import torch
    from packed_quantized_lm_amd import x_tensor_from_bits
    K = 16
    say(f"topk sampling M={M} tau={tau}")
    f = random_small_head(3000, 512, 32, 8, 128, M, seed=21 + M)
    h = load(f)
    X = x_tensor_from_bits(f["X"])
    u = np.random.default_rng(M).random(M, dtype=np.float32)
    u[0] = 0.0
    s, v, i, y = h.forward_sample(X, K, tau, torch.from_numpy(u).cuda())
    torch.cuda.synchronize()
    s, v, i = s.cpu().numpy(), v.cpu().numpy(), i.cpu().numpy()
    check_exact(v, i.astype(np.int64), y.cpu().numpy(), K, "sampling top-k")
    check_draw(s, v, i, u, tau, "sampling")
    assert s[0] == i[0, 0]
    if tau == 1e-4:
        assert np.array_equal(s, i[:, 0])
    h.close()


@pytest.mark.parametrize("name", ["qwen_m1", "large_m8"])
def test_topk_sampling_full_size(name):
    """The draw at full size: the GPU's top-16 exact on its own logits and
    within tolerance of the oracle's, the draw equal to the oracle's draw over
    that top-16 (boundary rounding aside), at two temperatures."""
    import torch
    from packed_quantized_lm_amd import x_tensor_from_bits
    say(f"topk sampling full size {name}")
    c = make_config(name)
    h = load(c)
    X = x_tensor_from_bits(c["X"])
    M = c["M"]
    ref = oracle_forward.forward(c, c["X"])
    for tau in (1.0, 0.3):
        u = np.random.default_rng(int(100 * tau) + M).random(M, dtype=np.float32)
        s, v, i, y = h.forward_sample(X, 16, tau, torch.from_numpy(u).cuda())
        torch.cuda.synchronize()
        s, v, i, y = s.cpu().numpy(), v.cpu().numpy(), i.cpu().numpy(), y.cpu().numpy()
        check_exact(v, i.astype(np.int64), y, 16, f"{name} tau={tau}")
        check_oracle(i.astype(np.int64), ref, 16, f"{name} tau={tau}")
        check_draw(s, v, i, u, tau, f"{name} tau={tau}")
    h.close()

"""The prefill workload (151936 x 4096 head, k = 256, r = 64, g = 128, M = 2048)
against the fp64 oracle over the FULL vocabulary, for one hidden state in
every 128-row m-tile of the large-M kernel (at a different offset inside each
tile) plus the first and the last hidden state.

On those rows every logit is held to 2e-3 x the row's RMS, the argmax to the
oracle's except at near-ties, lse and nll to the bounds derived from the
logits' (|d lse| <= 2e-3 rms, |d nll| <= 4e-3 rms), and the top-16 to the
oracle's top-16 up to near-ties.  On every row the outputs are also checked
against the GPU's own logits (argmax bit-exact, top-16 exact, lse and nll to
fp32 rounding of the epilogue).
"""
import numpy as np
import pytest

from gpu_util import TOL, assert_argmax_ok, assert_logits_close, row_rms, say
from oracle import forward as oracle_forward
from oracle import softmax as oracle_softmax
from oracle.select import top_k
from packed_quantized_lm_amd.synth import make_config

pytestmark = pytest.mark.gpu

K = 16
EPS_ABS, EPS_REL = 2e-5, 2e-6


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from packed_quantized_lm_amd import load_library
    load_library()


def sample_rows(M, tile=128):
    """One row per m-tile at offset (37 t) mod 128 inside tile t, plus 0 and M - 1."""
    rows = {0, M - 1}
    for t in range((M + tile - 1) // tile):
        rows.add(min(M - 1, t * tile + (37 * t) % tile))
    return np.array(sorted(rows))


def test_prefill_full_vocabulary_rows():
    import torch
    from packed_quantized_lm_amd import PackedHead, x_tensor_from_bits
    say("prefill full-vocabulary oracle rows: generating + loading qwen_m2048")
    c = make_config("qwen_m2048")
    M, V = c["M"], c["V"]
    h = PackedHead(c)
    X = x_tensor_from_bits(c["X"])
    targets = np.random.default_rng(23).integers(0, V, M).astype(np.int32)
    say(f"prefill: GPU forward_ce + forward_topk M={M}")
    lse, nll, y, a = h.forward_ce(X, torch.from_numpy(targets).cuda(), want_logits=True, want_argmax=True)
    tv, ti, y2 = h.forward_topk(X, K)
    torch.cuda.synchronize()
    rows = sample_rows(M)
    y_rows = y[torch.from_numpy(rows).cuda()].cpu().numpy()
    lse, nll, a = lse.cpu().numpy(), nll.cpu().numpy(), a.cpu().numpy().astype(np.int64)
    tv, ti = tv.cpu().numpy(), ti.cpu().numpy().astype(np.int64)
    # both launches compute the same logits
    assert torch.equal(y, y2), "forward_ce and forward_topk wrote different logits"
    # every row against the GPU's own logits, in blocks to bound host memory
    for m0 in range(0, M, 256):
        yb = y[m0:m0 + 256].cpu().numpy()
        sl = slice(m0, m0 + yb.shape[0])
        assert np.array_equal(a[sl], np.argmax(yb, axis=1)), f"rows {m0}..: argmax != first argmax of logits"
        rv, ri = top_k(yb, K)
        assert np.array_equal(ti[sl], ri) and np.array_equal(tv[sl], rv), f"rows {m0}..: top-{K} not exact"
        ref_lse = oracle_softmax.log_sum_exp(yb)
        bound = EPS_ABS + EPS_REL * np.abs(ref_lse)
        assert np.all(np.abs(lse[sl] - ref_lse) <= bound), f"rows {m0}..: lse vs own logits"
        ref_nll = oracle_softmax.cross_entropy(yb, targets[sl])
        assert np.all(np.abs(nll[sl] - ref_nll) <= bound), f"rows {m0}..: nll vs own logits"
    del y, y2
    say(f"prefill: oracle over all {V} vocabulary rows for {rows.size} hidden states")
    ref = oracle_forward.forward(c, c["X"][rows])
    rms = row_rms(ref)
    worst = assert_logits_close(y_rows, ref, rms=rms, what="prefill full-vocabulary rows")
    assert_argmax_ok(a[rows], y_rows, ref, rms=rms, what="prefill full-vocabulary rows")
    r1 = np.abs(lse[rows] - oracle_softmax.log_sum_exp(ref)) / (TOL * rms)
    r2 = np.abs(nll[rows] - oracle_softmax.cross_entropy(ref, targets[rows])) / (2 * TOL * rms)
    assert np.all(r1 <= 1.0), f"lse vs oracle: {r1.max():.3g} x bound"
    assert np.all(r2 <= 1.0), f"nll vs oracle: {r2.max():.3g} x bound"
    kth = np.sort(ref, axis=1)[:, -K]
    for j, m in enumerate(rows):
        chosen = set(ti[m].tolist())
        assert np.all(ref[j, ti[m]] >= kth[j] - TOL * rms[j]), f"row {m}: a top-{K} row far below the oracle's K-th"
        must = np.nonzero(ref[j] > kth[j] + TOL * rms[j])[0]
        assert set(must.tolist()) <= chosen, f"row {m}: missed a clear top-{K} row"
    n_exact = int(np.sum(a[rows] == np.argmax(ref, axis=1)))
    say(f"prefill: {rows.size} rows, worst |d|/(2e-3 rms) = {worst:.3g}, lse {r1.max():.3g}, "
        f"nll {r2.max():.3g}, argmax equal to the oracle's on {n_exact}/{rows.size}")
    h.close()

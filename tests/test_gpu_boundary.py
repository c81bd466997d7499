"""The boundary's argument and workspace rules on the GPU: the binding rejects
tensors of the wrong device, type or shape before any launch; the library
rejects a temperature whose reciprocal overflows; a forward call that must
grow the workspace does so in stream order (results stay right when calls
of growing M follow each other without a wait), and refuses to grow while
its stream is being captured into a graph; a device allocation refused by the
ARCHEAD_TEST_ALLOC_LIMIT hook comes back as ENOMEM and the handle survives it."""
import numpy as np
import pytest

from gpu_util import assert_argmax_ok, assert_logits_close, say
from oracle import forward as oracle_forward
from packed_quantized_lm_amd.synth import random_small_head

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from packed_quantized_lm_amd import load_library
    load_library()


@pytest.fixture(scope="module")
def small():
    from packed_quantized_lm_amd import PackedHead
    f = random_small_head(1200, 512, 32, 8, 128, 8, seed=31)
    h = PackedHead(f)
    yield f, h
    h.close()


def test_binding_rejects_bad_tensors(small):
    import torch
    from packed_quantized_lm_amd import x_tensor_from_bits
    f, h = small
    say("binding: tensors of the wrong device, type or shape")
    X = x_tensor_from_bits(f["X"])
    M, K = X.shape[0], 4
    dev = X.device
    logits = torch.empty((M, f["V"]), dtype=torch.float32, device=dev)
    vals = torch.empty((M, K), dtype=torch.float32, device=dev)
    idx = torch.empty((M, K), dtype=torch.int32, device=dev)
    smp = torch.empty((M,), dtype=torch.int32, device=dev)
    u = torch.rand(M, device=dev)
    bad_u = [u.double(), u[:M - 1], u.cpu(), torch.rand(2 * M, device=dev)[::2]]
    for b in bad_u:
        with pytest.raises((ValueError, TypeError)):
            h.forward_sample_into(X, K, 1.0, b, logits, vals, idx, smp)
    with pytest.raises((ValueError, TypeError)):
        h.forward_sample_into(X.cpu(), K, 1.0, u, logits, vals, idx, smp)
    with pytest.raises((ValueError, TypeError)):
        h.forward_topk_into(X, K, logits, vals.double(), idx)
    with pytest.raises((ValueError, TypeError)):
        h.forward_topk_into(X, K, logits, vals, idx[:, :K - 1])
    with pytest.raises((ValueError, TypeError)):
        h.forward_into(X, logits.cpu(), None)
    with pytest.raises((ValueError, TypeError)):
        h.forward_into(X, logits[:, :-1], None)
    with pytest.raises((ValueError, TypeError)):
        h.forward_into(X, None, torch.empty((M,), dtype=torch.int64, device=dev))
    with pytest.raises((ValueError, TypeError)):
        h.forward_ce_into(X, torch.zeros(M, dtype=torch.int64, device=dev), None, None,
                          torch.empty(M, device=dev), torch.empty(M, device=dev))
    torch.cuda.synchronize()
    # nothing was launched: the right tensors still give the right answer
    h.forward_into(X, logits, None)
    torch.cuda.synchronize()
    ref = oracle_forward.forward(f, f["X"])
    assert_logits_close(logits.cpu().numpy(), ref, what="after rejected calls")


def test_subnormal_temperature_is_rejected(small):
    import torch
    from packed_quantized_lm_amd import x_tensor_from_bits
    from packed_quantized_lm_amd.binding import EINVAL, ArcheadError
    f, h = small
    X = x_tensor_from_bits(f["X"])
    u = torch.rand(X.shape[0], device=X.device)
    for tau in (1e-40, 0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(ArcheadError) as e:
            h.forward_sample(X, 4, tau, u)
        assert e.value.status == EINVAL
    s, v, i, _ = h.forward_sample(X, 4, 1e-30, u)   # tiny but normal: the greedy limit
    torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy(), i[:, 0].cpu().numpy())


def test_workspace_grows_in_stream_order():
    """Calls of growing M enqueued back to back, with no wait between them:
    each growth allocates and zeroes the new workspace on the stream and frees
    the old one behind the calls still using it."""
    import torch
    from packed_quantized_lm_amd import PackedHead, x_tensor_from_bits
    say("workspace growth in stream order")
    f = random_small_head(3000, 1024, 64, 16, 128, 200, seed=33)
    h = PackedHead(f)
    X = x_tensor_from_bits(f["X"])
    outs = []
    for M in (1, 2, 5, 40, 130, 200, 3):
        y = torch.empty((M, f["V"]), dtype=torch.float32, device=X.device)
        a = torch.empty((M,), dtype=torch.int32, device=X.device)
        h.forward_into(X[:M], y, a)
        outs.append((M, y, a))
    torch.cuda.synchronize()
    ref = oracle_forward.forward(f, f["X"])
    for M, y, a in outs:
        yy = y.cpu().numpy()
        assert_logits_close(yy, ref[:M], what=f"M={M}")
        assert_argmax_ok(a.cpu().numpy().astype(np.int64), yy, ref[:M], what=f"M={M}")
    h.close()


def test_growth_refused_while_capturing():
    import torch
    from packed_quantized_lm_amd import PackedHead, x_tensor_from_bits
    from packed_quantized_lm_amd.binding import EINVAL, ArcheadError
    say("workspace growth refused under graph capture")
    f = random_small_head(1000, 512, 32, 8, 128, 40, seed=34)
    h = PackedHead(f)
    X = x_tensor_from_bits(f["X"])
    y = torch.empty((40, f["V"]), dtype=torch.float32, device=X.device)
    a = torch.empty((40,), dtype=torch.int32, device=X.device)
    h.reserve(8)
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    err = None
    with torch.cuda.graph(g, stream=side):
        try:
            h.forward_into(X, y, a)          # M = 40 > 8: would grow
        except ArcheadError as e:
            err = e
        h.forward_into(X[:8], y[:8], a[:8])  # fits: captured
    assert err is not None and err.status == EINVAL, "growth under capture was not refused"
    torch.cuda.synchronize()
    ref = oracle_forward.forward(f, f["X"][:8])
    for rep in range(3):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        yy = y[:8].cpu().numpy()
        assert_logits_close(yy, ref, what=f"replay {rep}")
        assert_argmax_ok(a[:8].cpu().numpy().astype(np.int64), yy, ref, what=f"replay {rep}")
    del g
    # outside the capture the same call grows the workspace and succeeds
    h.forward_into(X, y, a)
    torch.cuda.synchronize()
    ref = oracle_forward.forward(f, f["X"])
    assert_logits_close(y.cpu().numpy(), ref, what="after capture")
    h.close()


def test_allocation_failure_is_a_status(monkeypatch):
    """With ARCHEAD_TEST_ALLOC_LIMIT set, the packed head's block, a workspace
    growth and the construction's buffers are refused as if the device were out
    of memory: each call returns ENOMEM, nothing aborts, and the handle keeps
    its old workspace and works again once the limit is lifted."""
    import torch
    from packed_quantized_lm_amd import PackedHead, build_head, x_tensor_from_bits
    from packed_quantized_lm_amd.binding import ENOMEM, ArcheadError
    say("allocation failure injected through ARCHEAD_TEST_ALLOC_LIMIT")
    f = random_small_head(2000, 512, 32, 8, 128, 150, seed=35)
    monkeypatch.setenv("ARCHEAD_TEST_ALLOC_LIMIT", "1024")
    with pytest.raises(ArcheadError) as e:
        PackedHead(f)
    assert e.value.status == ENOMEM
    monkeypatch.delenv("ARCHEAD_TEST_ALLOC_LIMIT")
    h = PackedHead(f)
    h.reserve(2)
    X = x_tensor_from_bits(f["X"])
    y = torch.empty((150, f["V"]), dtype=torch.float32, device=X.device)
    a = torch.empty((150,), dtype=torch.int32, device=X.device)
    monkeypatch.setenv("ARCHEAD_TEST_ALLOC_LIMIT", "1024")
    with pytest.raises(ArcheadError) as e:
        h.forward_into(X, y, a)                 # M = 150 would grow the workspace
    assert e.value.status == ENOMEM
    h.forward_into(X[:2], y[:2], a[:2])         # fits the workspace it has
    torch.cuda.synchronize()
    ref = oracle_forward.forward(f, f["X"])
    assert_logits_close(y[:2].cpu().numpy(), ref[:2], what="after a refused growth")
    W = torch.randn(256, 128, dtype=torch.float64, device=X.device)
    H = torch.randn(64, 128, dtype=torch.float64, device=X.device)
    with pytest.raises(ArcheadError) as e:
        build_head(W, H, 8, 4, 32)
    assert e.value.status == ENOMEM
    monkeypatch.delenv("ARCHEAD_TEST_ALLOC_LIMIT")
    h.forward_into(X, y, a)
    torch.cuda.synchronize()
    yy = y.cpu().numpy()
    assert_logits_close(yy, ref, what="limit lifted")
    assert_argmax_ok(a.cpu().numpy().astype(np.int64), yy, ref, what="limit lifted")
    h.close()

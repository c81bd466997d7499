"""archead_forward_argmax_noalloc through the C ABI: the forward on the
library's fixed per-GPU workspace gives exactly what archead_forward_argmax
gives (logits bit for bit, the same indices), on two calls in a row with the
second one smaller, across heads of different shapes that share the one
workspace, at the full decode and batched-decode shapes, and under graph
capture; a call whose workspace would not fit is refused before any launch."""
import numpy as np
import pytest

from gpu_util import assert_argmax_ok, assert_logits_close, say
from oracle import forward as oracle_forward
from packed_quantized_lm_amd.synth import make_config, random_small_head

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from packed_quantized_lm_amd import load_library
    load_library()


def both(h, X, V):
    """(logits, argmax) from archead_forward_argmax and from the no-allocation call."""
    import torch
    M = X.shape[0]
    y0 = torch.empty((M, V), dtype=torch.float32, device=X.device)
    a0 = torch.empty((M,), dtype=torch.int32, device=X.device)
    y1 = torch.full((M, V), float("nan"), dtype=torch.float32, device=X.device)
    a1 = torch.full((M,), -1, dtype=torch.int32, device=X.device)
    h.forward_into(X, y0, a0)
    h.forward_argmax_noalloc_into(X, y1, a1)
    torch.cuda.synchronize()
    return y0.cpu().numpy(), a0.cpu().numpy(), y1.cpu().numpy(), a1.cpu().numpy()


def check(h, f, Xb, what):
    from packed_quantized_lm_amd import x_tensor_from_bits
    X = x_tensor_from_bits(Xb)
    y0, a0, y1, a1 = both(h, X, f["V"])
    assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32)), f"{what}: logits differ"
    assert np.array_equal(a0, a1), f"{what}: argmax differs"
    return y1, a1


@pytest.mark.parametrize("shape", [
    # V,    d,    k,   r,   g,  M first, M second
    (3000, 1024, 64, 16, 128, 2, 1),     # single launch, then single launch with fewer rows
    (2500, 1536, 96, 33, 128, 40, 3),    # streaming kernel, then the single launch's neighbour
    (1200, 512, 16, 8, 32, 130, 17),     # large-M kernel, then the streaming kernel
])
def test_two_calls_second_smaller(shape):
    V, d, k, r, g, M1, M2 = shape
    say(f"no-alloc {shape}")
    from packed_quantized_lm_amd import PackedHead
    f = random_small_head(V, d, k, r, g, M1, seed=V + d + M1)
    h = PackedHead(f)
    ref = oracle_forward.forward(f, f["X"])
    for M in (M1, M2):
        y, a = check(h, f, f["X"][:M], f"{shape} M={M}")
        assert_logits_close(y, ref[:M], what=f"{shape} M={M}")
        assert_argmax_ok(a.astype(np.int64), y, ref[:M], what=f"{shape} M={M}")
    h.close()


def test_heads_of_different_shapes_share_the_workspace():
    """The workspace keeps the last call's contents: a head with a larger
    rank leaves values where a smaller head's padding columns and counters
    lie; each call must clear what has to start at zero."""
    from packed_quantized_lm_amd import PackedHead
    say("no-alloc: heads of different shapes in turn")
    fa = random_small_head(4000, 1024, 200, 60, 128, 2, seed=41)
    fb = random_small_head(3001, 512, 33, 7, 128, 2, seed=42)
    ha, hb = PackedHead(fa), PackedHead(fb)
    ra, rb = oracle_forward.forward(fa, fa["X"]), oracle_forward.forward(fb, fb["X"])
    for f, h, ref in ((fa, ha, ra), (fb, hb, rb), (fa, ha, ra), (fb, hb, rb)):
        for M in (2, 1):
            y, a = check(h, f, f["X"][:M], f"V={f['V']} M={M}")
            assert_logits_close(y, ref[:M], what=f"V={f['V']} M={M}")
    ha.close()
    hb.close()


@pytest.mark.parametrize("name,M", [("qwen_m1", 1), ("qwen_m32", 32), ("qwen_m32", 5)])
def test_full_size(name, M):
    from packed_quantized_lm_amd import PackedHead
    say(f"no-alloc full size {name} M={M}")
    c = make_config(name)
    h = PackedHead(c)
    check(h, c, c["X"][:M], f"{name} M={M}")
    h.close()


def test_too_large_is_refused():
    import torch
    from packed_quantized_lm_amd import PackedHead, x_tensor_from_bits
    from packed_quantized_lm_amd.binding import ESHAPE, ArcheadError
    say("no-alloc: refusal above the fixed workspace")
    f = random_small_head(1000, 4096, 32, 8, 128, 1100, seed=43)
    h = PackedHead(f)
    X = x_tensor_from_bits(f["X"])
    y = torch.empty((1100, 1000), dtype=torch.float32, device=X.device)
    a = torch.empty((1100,), dtype=torch.int32, device=X.device)
    with pytest.raises(ArcheadError) as e:
        h.forward_argmax_noalloc_into(X, y, a)
    assert e.value.status == ESHAPE
    h.close()


def test_graph_capture_replays():
    import torch
    from packed_quantized_lm_amd import PackedHead, x_tensor_from_bits
    say("no-alloc: captured in a graph, replayed")
    f = random_small_head(3000, 1024, 64, 16, 128, 40, seed=44)
    h = PackedHead(f)
    X = x_tensor_from_bits(f["X"])
    outs = {}
    for M in (1, 40):
        y = torch.empty((M, f["V"]), dtype=torch.float32, device=X.device)
        a = torch.empty((M,), dtype=torch.int32, device=X.device)
        h.forward_into(X[:M], y, a)
        torch.cuda.synchronize()
        outs[M] = (y.clone(), a.clone(), y, a)
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for M in (1, 40):
            h.forward_argmax_noalloc_into(X[:M], outs[M][2], outs[M][3])
    for rep in range(4):
        for M in (1, 40):
            outs[M][2].fill_(float("nan"))
            outs[M][3].fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for M in (1, 40):
            y0, a0, y, a = outs[M]
            assert torch.equal(y, y0), f"replay {rep} M={M}: logits differ"
            assert torch.equal(a, a0), f"replay {rep} M={M}: argmax differs"
        h.forward_into(X[:1], outs[1][2], outs[1][3])  # eager work between replays
        torch.cuda.synchronize()
    del g
    h.close()

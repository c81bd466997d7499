"""The construction of a packed head on the GPU (archead_build,
archead_quantize) against the oracle's packer (oracle/packer.py).

- The quantiser alone is bit-exact against oracle/quant.py: on the oracle's
  own unquantised factors of the tiny head (A_c, B_c, W - A_c B_c, A_w,
  B_w) and on random rows with edge cases (zero groups, scales that round to
  fp16 subnormals or overflow, exact rounding ties).
- The whole construction, on the tiny head, meets the pins the oracle's own
  construction meets (tests/test_oracle_packer.py): the core is the best
  rank-k approximation of W with sqrt(sigma) on each side, the residual
  codes and scales are those of W minus the unquantised core.  Its
  correction attains the metric objective of the oracle's exact one to
  within the randomized SVD's approximation (a stated tolerance), and never
  beats the Eckart-Young-Mirsky tail of its own E T_p.
"""
import numpy as np
import pytest

from gpu_util import say
from oracle import packer
from oracle.layout import f16_bits_to_f64, unpack_r4
from oracle.quant import dequantize_groups, quantize_groups
from packed_quantized_lm_amd.synth import make_config
from test_oracle_packer import _core_and_residual_pins

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from packed_quantized_lm_amd import load_library
    load_library()


@pytest.fixture(scope="module")
def tiny():
    c = make_config("tiny")
    f, inter = packer.pack(c["W"], c["H"], c["k"], c["r"], c["g"], p=0.75, lam=1e-2)
    return c, f, inter


def gpu_quantize(x, bits, group):
    import torch
    from packed_quantized_lm_amd import quantize
    q, s = quantize(torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)).cuda(), bits, group)
    torch.cuda.synchronize()
    s = s.cpu().numpy().view(np.uint16)
    return q.cpu().numpy(), (s.reshape(-1) if group is None else s)


def assert_same_quant(x, bits, group, what):
    q, s = gpu_quantize(x, bits, group)
    rq, rs = quantize_groups(x, bits, group)
    assert np.array_equal(s.reshape(rs.shape), rs), f"{what}: scales differ at {np.argwhere(s.reshape(rs.shape) != rs)[:5]}"
    assert np.array_equal(q, rq), f"{what}: codes differ at {np.argwhere(q != rq)[:5]}"


def test_quantiser_on_the_oracle_factors(tiny):
    c, f, inter = tiny
    say("quantiser on the oracle's unquantised factors")
    assert_same_quant(inter["A_c"], 5, None, "A_c")
    assert_same_quant(inter["B_c"], 8, None, "B_c")
    assert_same_quant(c["W"] - inter["A_c"] @ inter["B_c"], 4, c["g"], "residual")
    assert_same_quant(inter["A_w"], 8, None, "A_w")
    assert_same_quant(inter["B_w"], 8, c["g"], "B_w")


@pytest.mark.parametrize("bits,group", [(4, 32), (5, None), (8, None), (8, 64), (4, 128), (2, 16)])
def test_quantiser_edge_cases(bits, group):
    rng = np.random.default_rng(bits * 100 + (group or 0))
    cols = 256
    x = rng.standard_normal((64, cols)) * np.exp(rng.uniform(-20, 12, size=(64, 1)))
    x[3] = 0.0                                            # an all-zero row (zero scale)
    x[5, : (group or cols)] = 0.0                         # one zero group
    x[7] *= 1e-9                                          # scales deep in the fp16 subnormals
    x[9] = 1e6                                            # absmax / qmax past fp16's range (infinite scale)
    x[11] = -x[11]
    # exact rounding ties: x / s lands on k + 1/2 for the fp16 scale the row gets
    qmax = 2 ** (bits - 1) - 1
    g = group or cols
    for row in (13, 15):
        s = np.float64(np.float16(3.0 / qmax))
        x[row] = s * (rng.integers(-qmax, qmax, size=cols) + 0.5)
        x[row, ::g] = 3.0                                  # each group's maximum fixes s
    say(f"quantiser edge cases bits={bits} group={group}")
    assert_same_quant(x, bits, group, f"bits={bits} group={group}")


def gpu_build(c, p=0.75, lam=1e-2, power_iters=8, oversample=16, seed=7):
    import torch
    from packed_quantized_lm_amd import build_head
    W = torch.from_numpy(np.ascontiguousarray(c["W"], dtype=np.float64)).cuda()
    H = torch.from_numpy(np.ascontiguousarray(c["H"], dtype=np.float64)).cuda()
    f = build_head(W, H, c["k"], c["r"], c["g"], p=p, lam=lam, power_iters=power_iters, oversample=oversample,
                   seed=seed)
    torch.cuda.synchronize()
    return f


def test_build_core_and_residual_meet_the_pins(tiny):
    c, _, _ = tiny
    say("GPU construction of the tiny head: core and residual")
    f = gpu_build(c)
    assert f["A5"].min() >= -16 and f["A5"].max() <= 15
    assert _core_and_residual_pins(c["W"], f) == []


def _correction_objective(W, f, T):
    """||(E - (sC o C8)(sD o D8)) T||_F^2 with E = W - W_d of the fields."""
    g = f["g"]
    A = dequantize_groups(f["A5"], f["sA"], None) if f["k"] else 0
    B = dequantize_groups(f["B8"], f["sB"], None) if f["k"] else 0
    R = dequantize_groups(unpack_r4(f["R4"], f["d"]), f["sR"], g)
    E = W - (A @ B if f["k"] else 0) - R
    C = f16_bits_to_f64(f["sC"])[:, None] * f["C8"]
    D = np.repeat(f16_bits_to_f64(f["sD"]), g, axis=1) * f["D8"]
    return float(np.sum(((E - C @ D) @ T) ** 2)), E


@pytest.mark.parametrize("p", [0.75, 0.5])
def test_build_correction_against_the_oracle(tiny, p):
    c = tiny[0]
    say(f"GPU construction of the tiny head: correction, p={p}")
    of, inter = packer.pack(c["W"], c["H"], c["k"], c["r"], c["g"], p=p, lam=1e-2)
    T = inter["metric"]["T"]
    f = gpu_build(c, p=p, oversample=48)
    obj_gpu, E_gpu = _correction_objective(c["W"], f, T)
    obj_ora, _ = _correction_objective(c["W"], of, T)
    # the quantised correction of the GPU's own E T_p cannot beat that
    # matrix's Eckart-Young-Mirsky tail
    s = np.linalg.svd(E_gpu @ T, compute_uv=False)
    tail = float(np.sum(s[c["r"]:] ** 2))
    assert obj_gpu >= tail * (1 - 1e-12)
    # and it is as good as the oracle's (exact SVD, same quantisers) to within
    # the randomized SVD's shortfall: 1 % of the objective
    assert obj_gpu <= obj_ora * 1.01, f"objective {obj_gpu} vs oracle {obj_ora} (tail {tail})"
    # the correction removes most of what the exact one removes
    total = float(np.sum((E_gpu @ T) ** 2))
    assert total - obj_gpu >= 0.97 * (total - obj_ora)
    say(f"  objective GPU {obj_gpu:.6g}, oracle {obj_ora:.6g}, tail {tail:.6g}, uncorrected {total:.6g}")


def test_build_rejects_bad_arguments(tiny):
    import torch
    from packed_quantized_lm_amd import build_head
    from packed_quantized_lm_amd.binding import EINVAL, ESHAPE, ArcheadError
    c = tiny[0]
    W = torch.from_numpy(np.ascontiguousarray(c["W"], dtype=np.float64)).cuda()
    H = torch.from_numpy(np.ascontiguousarray(c["H"], dtype=np.float64)).cuda()
    with pytest.raises(ArcheadError) as e:
        build_head(W, H, c["k"], c["r"], c["g"], p=0.6)
    assert e.value.status == EINVAL
    with pytest.raises(ArcheadError) as e:
        build_head(W, H, c["k"], c["r"], 48)
    assert e.value.status == ESHAPE
    with pytest.raises(ArcheadError) as e:
        build_head(W, H, c["k"], c["r"], c["g"], lam=0.0)
    assert e.value.status == EINVAL


def test_built_head_runs_through_the_forward(tiny):
    """The GPU-built fields load into archead_pack_load, and the forward of that
    head matches the oracle's forward of the same fields."""
    from gpu_util import assert_logits_close, gpu_forward
    from oracle import forward as oracle_forward
    from packed_quantized_lm_amd import PackedHead
    c = tiny[0]
    f = gpu_build(c)
    h = PackedHead(f)
    y, _ = gpu_forward(h, c["X"])
    assert_logits_close(y, oracle_forward.forward(f, c["X"]), what="GPU-built head")
    h.close()

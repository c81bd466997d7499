"""Pins of the oracle's dense forward (ARCHead paper eqs 3, 6, 7).

The forward has a plain definition, so it is pinned to things other than
itself: an independent C triple loop that decodes the canonical bytes with
its own code, a hand-worked example (tests/golden/forward_example.txt),
one-hot closed forms, and special cases that reduce to plain integer matrix
products.  The last tests plant typical mistakes in a copy of the oracle and
check that the pins catch every one of them.
"""
import numpy as np
import pytest

from conftest import golden_lines
from oracle import forward, naive
from packed_quantized_lm_amd.synth import make_config, random_small_head, to_bf16_bits, to_f16_bits


def hand_example():
    V, d, k, r, g = 2, 64, 1, 1, 32
    j = np.arange(d)
    R4 = np.stack([(j % 16) - 8, np.ones(d, dtype=int)])
    nib = (R4 & 0xF).astype(np.uint8)                    # the test's own packing
    f = {"V": V, "d": d, "k": k, "r": r, "g": g,
         "A5": np.array([[3], [-16]], np.int8), "sA": to_f16_bits([0.5, 0.25]),
         "B8": (j - 32).astype(np.int8)[None, :], "sB": to_f16_bits([0.125]),
         "R4": nib[:, 0::2] | (nib[:, 1::2] << 4),
         "sR": to_f16_bits([[1.0, 0.5], [2.0, 0.0625]]),
         "C8": np.array([[10], [-128]], np.int8), "sC": to_f16_bits([0.015625, 1.0]),
         "D8": np.where(j % 2 == 0, 127, -127).astype(np.int8)[None, :],
         "sD": to_f16_bits([[0.5, 0.25]])}
    x = np.zeros((1, d))
    x[0, 0], x[0, 33], x[0, 63] = 1.0, 2.0, -0.5
    return f, to_bf16_bits(x)


def expected_hand():
    rows = dict(golden_lines("forward_example.txt"))
    return (np.array([[float(v) for v in rows["logits"].split(",")]]),
            np.array([int(rows["argmax"])]))


def test_hand_worked_example():
    f, X = hand_example()
    want, want_arg = expected_hand()
    got = forward.forward(f, X)
    assert np.array_equal(got, want)              # every step is exact in fp64
    assert np.array_equal(forward.argmax_first(got), want_arg)
    assert np.array_equal(naive.forward(f, X), want)


@pytest.mark.parametrize("shape", [(2048, 256, 16, 4, 32, 4), (37, 128, 5, 3, 64, 3),
                                   (16, 64, 1, 0, 32, 1), (9, 384, 33, 7, 128, 5)])
def test_numpy_oracle_matches_independent_c_triple_loop(shape):
    V, d, k, r, g, M = shape
    f = random_small_head(V, d, k, r, g, M, seed=V + d)
    a = forward.forward(f, f["X"])
    b = naive.forward(f, f["X"])
    scale = np.abs(a).max()
    assert np.max(np.abs(a - b)) <= 1e-12 * scale


def test_tiny_config_packed_by_the_oracle_matches_c():
    from oracle import packer
    c = make_config("tiny")
    f, _ = packer.pack(c["W"], c["H"], c["k"], c["r"], c["g"])
    a = forward.forward(f, c["X"])
    assert np.max(np.abs(a - naive.forward(f, c["X"]))) <= 1e-12 * np.abs(a).max()


def _one_hot_rows(d, cols):
    x = np.zeros((len(cols), d))
    x[np.arange(len(cols)), cols] = 1.0
    return to_bf16_bits(x)


def _test_packed_r4(vals):
    nib = (np.asarray(vals) & 0xF).astype(np.uint8)
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


def test_one_hot_reads_back_each_integer_field():
    rng = np.random.default_rng(11)
    V, d, k, r, g = 40, 128, 8, 4, 32
    G = d // g
    one, zero = to_f16_bits(1.0), to_f16_bits(0.0)
    cols = [0, 5, 77, 127]
    X = _one_hot_rows(d, cols)
    base = {"V": V, "d": d, "k": k, "r": r, "g": g,
            "A5": np.zeros((V, k), np.int8), "sA": np.full(V, zero, np.uint16),
            "B8": np.zeros((k, d), np.int8), "sB": np.full(k, one, np.uint16),
            "R4": np.zeros((V, d // 2), np.uint8), "sR": np.full((V, G), one, np.uint16),
            "C8": np.zeros((V, r), np.int8), "sC": np.full(V, zero, np.uint16),
            "D8": np.zeros((r, d), np.int8), "sD": np.full((r, G), one, np.uint16)}
    # R4: logits[m, v] = R4[v, col_m]
    r4 = rng.integers(-8, 8, size=(V, d))
    f = dict(base, R4=_test_packed_r4(r4))
    assert np.array_equal(forward.forward(f, X), r4[:, cols].T)
    # A5 through B8 = [I | 0]: logits[m, v] = A5[v, col_m] for col_m < k
    a5 = rng.integers(-16, 16, size=(V, k)).astype(np.int8)
    eye = np.zeros((k, d), np.int8)
    eye[np.arange(k), np.arange(k)] = 1
    f = dict(base, A5=a5, B8=eye, sA=np.full(V, one, np.uint16), sR=np.full((V, G), zero, np.uint16))
    Xa = _one_hot_rows(d, [0, 3, 7])
    assert np.array_equal(forward.forward(f, Xa), a5[:, [0, 3, 7]].T)
    # B8 through A5 = delta: logits[m, v] = B8[v, col_m] for v < k
    b8 = rng.integers(-128, 128, size=(k, d)).astype(np.int8)
    a5d = np.zeros((V, k), np.int8)
    a5d[np.arange(k), np.arange(k)] = 1
    f = dict(base, A5=a5d, B8=b8, sA=np.full(V, one, np.uint16), sR=np.full((V, G), zero, np.uint16))
    got = forward.forward(f, X)
    assert np.array_equal(got[:, :k], b8[:, cols].T)
    assert np.array_equal(got[:, k:], np.zeros((len(cols), V - k)))
    # C8 through D8 = [I | 0]
    c8 = rng.integers(-128, 128, size=(V, r)).astype(np.int8)
    eye = np.zeros((r, d), np.int8)
    eye[np.arange(r), np.arange(r)] = 1
    f = dict(base, C8=c8, D8=eye, sC=np.full(V, one, np.uint16), sR=np.full((V, G), zero, np.uint16))
    assert np.array_equal(forward.forward(f, _one_hot_rows(d, [1, 2])), c8[:, [1, 2]].T)
    # D8 through C8 = delta
    d8 = rng.integers(-128, 128, size=(r, d)).astype(np.int8)
    c8d = np.zeros((V, r), np.int8)
    c8d[np.arange(r), np.arange(r)] = 1
    f = dict(base, C8=c8d, D8=d8, sC=np.full(V, one, np.uint16), sR=np.full((V, G), zero, np.uint16))
    got = forward.forward(f, X)
    assert np.array_equal(got[:, :r], d8[:, cols].T)


def test_residual_only_head_is_a_group_dequant_gemv():
    # sA = sC = 0: the head is the plain group-INT4 baseline; its logits are
    # sum over groups of sR[v, grp] * (integer dot of X's group with R4's group).
    rng = np.random.default_rng(5)
    V, d, g, M = 50, 256, 64, 3
    f = random_small_head(V, d, 4, 2, g, M, seed=9)
    r4 = rng.integers(-8, 8, size=(V, d))
    f.update(R4=_test_packed_r4(r4), sA=to_f16_bits(np.zeros(V)), sC=to_f16_bits(np.zeros(V)))
    # X with small-integer entries so every product and sum is an exact integer
    xi = rng.integers(-5, 6, size=(M, d))
    sR = np.asarray(f["sR"]).view(np.float16).astype(np.float64)
    want = np.zeros((M, V))
    for grp in range(d // g):
        sl = slice(grp * g, (grp + 1) * g)
        want += (xi[:, sl] @ r4[:, sl].T) * sR[:, grp][None, :]
    got = forward.forward(f, to_bf16_bits(xi.astype(np.float64)))
    assert np.allclose(got, want, rtol=1e-13, atol=0)


def test_low_rank_only_head_is_the_factored_product_of_eq7():
    # R4 = 0 and sC = 0: the head is (sA o A5)(sB o B8); eq 7 factors the
    # logits as (X (sB o B8)^T)(sA o A5)^T.  With integer X the inner product
    # is an exact integer matrix product.
    rng = np.random.default_rng(6)
    V, d, k, M = 30, 128, 12, 4
    f = random_small_head(V, d, k, 3, 32, M, seed=2)
    f.update(R4=np.zeros((V, d // 2), np.uint8), sC=to_f16_bits(np.zeros(V)))
    xi = rng.integers(-3, 4, size=(M, d))
    t = (xi @ f["B8"].astype(np.int64).T) * np.asarray(f["sB"]).view(np.float16).astype(np.float64)
    want = t @ (f["A5"].astype(np.float64) * np.asarray(f["sA"]).view(np.float16).astype(np.float64)[:, None]).T
    got = forward.forward(f, to_bf16_bits(xi.astype(np.float64)))
    assert np.allclose(got, want, rtol=1e-12, atol=0)


def test_argmax_takes_the_lowest_index_among_ties():
    y = np.array([[1.0, 3.0, 3.0, -1.0], [0.0, 0.0, 0.0, 0.0], [-5.0, -4.0, -4.0, -4.5]])
    assert list(forward.argmax_first(y)) == [1, 0, 1]


def test_row_subset_equals_full_forward():
    f = random_small_head(100, 128, 8, 4, 32, 2, seed=4)
    full = forward.forward(f, f["X"])
    rows = np.array([99, 0, 17, 64])
    # BLAS may block differently for different row counts: equal to round-off
    tol = 1e-13 * np.abs(full).max()
    assert np.max(np.abs(forward.forward(f, f["X"], rows=rows) - full[:, rows])) <= tol
    assert np.max(np.abs(forward.forward(f, f["X"], block=7) - full)) <= tol


# --- planted mistakes: each must break at least one pin --------------------------

def _mutants():
    from oracle.layout import f16_bits_to_f64, unpack_r4

    def make(drop=None, sign=False, transpose_r4=False, group_of_row=False, swap_scales=False):
        def dense_rows(f, rows):
            d, g = f["d"], f["g"]
            rows = np.asarray(rows)
            sA = f16_bits_to_f64(f["sA"][rows])
            sC = f16_bits_to_f64(f["sC"][rows])
            if swap_scales:
                sA, sC = sC, sA
            A = f["A5"][rows].astype(np.float64) * sA[:, None]
            B = f["B8"].astype(np.float64) * f16_bits_to_f64(f["sB"])[:, None]
            R = unpack_r4(f["R4"][rows], d).astype(np.float64)
            if transpose_r4:
                R = R.reshape(len(rows), d // 2, 2)[:, :, ::-1].reshape(len(rows), d)
            sRm = f16_bits_to_f64(f["sR"][rows])
            sR = np.repeat(sRm, g, axis=1) if not group_of_row else np.tile(sRm, (1, g))
            C = f["C8"][rows].astype(np.float64) * sC[:, None]
            D = f["D8"].astype(np.float64) * np.repeat(f16_bits_to_f64(f["sD"]), g, axis=1)
            terms = {"core": A @ B, "resid": sR * R, "corr": C @ D}
            if sign:
                terms["corr"] = -terms["corr"]
            return sum(v for n, v in terms.items() if n != drop)
        return dense_rows

    return {"drop core": make(drop="core"), "drop residual": make(drop="resid"),
            "drop correction": make(drop="corr"), "wrong sign": make(sign=True),
            "swapped nibbles": make(transpose_r4=True), "wrong group index": make(group_of_row=True),
            "swapped row scales": make(swap_scales=True)}


@pytest.mark.parametrize("name", list(_mutants()))
def test_pins_catch_planted_mistake(name, monkeypatch):
    monkeypatch.setattr(forward, "dense_rows", _mutants()[name])
    caught = []
    for pin in (test_hand_worked_example, test_one_hot_reads_back_each_integer_field,
                lambda: test_numpy_oracle_matches_independent_c_triple_loop((37, 128, 5, 3, 64, 3))):
        try:
            pin()
        except AssertionError:
            caught.append(pin)
    assert caught, f"no pin caught the planted mistake: {name}"

"""Seeded synthetic inputs for the packed ARCHead LM-head forward.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic (no quantiser, no dequantisation, no product).  Both the
CPU oracle's tests and the HIP path's tests take their inputs from here.

The shapes follow the heads the ARCHead pages name: the Qwen3-8B-Base output
head is 151,936 x 4,096 (ARCHead paper, section 1), and a 2,048-token
calibration budget is the smallest one the pages sweep (aifeed.sk article,
GPTQ comparison paragraph).  The pages give no weights, so the packed fields
are drawn directly with the value ranges each field can hold:

* A5 (V x k) signed 5-bit in [-16, 15], one fp16 scale per row (sA);
* B8 (k x d) int8, one fp16 scale per row (sB);
* R4 (V x d) signed 4-bit in [-8, 7], nibble-packed, one fp16 scale per
  (row, g-column group) (sR);
* C8 (V x r) int8, one fp16 scale per row (sC);
* D8 (r x d) int8, one fp16 scale per (row, g-column group) (sD).

The canonical host layout (also the C ABI's) is row-major everywhere; R4 byte
[v, c] holds column 2c in its low nibble and column 2c+1 in its high nibble,
both 4-bit two's complement.  A uniform random byte therefore carries two
independent uniform draws from [-8, 7], so R4 is drawn as raw bytes.  Scales
are fp16 bit patterns (uint16), X rows are bf16 bit patterns (uint16).

For the tiny head the generator returns a dense W and calibration states H
instead of packed fields; the construction that packs them is the oracle's.
"""
from __future__ import annotations

import numpy as np

# name -> (V, d, k, r, g, M)
CONFIGS = {
    "tiny": dict(V=2048, d=256, k=16, r=4, g=32, M=4),
    "qwen_m1": dict(V=151936, d=4096, k=256, r=64, g=128, M=1),
    "qwen_m32": dict(V=151936, d=4096, k=256, r=64, g=128, M=32),
    "qwen_m2048": dict(V=151936, d=4096, k=256, r=64, g=128, M=2048),
    "large_m8": dict(V=262144, d=2560, k=192, r=48, g=128, M=8),
    # the baselines the pages compare against, at the Qwen head's shape and on
    # the same kernels: a plain group-INT4 head (no core, no correction) with
    # the group size whose bytes come closest to the packed head's from below
    # (g = 32: 350.1 MB against 356.8 MB by eq 10), and "SVD8 + INT4": a rank-256 INT8
    # low-rank pair (held in the INT8 pair's slot) plus the group-INT4
    # residual, without the activation-metric correction
    "int4_g32_m1": dict(V=151936, d=4096, k=0, r=0, g=32, M=1),
    "int4_g32_m2048": dict(V=151936, d=4096, k=0, r=0, g=32, M=2048),
    "svd8_int4_m1": dict(V=151936, d=4096, k=0, r=256, g=128, M=1),
    "svd8_int4_m2048": dict(V=151936, d=4096, k=0, r=256, g=128, M=2048),
}
CONFIG_ORDER = ["tiny", "qwen_m1", "qwen_m32", "qwen_m2048", "large_m8",
                "int4_g32_m1", "int4_g32_m2048", "svd8_int4_m1", "svd8_int4_m2048"]
# configs that share one head (same seed) and differ only in X
_HEAD_FAMILIES = {"qwen": 1, "int4_g32": 10, "svd8_int4": 11}

_BASE_SEED = 0xA4C0


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *key])))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Encode float values as bf16 bit patterns, rounding to nearest even."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Encode float values as IEEE binary16 bit patterns (numpy rounds to nearest even)."""
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float16)).view(np.uint16)


def log_uniform(rng: np.random.Generator, lo: float, hi: float, shape) -> np.ndarray:
    return np.exp(rng.uniform(np.log(lo), np.log(hi), size=shape))


def channel_sigmas(rng: np.random.Generator, d: int, n_outliers: int, outlier_factor: float) -> np.ndarray:
    """Anisotropic per-channel standard deviations: LogNormal(0, 1), with a few
    seeded outlier channels scaled up (the pages' motivation: final hidden
    states are anisotropic, ARCHead paper section 1)."""
    sigma = rng.lognormal(0.0, 1.0, size=d)
    if n_outliers:
        idx = rng.choice(d, size=n_outliers, replace=False)
        sigma[idx] *= outlier_factor
    return sigma


def hidden_states(rng: np.random.Generator, n: int, sigma: np.ndarray) -> np.ndarray:
    return rng.standard_normal((n, sigma.shape[0])) * sigma[None, :]


def random_head(V: int, d: int, k: int, r: int, g: int, seed: int) -> dict:
    """Packed fields drawn directly from their value ranges (canonical host layout)."""
    G = d // g
    out = {"V": V, "d": d, "k": k, "r": r, "g": g}
    rng = _rng(seed, 1)
    out["A5"] = rng.integers(-16, 16, size=(V, k), dtype=np.int8)
    out["sA"] = to_f16_bits(log_uniform(rng, 1e-3, 1e-2, V))
    rng = _rng(seed, 2)
    out["B8"] = rng.integers(-128, 128, size=(k, d), dtype=np.int8)
    out["sB"] = to_f16_bits(log_uniform(rng, 1e-3, 1e-2, k))
    rng = _rng(seed, 3)
    out["R4"] = np.frombuffer(rng.bytes(V * (d // 2)), dtype=np.uint8).reshape(V, d // 2).copy()
    out["sR"] = to_f16_bits(log_uniform(rng, 1e-4, 1e-3, (V, G)))
    rng = _rng(seed, 4)
    out["C8"] = rng.integers(-128, 128, size=(V, r), dtype=np.int8)
    out["sC"] = to_f16_bits(log_uniform(rng, 1e-3, 1e-2, V))
    rng = _rng(seed, 5)
    out["D8"] = rng.integers(-128, 128, size=(r, d), dtype=np.int8)
    out["sD"] = to_f16_bits(log_uniform(rng, 1e-4, 1e-3, (r, G)))
    return out


def random_x(M: int, d: int, seed: int, n_outliers: int = 0, outlier_factor: float = 1.0) -> np.ndarray:
    """M bf16 hidden states (bit patterns), per-channel sigma ~ LogNormal(0, 1)."""
    rng = _rng(seed, 7)
    sigma = channel_sigmas(rng, d, n_outliers, outlier_factor)
    return to_bf16_bits(hidden_states(_rng(seed, 8), M, sigma))


def tiny_dense(seed: int = _BASE_SEED) -> dict:
    """Dense head and calibration set of the tiny configuration.

    W = P Q + N with P (V x 16), Q (16 x d) ~ N(0, 0.05^2) and N ~ N(0, 0.01^2);
    512 calibration rows and 4 forward rows share one anisotropic channel-sigma
    vector with 2 outlier channels x20.
    """
    c = CONFIGS["tiny"]
    V, d = c["V"], c["d"]
    rng = _rng(seed, 10)
    P = rng.normal(0.0, 0.05, size=(V, 16))
    Q = rng.normal(0.0, 0.05, size=(16, d))
    N = rng.normal(0.0, 0.01, size=(V, d))
    sigma = channel_sigmas(_rng(seed, 11), d, 2, 20.0)
    H = hidden_states(_rng(seed, 12), 512, sigma)
    X = to_bf16_bits(hidden_states(_rng(seed, 13), c["M"], sigma))
    return {"W": P @ Q + N, "H": H, "X": X, "sigma": sigma, **c}


def dense_head(V: int, d: int, rank: int, n_calib: int, seed: int = _BASE_SEED,
               n_outliers: int = 4, outlier_factor: float = 20.0) -> dict:
    """A dense head and calibration states of any shape, drawn like the tiny
    configuration: W = P Q + N with P (V x rank), Q (rank x d) ~ N(0, 0.05^2)
    and N ~ N(0, 0.01^2); n_calib calibration rows with one anisotropic
    channel-sigma vector (n_outliers outlier channels)."""
    rng = _rng(seed, 20)
    P = rng.normal(0.0, 0.05, size=(V, rank))
    Q = rng.normal(0.0, 0.05, size=(rank, d))
    W = P @ Q
    W += rng.normal(0.0, 0.01, size=(V, d))
    sigma = channel_sigmas(_rng(seed, 21), d, n_outliers, outlier_factor)
    H = hidden_states(_rng(seed, 22), n_calib, sigma)
    return {"W": W, "H": H, "V": V, "d": d}


def make_config(name: str, M: int | None = None) -> dict:
    """Inputs of one named configuration.

    For every config but "tiny" this returns packed fields + X.  Configs
    qwen_m1 / qwen_m32 / qwen_m2048 share the same head (same seed) and differ
    only in X; so do the two sizes of each baseline head.  For "tiny" it returns W, H, X (the oracle packs them).
    """
    c = dict(CONFIGS[name])
    if M is not None:
        c["M"] = M
    cfg_id = CONFIG_ORDER.index(name)
    if name == "tiny":
        out = tiny_dense(_BASE_SEED + cfg_id)
        if M is not None and M != out["X"].shape[0]:
            out["X"] = to_bf16_bits(hidden_states(_rng(_BASE_SEED, 14, M), M, out["sigma"]))
            out["M"] = M
        return out
    family = name.rsplit("_m", 1)[0]
    head_seed = _BASE_SEED + _HEAD_FAMILIES.get(family, cfg_id)
    out = random_head(c["V"], c["d"], c["k"], c["r"], c["g"], head_seed)
    if name == "large_m8":
        X = random_x(c["M"], c["d"], _BASE_SEED + cfg_id, n_outliers=8, outlier_factor=30.0)
    else:
        X = random_x(c["M"], c["d"], _BASE_SEED + cfg_id)
    out["X"] = X
    out["M"] = c["M"]
    return out


def random_small_head(V: int, d: int, k: int, r: int, g: int, M: int, seed: int,
                      n_outliers: int = 0, outlier_factor: float = 1.0) -> dict:
    """Random packed head + X at an arbitrary (small) shape, same distributions
    as the large configs.  Used for ragged-shape and edge-case tests."""
    out = random_head(V, d, k, r, g, seed)
    out["X"] = random_x(M, d, seed + 1, n_outliers, outlier_factor)
    out["M"] = M
    return out

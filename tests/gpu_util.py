"""Helpers shared by the GPU tests: running the HIP path through the C ABI and
judging it against the oracle with the acceptance rule of the packed head:
fp32 logits within 2e-3 x the per-row RMS of the fp64 oracle logits, argmax
bit-exact except at near-ties within that same tolerance."""
import sys

import numpy as np

TOL = 2e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_forward(head, X_bits, path="auto", want_logits=True, want_argmax=True):
    import torch
    from packed_quantized_lm_amd import x_tensor_from_bits
    X = x_tensor_from_bits(X_bits)
    logits, arg = head.forward(X, want_logits=want_logits, want_argmax=want_argmax, path=path)
    torch.cuda.synchronize()
    return (None if logits is None else logits.cpu().numpy(),
            None if arg is None else arg.cpu().numpy().astype(np.int64))


def row_rms(y):
    return np.sqrt(np.mean(np.square(y), axis=1))


def assert_logits_close(gpu, ref, rms=None, tol=TOL, what=""):
    rms = row_rms(ref) if rms is None else rms
    err = np.abs(gpu.astype(np.float64) - ref).max(axis=1)
    bound = np.maximum(tol * rms, 1e-30)
    ratio = err / bound
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite logits"
    assert np.all(ratio <= 1.0), f"{what}: max|d|/(2e-3 rms) = {ratio.max():.3g} at row {ratio.argmax()}"
    return float(ratio.max())


def assert_argmax_ok(gpu_arg, gpu_logits, ref, rms=None, tol=TOL, cols=None, what=""):
    """gpu_arg must be the first argmax of the GPU's own logits (bit-exact); against
    the oracle it must agree except where the oracle gap is within tolerance.
    cols maps the columns of ref to vocabulary indices when ref is a sample."""
    if gpu_logits is not None:
        assert np.array_equal(gpu_arg, np.argmax(gpu_logits, axis=1)), f"{what}: argmax != first argmax of logits"
    rms = row_rms(ref) if rms is None else rms
    if cols is None:
        ora = np.argmax(ref, axis=1)
        for m in range(ref.shape[0]):
            if gpu_arg[m] != ora[m]:
                gap = ref[m, ora[m]] - ref[m, gpu_arg[m]]
                assert gap <= tol * rms[m], f"{what}: row {m}: argmax {gpu_arg[m]} vs {ora[m]}, gap {gap}"
    return True

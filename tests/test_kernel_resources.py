"""Resources of the streaming kernels, checked at compile time on the CPU.
Single-launch decode: every instance the library offers must run without
scratch memory (the library refuses an instance that spills, so a spill
would silently take a path away), at two waves per SIMD.  Batched decode:
no scratch memory and no full memory wait inside the stream."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "packed_quantized_lm_amd", "csrc")


def _compile(src, asm=False):
    """(resource usage per kernel, device assembly or None) of one source."""
    from packed_quantized_lm_amd import build as b
    hipcc = os.path.join(b.ROCM, "bin", "hipcc")
    if not os.path.exists(hipcc) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    out_args = ["--cuda-device-only", "-S", "-o", "-"] if asm else ["-c", "-o", os.devnull]
    cmd = [hipcc, *b.HIP_FLAGS, f"-I{b.INCLUDE}", f"-I{CSRC}", os.path.join(CSRC, src), *out_args,
           "-Rpass-analysis=kernel-resource-usage"]
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, check=True)
    usage, name = {}, None
    for line in (p.stderr + "\n" + (p.stdout if not asm else "")).splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            usage[name] = {}
            continue
        m = re.search(r"remark: +([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+)", line)
        if m and name:
            usage[name][m.group(1).strip()] = int(m.group(2))
    return usage, (p.stdout if asm else None)


def test_single_launch_decode_instances_do_not_spill():
    usage, _ = _compile("decode.hip")
    kernels = {n: u for n, u in usage.items() if "gemv_decode_kernel" in n}
    assert len(kernels) == 4, sorted(usage)
    for n, u in kernels.items():
        assert u.get("ScratchSize", -1) == 0, f"{n} spills: {u}"
        assert u.get("Occupancy", 0) >= 2, f"{n}: {u}"


def test_batched_decode_instances_keep_their_prefetches_in_flight():
    """The batched-decode kernel (vtile2.hip) streams with a fixed number of
    chunk loads in flight; its explicit partial waits assume that nothing
    else drains them.  Every instance must run without scratch memory (whose
    reloads would draw waits into the stream) and, after its first barrier
    (the end of the staging), must contain no full wait for every vector
    memory access (s_waitcnt vmcnt(0)): a load whose first use follows it at
    once -- such as a scale read from global memory at a group's start --
    would place one there and empty the prefetch queue."""
    usage, asm = _compile("vtile2.hip", asm=True)
    kernels = {n: u for n, u in usage.items() if "vtile_stream2_kernel" in n}
    assert len(kernels) == 8, sorted(usage)
    for n, u in kernels.items():
        assert u.get("ScratchSize", -1) == 0, f"{n} spills: {u}"
    bodies = re.findall(r"^(_Z\w*vtile_stream2_kernel\w*):(.*?)\.end_amdhsa_kernel", asm, re.S | re.M)
    assert len(bodies) == 8, [b[0] for b in bodies]
    for name, body in bodies:
        after = body.split("s_barrier", 1)
        assert len(after) == 2, f"{name}: no barrier"
        waits = re.findall(r"s_waitcnt vmcnt\(0\)", after[1])
        assert not waits, f"{name}: {len(waits)} full vmcnt waits after the staging barrier"

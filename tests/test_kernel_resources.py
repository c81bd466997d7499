"""Register budget of the single-launch decode kernel, checked at compile
time on the CPU: every instance the library offers must run without
scratch memory (the library refuses an instance that spills, so a spill
would silently take a path away), at two waves per SIMD."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "packed_quantized_lm_amd", "csrc")


def _resource_usage(src):
    from packed_quantized_lm_amd import build as b
    hipcc = os.path.join(b.ROCM, "bin", "hipcc")
    if not os.path.exists(hipcc) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    cmd = [hipcc, *b.HIP_FLAGS, f"-I{b.INCLUDE}", f"-I{CSRC}", "-c", os.path.join(CSRC, src), "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage"]
    out = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, check=True).stdout
    usage, name = {}, None
    for line in out.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            usage[name] = {}
            continue
        m = re.search(r"remark: +([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+)", line)
        if m and name:
            usage[name][m.group(1).strip()] = int(m.group(2))
    return usage


def test_single_launch_decode_instances_do_not_spill():
    usage = _resource_usage("decode.hip")
    kernels = {n: u for n, u in usage.items() if "gemv_decode_kernel" in n}
    assert len(kernels) == 4, sorted(usage)
    for n, u in kernels.items():
        assert u.get("ScratchSize", -1) == 0, f"{n} spills: {u}"
        assert u.get("Occupancy", 0) >= 2, f"{n}: {u}"

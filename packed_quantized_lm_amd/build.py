"""Build libarchead.so (the C-ABI library) in-tree for gfx950.

Every .hip file under csrc/ is compiled with hipcc for --offload-arch=gfx950;
the host-only .cpp files with amdclang++; the objects are linked into
packed_quantized_lm_amd/libarchead.so.  Objects go to _build/ at the repo
root.  Run as `python -m packed_quantized_lm_amd.build`.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libarchead.so")
BUILD = os.path.join(ROOT, "_build")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             # packed fp32 VALU ops stay off: the kernels are written for the
             # scalar fp32 forms only
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-munsafe-fp-atomics", "-Wno-unused-result"]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include"]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    cxx = os.path.join(ROCM, "llvm", "bin", "clang++")
    jobs = []
    for src in sources():
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        inc = [f"-I{INCLUDE}", f"-I{CSRC}"]
        if src.endswith(".hip"):
            cmd = [hipcc, *HIP_FLAGS, *inc, "-c", src, "-o", obj]
        else:
            cmd = [cxx, *CXX_FLAGS, *inc, "-c", src, "-o", obj]
        jobs.append((cmd, obj))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for out in ex.map(lambda j: _run(j[0]), jobs):
            if verbose and out.strip():
                print(out)
    tmp = OUT + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *[o for _, o in jobs],
          "-o", tmp, f"-L{ROCM}/lib", "-lamdhip64", "-lpthread"])
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

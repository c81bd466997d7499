"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

Two drivers in tests/sanitize/ are built with the sanitizers and run:
- host_abi_driver.cpp over the library's host code (api.cpp, pack.cpp and
  the host side of every .hip file, sanitised on the host only): valid
  shapes from one v-block to ragged multi-chunk heads go through the whole
  relayout of archead_pack_load, which then fails at its first device call;
  bad arguments and bogus handles must be refused with the documented
  status; every buffer is exactly sized, so a read or write past an end
  aborts the run;
- naive_driver.c over the oracle's C triple loop (oracle/naive.c).
Any sanitizer report fails the test.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "packed_quantized_lm_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")

pytestmark = pytest.mark.slow


def _run(cmd, **kw):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    assert p.returncode == 0, f"{' '.join(cmd[:3])} ... failed ({p.returncode}):\n{p.stdout[-4000:]}"
    return p.stdout


@pytest.fixture(scope="module")
def outdir(tmp_path_factory):
    return str(tmp_path_factory.mktemp("san"))


def test_oracle_c_triple_loop_is_clean(outdir):
    if not shutil.which("gcc"):
        pytest.skip("gcc missing")
    exe = os.path.join(outdir, "naive_san")
    _run(["gcc", "-O1", "-g", "-std=c99", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "naive.c"), os.path.join(SAN, "naive_driver.c"),
          "-o", exe, "-lm"])
    out = _run([exe], env=SAN_ENV)
    assert "0 failure(s)" in out, out


def test_library_host_code_is_clean(outdir):
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    cxx = os.path.join(ROCM, "llvm", "bin", "clang++")
    if not (os.path.exists(hipcc) and os.path.exists(cxx)):
        pytest.skip("ROCm toolchain missing")
    inc = [f"-I{ROOT}/include", f"-I{CSRC}"]
    host_san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    objs, jobs = [], []
    for src in sorted(os.listdir(CSRC)):
        path = os.path.join(CSRC, src)
        obj = os.path.join(outdir, src + ".o")
        if src.endswith(".hip"):
            # the device code is built as usual; the sanitizers go on the host side only
            cmd = [hipcc, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
                   "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                   *[x for f in host_san for x in ("-Xarch_host", f)], *inc, "-c", path, "-o", obj]
        elif src.endswith(".cpp"):
            cmd = [cxx, "-O1", "-g", "-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
                   *host_san, *inc, "-c", path, "-o", obj]
        else:
            continue
        objs.append(obj)
        jobs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
        if len(jobs) >= 4:
            for j in jobs:
                out, _ = j.communicate()
                assert j.returncode == 0, out[-4000:]
            jobs = []
    for j in jobs:
        out, _ = j.communicate()
        assert j.returncode == 0, out[-4000:]
    drv = os.path.join(outdir, "driver.o")
    _run([cxx, "-O1", "-g", "-std=c++17", *host_san, *inc, "-c", os.path.join(SAN, "host_abi_driver.cpp"),
          "-o", drv])
    exe = os.path.join(outdir, "host_abi_san")
    _run([cxx, *host_san, drv, *objs, f"-L{ROCM}/lib", "-lamdhip64", "-lpthread", f"-Wl,-rpath,{ROCM}/lib",
          "-o", exe])
    out = _run([exe], env=SAN_ENV, timeout=600)
    assert "0 failure(s)" in out, out

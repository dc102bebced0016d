"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU needed).

Every source under csrc/ is compiled with FA_DEBUG defined and the sanitizers on
its host side only (device code is never instrumented), and linked with
tests/asan/host_checks.cpp into one program. The program drives the argument
checks of the entry points, the size and split functions and
fa_check_cu_seqlens over 4,000+ cases, each with arrays in heap blocks of
exactly their size, and compares every status with the documented one; a read
or write past a block, or undefined behaviour, ends it with a sanitizer report.
The build is kept under exact_io_aware_12_amd/_build/asan and redone when a
source changes.
"""
import hashlib
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_io_aware_12_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HARNESS = os.path.join(ROOT, "tests", "asan", "host_checks.cpp")
OUT = os.path.join(ROOT, "exact_io_aware_12_amd", "_build", "asan")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

# host-side sanitizer flags for hipcc: each one behind -Xarch_host, so the
# device code is compiled exactly as in the release library
HOST_SAN = ["-Xarch_host", "-g", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
HIP_FLAGS = ["--offload-arch=gfx950", "-std=c++17", "-O1", "-fPIC", "-DFA_DEBUG",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", INCLUDE, "-I", CSRC] + HOST_SAN
CXX_SAN = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined"]


def _tools():
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    clangxx = os.path.join(ROCM, "llvm", "bin", "clang++")
    if not (os.path.exists(hipcc) and os.path.exists(clangxx)):
        pytest.skip("the ROCm toolchain (hipcc, clang++) is not installed")
    return hipcc, clangxx


def _sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".h")))


def _stamp():
    h = hashlib.sha256()
    for p in _sources() + [os.path.join(INCLUDE, "fa.h"), HARNESS]:
        h.update(p.encode())
        h.update(open(p, "rb").read())
    h.update(" ".join(HIP_FLAGS + CXX_SAN).encode())
    return h.hexdigest()


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")


def build_host_checks():
    """The sanitized program, rebuilt when a source or flag changed."""
    hipcc, clangxx = _tools()
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "host_checks")
    stamp_file = os.path.join(OUT, "stamp")
    stamp = _stamp()
    if os.path.exists(exe) and os.path.exists(stamp_file) and open(stamp_file).read() == stamp:
        return exe
    srcs = sorted((s for s in _sources() if s.endswith(".hip")), key=os.path.getsize,
                  reverse=True)
    objs = [os.path.join(OUT, os.path.basename(s) + ".o") for s in srcs]
    jobs = [[hipcc] + HIP_FLAGS + ["-c", s, "-o", o] for s, o in zip(srcs, objs)]
    hobj = os.path.join(OUT, "host_checks.o")
    jobs.append([clangxx, "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", "-I",
                 os.path.join(ROCM, "include"), "-I", INCLUDE] + CXX_SAN +
                ["-c", HARNESS, "-o", hobj])
    with ThreadPoolExecutor(min(len(jobs), os.cpu_count() or 1, 8)) as ex:
        list(ex.map(_run, jobs))
    _run([clangxx] + CXX_SAN + objs + [hobj, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                                       "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe])
    with open(stamp_file, "w") as f:
        f.write(stamp)
    return exe


def test_host_code_under_address_sanitizer():
    exe = build_host_checks()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "host checks ok:" in r.stdout, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]

"""Build libfa.so in-tree with hipcc for gfx950.

    python exact_io_aware_12_amd/build.py [--resource-usage] [-v]

(run as a script: importing the package itself loads the library).

Compiles every HIP source under csrc/ into exact_io_aware_12_amd/libfa.so.
Packed fp32 VALU instructions are disabled for all device code.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfa.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libfa.so")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only feature flag; that warning is noise
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(line for line in (res.stdout + res.stderr).splitlines() if noise not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    return msgs


def build(resource_usage: bool = False, verbose: bool = False) -> str:
    """Compile every source to an object in parallel (each holds its kernels and
    their launch code, so no device linking is needed), then link libfa.so."""
    from concurrent.futures import ThreadPoolExecutor
    tmpdir = os.path.join(HERE, "_build")
    os.makedirs(tmpdir, exist_ok=True)
    flags = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    if resource_usage:
        flags.insert(0, "-Rpass-analysis=kernel-resource-usage")
    jobs = []
    for src in sources():
        obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
        jobs.append((obj, [hipcc()] + flags + ["-c", src, "-o", obj]))
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(workers) as ex:
        outs = list(ex.map(lambda j: _run(j[1], verbose), jobs))
    tmp = LIB + ".tmp"
    outs.append(_run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] +
                     [o for o, _ in jobs], verbose))
    msgs = "\n".join(m for m in outs if m.strip())
    if msgs.strip() and (verbose or resource_usage):
        print(msgs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(resource_usage="--resource-usage" in sys.argv, verbose="-v" in sys.argv)
    print(LIB)

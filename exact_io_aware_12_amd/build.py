"""Build libfa.so in-tree with hipcc for gfx950.

    python exact_io_aware_12_amd/build.py [--resource-usage] [-v] [--debug | --all]

(run as a script: importing the package itself loads the library).

Compiles every HIP source under csrc/ into exact_io_aware_12_amd/libfa.so;
--debug builds libfa_debug.so instead (the same kernels, with FA_DEBUG defined:
cu_seqlens arguments checked on the host, a synchronisation after every launch),
--all both. Packed fp32 VALU instructions are disabled for all device code.
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
DEBUG_LIB = os.path.join(HERE, "libfa_debug.so")
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


def _jobs(debug: bool, resource_usage: bool):
    """(object, command) per source for one variant, the largest source first."""
    tmpdir = os.path.join(HERE, "_build", "debug" if debug else "")
    os.makedirs(tmpdir, exist_ok=True)
    # host symbols hidden except the C ABI that include/fa.h declares (device
    # code keeps its default visibility: the runtime finds kernels by name)
    flags = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fvisibility=hidden",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    if debug:
        flags.append("-DFA_DEBUG")
    if resource_usage:
        flags.insert(0, "-Rpass-analysis=kernel-resource-usage")
    jobs = []
    for src in sorted(sources(), key=os.path.getsize, reverse=True):
        obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
        jobs.append((obj, [hipcc()] + flags + ["-c", src, "-o", obj]))
    return jobs


def _build_variants(variants, resource_usage: bool = False, verbose: bool = False):
    """Compile every source of every variant (debug flag, library path) to
    objects in one pool (each object holds its kernels and their launch code,
    so no device linking is needed), then link each library."""
    from concurrent.futures import ThreadPoolExecutor
    per = [(lib, _jobs(debug, resource_usage)) for debug, lib in variants]
    jobs = sorted((j for _, js in per for j in js),
                  key=lambda j: os.path.getsize(j[1][-3]), reverse=True)
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(workers) as ex:
        outs = list(ex.map(lambda j: _run(j[1], verbose), jobs))
    for lib, js in per:
        tmp = lib + ".tmp"
        outs.append(_run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] +
                         [o for o, _ in js], verbose))
        os.replace(tmp, lib)
    msgs = "\n".join(m for m in outs if m.strip())
    if msgs.strip() and (verbose or resource_usage):
        print(msgs)
    return [lib for _, lib in variants]


def build(resource_usage: bool = False, verbose: bool = False, debug: bool = False) -> str:
    """Build libfa.so (or, with debug, libfa_debug.so); returns its path."""
    return _build_variants([(debug, DEBUG_LIB if debug else LIB)], resource_usage, verbose)[0]


def build_all(verbose: bool = False):
    """Build libfa.so and libfa_debug.so together; returns both paths."""
    return _build_variants([(False, LIB), (True, DEBUG_LIB)], False, verbose)


if __name__ == "__main__":
    if "--all" in sys.argv:
        print("\n".join(build_all(verbose="-v" in sys.argv)))
    else:
        print(build(resource_usage="--resource-usage" in sys.argv, verbose="-v" in sys.argv,
                    debug="--debug" in sys.argv))

"""Builds libfa.so in-tree for gfx950.

    python -m io_aware_exact_17_amd.build          # or: python io_aware_exact_17_amd/build.py
    python -m io_aware_exact_17_amd.build --paranoid

Every .hip file under csrc/ is compiled with hipcc for gfx950 (packed fp32
instructions disabled), the C ABI (api.cpp) with the host compiler, and the
objects are linked into io_aware_exact_17_amd/libfa.so with an rpath to the
ROCm runtime.  Always rebuilds.

--paranoid builds the race-check variant libfa_paranoid.so: the same sources
with FA_PARANOID_SYNC defined, which drains every memory operation at a
barrier at each LDS stage boundary of the hand-pipelined kernels and uses
full device-scope fences around the decode arrival counters.  Its results
must be bit-identical to the normal build's.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfa.so")
BUILD_PARANOID = os.path.join(PKG, "_build_paranoid")
LIB_PARANOID = os.path.join(PKG, "libfa_paranoid.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-Wno-unused-function",
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-D__HIP_PLATFORM_AMD__"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n  " + " ".join(cmd) + "\n" + out)
    return out


def build(verbose: bool = False, paranoid: bool = False) -> str:
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    out_dir, lib = (BUILD_PARANOID, LIB_PARANOID) if paranoid else (BUILD, LIB)
    os.makedirs(out_dir, exist_ok=True)
    incs = [f"-I{INCLUDE}", f"-I{CSRC}", f"-I{ROCM}/include"]
    defs = ["-DFA_PARANOID_SYNC"] if paranoid else []
    jobs = []
    for f in sorted(os.listdir(CSRC)):
        src = os.path.join(CSRC, f)
        obj = os.path.join(out_dir, f + ".o")
        if f.endswith(".hip"):
            jobs.append([hipcc, *HIP_FLAGS, *defs, *incs, "-c", src, "-o", obj])
        elif f.endswith(".cpp"):
            jobs.append(["g++", *HOST_FLAGS, *incs, "-c", src, "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for out in ex.map(_run, jobs):
            if verbose and out.strip():
                print(out)
    objs = [j[-1] for j in jobs]
    tmp = lib + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp,
          f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"])
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, paranoid="--paranoid" in sys.argv))

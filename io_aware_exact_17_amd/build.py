"""Builds libfa.so in-tree for gfx950.

    python -m io_aware_exact_17_amd.build          # or: python io_aware_exact_17_amd/build.py

Every .hip file under csrc/ is compiled with hipcc for gfx950 (packed fp32
instructions disabled), the C ABI (api.cpp) with the host compiler, and the
objects are linked into io_aware_exact_17_amd/libfa.so with an rpath to the
ROCm runtime.  Always rebuilds.
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


def build(verbose: bool = False) -> str:
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    os.makedirs(BUILD, exist_ok=True)
    incs = [f"-I{INCLUDE}", f"-I{CSRC}", f"-I{ROCM}/include"]
    jobs = []
    for f in sorted(os.listdir(CSRC)):
        src = os.path.join(CSRC, f)
        obj = os.path.join(BUILD, f + ".o")
        if f.endswith(".hip"):
            jobs.append([hipcc, *HIP_FLAGS, *incs, "-c", src, "-o", obj])
        elif f.endswith(".cpp"):
            jobs.append(["g++", *HOST_FLAGS, *incs, "-c", src, "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for out in ex.map(_run, jobs):
            if verbose and out.strip():
                print(out)
    objs = [j[-1] for j in jobs]
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp,
          f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

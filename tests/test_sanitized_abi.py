"""The C ABI's host code (api.cpp: argument checks, sizes, plans) under
AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

api.cpp is compiled with g++ -fsanitize=address,undefined into a scratch
library beside the normal HIP objects; a child process (libasan preloaded,
any sanitizer report fatal) drives every entry point through invalid and
extreme arguments -- null and misaligned pointers, zero, negative and
near-INT_MAX sizes -- and the valid calls that reach the (absent) HIP
runtime.  A signed overflow, out-of-bounds access or use of freed memory in
the host code fails the test.  No GPU is used; skipped where one is present
(the fake device pointers of the valid calls are only safe without one).
"""
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

from conftest import ROOT, gpu_available

PKG = os.path.join(ROOT, "io_aware_exact_17_amd")
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

DRIVER = textwrap.dedent(r'''
    import ctypes, sys
    sys.path.insert(0, sys.argv[2])
    from io_aware_exact_17_amd import SIGNATURES
    lib = ctypes.CDLL(sys.argv[1])
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name); f.restype = res; f.argtypes = args
    A, A2, M = 0x10000, 0x20000, 0x7fffffff
    calls = 0
    def run(fn, *a):
        global calls
        calls += 1
        return getattr(lib, fn)(*a)
    sizes = [0, 1, -1, 7, 63, 64, 65, 255, 256, 257, 8192, 65535, 65536, 1 << 20, M - 1, M, -M]
    for B in (1, 3, M):
        for H in (1, 32, M):
            for N in sizes:
                for d in (64, 128, 96):
                    run("fa_fwd", A, A, A, A2, A2, B, H, N, N, d, 0.1, 1, None)
                    run("fa_fwd", None, A, A, A2, A2, B, H, N, N, d, 0.1, 0, None)
                    run("fa_fwd_f32", A, A, A, A2, A2, B, H, N, 5, d, 0.1, 1, None)
                    run("fa_fwd_block_sparse", A, A, A, A2, A2, A2, B, H, N, N, d, 0.1, 1, None)
                    run("fa_bwd_workspace_bytes", B, H, N)
                    run("fa_bwd", A, A, A, A, A, A2, A2, A2, A2, B, H, N, N, d, 0.1, 1, A, 1 << 40, None)
                    run("fa_decode_split_keys", B, H, d, N)
                    run("fa_decode_workspace_bytes", B, H, d, N)
                    for sk in (0, 64, 100, 1 << 20, M):
                        run("fa_decode_split_workspace_bytes", B, H, d, N, sk)
                        run("fa_decode_varlen_split", A, A, A, A2, A2, A2, A2, B, H, d, N, 0.1, sk,
                            A, 1 << 40, None)
                    run("fa_decode_varlen", A, A, A, A2, A2, A2, A2, B, H, d, N, 0.1, A, 1 << 40, None)
                    run("fa_decode_varlen_noalloc", A, A, A, A2, A2, A2, A2, B, H, d, N, 0.1, None)
                    for page in (1, 3, 16, 65536, M):
                        run("fa_decode_paged_split_keys", B, H, d, N, page)
                        run("fa_decode_paged", A, A, A, A2, A2, A2, A2, B, H, d, page, 100, N, N, 0.1,
                            0, A, 1 << 40, None)
                    run("fa_fwd_varlen", A, A, A, A2, A2, A2, A2, B, H, d, N, N, 0.1, 1, None)
    for s in range(-6, 2):
        run("fa_status_string", s)
    run("fa_probe_read", A, 1 << 20, A2, None)
    run("fa_probe_read", None, 16, A2, None)
    print("calls", calls)
''')


def _san_flags():
    return ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(gpu_available(), reason="valid calls use fake device pointers; CPU only")
def test_host_abi_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    objs = sorted(os.path.join(BUILD, f) for f in os.listdir(BUILD) if f.endswith(".hip.o"))
    assert objs, "build the library first (io_aware_exact_17_amd/build.py)"
    api_o = str(tmp_path / "api_san.o")
    lib = str(tmp_path / "libfa_san.so")
    incs = [f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", f"-I{ROCM}/include"]
    subprocess.run([gxx, "-O1", "-g", "-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__", *_san_flags(),
                    *incs, "-c", os.path.join(CSRC, "api.cpp"), "-o", api_o], check=True)
    subprocess.run([gxx, "-shared", *_san_flags(), api_o, *objs, "-o", lib, f"-L{ROCM}/lib",
                    "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"], check=True)
    asan = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", DRIVER, lib, ROOT], env=env, capture_output=True,
                       text=True, timeout=600)
    report = r.stderr[-4000:]
    assert r.returncode == 0, report
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, report
    assert "calls" in r.stdout

"""The host side of libmoonep under AddressSanitizer (no GPU needed).

Every HIP source is compiled again with the host half instrumented by ASan (the device code is
built as usual), linked into a separate library, and a C driver (tests/capi_asan_driver.c) calls
every entry point with the arguments the header says are rejected on the host: NULL and bad
dims, NULL and misaligned pointers, unsupported flags, workspace sizes over the whole accepted
range.  ASan aborts the driver on any out-of-bounds or use-after-free access of host memory and
reports leaks at exit.
"""
import concurrent.futures
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "balanced_token_dispatch_moonep_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "asan")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]

pytestmark = pytest.mark.slow


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_host_side_under_asan():
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("ROCm compilers not installed")
    rt = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not rt:
        pytest.skip("no ASan runtime")
    rtdir = os.path.dirname(rt[0])
    os.makedirs(OUT, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))

    def compile_one(src):
        obj = os.path.join(OUT, os.path.basename(src)[:-4] + ".o")
        _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_ASAN,
              "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj])
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    lib = os.path.join(OUT, "libmoonep_asan.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-shared-libsan", "-o", lib, *objs])
    drv = os.path.join(OUT, "capi_asan_driver")
    _run([CLANG, "-g", "-fsanitize=address", "-shared-libsan", "-fno-omit-frame-pointer",
          "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "capi_asan_driver.c"),
          "-L", OUT, "-lmoonep_asan", f"-Wl,-rpath,{OUT}", f"-Wl,-rpath,{rtdir}", "-Wl,-rpath,/opt/rocm/lib",
          "-o", drv])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1")
    r = subprocess.run([drv], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and "host checks passed" in r.stdout, r.stdout + r.stderr
    assert "AddressSanitizer" not in r.stderr, r.stderr

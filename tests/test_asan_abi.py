"""The C ABI layer's host code under AddressSanitizer (CPU only): the host
sources of the library are built with -fsanitize=address on their host
pass only (device code is not instrumented), the decode kernels' launchers
replaced by stubs (tests/asan/launch_stubs.cpp), and tests/test_abi.py runs
against that build with the sanitizer runtime preloaded.  Every validation
path of the ABI runs; any out-of-bounds or use-after-free access in the host
code fails the run."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_120_amd", "csrc")
SOURCES = [os.path.join(CSRC, f) for f in
           ("api.cpp", "check.hip", "noalloc.hip", "cache_ops.hip", "probe.hip")]
SOURCES.append(os.path.join(ROOT, "tests", "asan", "launch_stubs.cpp"))


def _tools():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    clang = "/opt/rocm/llvm/bin/clang"
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("hipcc / clang not available")
    rt = subprocess.run([clang, "--print-file-name=libclang_rt.asan-x86_64.so"],
                        capture_output=True, text=True).stdout.strip()
    if not os.path.exists(rt):
        pytest.skip("AddressSanitizer runtime not available")
    return hipcc, rt


def test_abi_under_address_sanitizer(tmp_path):
    hipcc, runtime = _tools()
    lib = str(tmp_path / "libpagedkv_asan.so")
    cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-Xarch_host", "-fsanitize=address",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, *SOURCES, "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_" in syms, "the host code is not instrumented"
    env = dict(os.environ, LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0",
               PAGEDKV_LIBRARY=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "AddressSanitizer" not in out, out[-4000:]

"""The host front end of the boundary (abi.cpp: argument checks, workspace
sizing, symbol exports, status words) under AddressSanitizer.

The host tests of the C ABI (test_abi_host.py) run in a child process against
lib/asan/libmoeq.so, whose abi.cpp is compiled with the sanitizer (host code
only; the kernels are the product build's), with the clang sanitizer runtime
preloaded.  Any sanitizer report fails the test.  No GPU is used."""

import os
import shutil
import subprocess
import sys

import pytest

from quantized_moe_expert_unpack_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_boundary_host_tests_under_address_sanitizer():
    try:
        B._hipcc()
    except RuntimeError:
        pytest.skip("no HIP toolchain to build the sanitized front end")
    rt = B.asan_runtime()
    if rt is None:
        pytest.skip("the toolchain has no AddressSanitizer runtime")
    lib = B.build(verbose=False, asan=True)           # the front end again (seconds)
    if shutil.which("nm"):
        syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
        assert "__asan_" in syms, "the sanitized build carries no sanitizer calls"
    env = dict(os.environ, LD_PRELOAD=rt, MOEQ_LIBRARY=lib, ASAN_OPTIONS="detect_leaks=0")
    probe = subprocess.run([sys.executable, "-c",
                            "from quantized_moe_expert_unpack_amd import moeq; moeq.lib(); print(moeq.LIB_PATH)"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0, probe.stderr[-3000:]
    assert probe.stdout.strip().endswith(os.path.join("asan", "libmoeq.so"))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in r.stderr, out

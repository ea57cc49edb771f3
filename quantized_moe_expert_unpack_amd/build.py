"""Build libmoeq.so (HIP kernels for gfx950 + the C-ABI front end) in-tree.

Usage: ``python -m quantized_moe_expert_unpack_amd.build`` (or call
``build()``).  Every call recompiles every translation unit with hipcc and
links ``quantized_moe_expert_unpack_amd/lib/libmoeq.so``.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libmoeq.so")

ARCH = "gfx950"
SOURCES = ["abi.cpp", "k_matvec.hip", "k_decode.hip", "k_sort.hip", "k_gemm.hip", "k_batch.hip", "k_requant.hip",
           "k_stream.hip"]
# packed fp32 instructions are turned off for all device code
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libmoeq.so")


def _compile(src: str, build_dir: str = BUILD, defines=(), extra=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *FLAGS, *extra, *[f"-D{d}" for d in defines], "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-xhip")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if warn:
        print(f"[{src}]\n{warn}", file=sys.stderr)
    return obj


TIMELINE_LIB = os.path.join(LIBDIR, "timeline", "libmoeq.so")
ASAN_LIB = os.path.join(LIBDIR, "asan", "libmoeq.so")
# host code only: every sanitizer flag goes to the host compilation (the
# device code of the library is compiled as in the product build)
ASAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str | None:
    """The clang AddressSanitizer runtime that a process loading the ASan
    build must preload (None if the toolchain has none)."""
    r = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
        return path
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def build(verbose: bool = True, timeline: bool = False, asan: bool = False) -> str:
    """Build lib/libmoeq.so; with ``timeline`` the instrumented variant
    lib/timeline/libmoeq.so (MOEQ_TIMELINE: the decode kernel records
    per-unit timestamps, read back by ``timeline.py``); with ``asan``
    lib/asan/libmoeq.so, whose host front end (abi.cpp) is built with
    AddressSanitizer (run it with the runtime of ``asan_runtime()`` preloaded
    and MOEQ_LIBRARY pointing at it; the host tests of the boundary do)."""
    build_dir = BUILD + ("_timeline" if timeline else "_asan" if asan else "")
    lib = TIMELINE_LIB if timeline else ASAN_LIB if asan else LIB
    defines = ("MOEQ_TIMELINE",) if timeline else ()
    os.makedirs(build_dir, exist_ok=True)
    os.makedirs(os.path.dirname(lib), exist_ok=True)
    if asan:
        # the front end again with the sanitizer; the kernels' objects of the
        # product build as they are (built first if missing)
        kobjs = [os.path.join(BUILD, os.path.splitext(src)[0] + ".o") for src in SOURCES if not src.endswith(".cpp")]
        if not all(os.path.exists(o) for o in kobjs):
            build(verbose=False)
        objs = [_compile(src, build_dir, defines, ASAN_HOST) for src in SOURCES if src.endswith(".cpp")] + kobjs
    else:
        with ThreadPoolExecutor(max(1, min(len(SOURCES), os.cpu_count() or 1))) as ex:
            objs = list(ex.map(lambda src: _compile(src, build_dir, defines), SOURCES))
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if asan:
        cmd[1:1] = ["-Xarch_host", "-fsanitize=address", "-shared-libasan"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(timeline="--timeline" in sys.argv, asan="--asan" in sys.argv)

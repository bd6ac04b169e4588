"""Builds libspk.so (the C-ABI library of HIP kernels for gfx950) in-tree.

Usage: python -m sparse_top_kv_gqa_amd._build [--verbose]
Each source under csrc/ compiles to an object in _build/ in parallel, then one shared library
is linked next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libspk.so")
OBJ_ASAN = os.path.join(HERE, "_build_asan")
LIB_ASAN = os.path.join(HERE, "libspk_asan.so")
# AddressSanitizer on the host code only (argument validation, planning, launches); the device
# code is built as usual
ASAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libspk)")


FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-Wall",
    "-Wno-unused-function",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str, verbose: bool, asan: bool = False) -> str:
    obj = os.path.join(OBJ_ASAN if asan else OBJ, os.path.basename(src) + ".o")
    cmd = [hipcc()] + FLAGS + (ASAN_HOST if asan else []) + ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, flush=True)
    return obj


def build(verbose: bool = False, asan: bool = False) -> str:
    """Compile every source and link libspk.so (or, with asan, libspk_asan.so: host code under
    AddressSanitizer, loadable with the sanitizer runtime preloaded); returns the path."""
    os.makedirs(OBJ_ASAN if asan else OBJ, exist_ok=True)
    srcs = sources()
    jobs = min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, asan), srcs))
    lib = LIB_ASAN if asan else LIB
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + \
        (["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-shared-libasan"] if asan else []) + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


def asan_runtime() -> str:
    """Path of the host AddressSanitizer runtime of the ROCm toolchain."""
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    return r.stdout.strip()


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv, asan="--asan" in sys.argv))

"""Build the C-ABI shared library libawq_mi355x.so for gfx950 with hipcc.

Every source of the library under csrc/ is compiled as HIP for gfx950 into
_build/, then linked into the package directory, where the Python binding
loads it from.  Packed fp32 VALU instructions are disabled in device code.
A second, separate library, libawq_bench.so (csrc/bench_read.hip: a plain
read stream that the benchmark uses as a same-box reference), is built the
same way; the W4A16 path never loads it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libawq_mi355x.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
BENCH_LIB_PATH = os.path.join(PKG_DIR, "libawq_bench.so")
BENCH_SOURCES = ["bench_read.hip"]
ARCH = "gfx950"

SOURCES = [
    "awq_plan.cpp",
    "awq_api.cpp",
    "awq_dequant.hip",
    "awq_generic.hip",
    "awq_decode.hip",
    "awq_prefill.hip",
    "awq_dense.hip",
    "awq_gidx.hip",
]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build")


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + COMMON_FLAGS + extra
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False, extra_flags: list[str] | None = None, jobs: int = 6) -> str:
    """Compile every HIP source for gfx950 and link the shared library.
    Always recompiles.  Returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    extra = list(extra_flags or [])
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES + BENCH_SOURCES))
    _link(objs[:len(SOURCES)], LIB_PATH, verbose)
    _link(objs[len(SOURCES):], BENCH_LIB_PATH, verbose)
    return LIB_PATH


def _link(objs: list[str], path: str, verbose: bool) -> None:
    tmp = path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, path)
    if verbose:
        print(f"built {path}")


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])

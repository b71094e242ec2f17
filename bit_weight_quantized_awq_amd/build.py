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


# Per-file flags.  The decode kernels are short (about 9 us), so the start
# of every wave counts: their first kernel arguments are preloaded into
# SGPRs at wave launch instead of being fetched from the argument segment by
# the first instructions (a code-object feature of gfx950; the kernel keeps
# a fallback prologue that fetches them itself when the launcher does not
# preload).  Same box, K=8192 N=7168: M=1 9.375 -> 9.316 us, M=16 13.47 ->
# 13.34 us; K=14336 N=4096 M=1 9.566 -> 9.520 us.
FILE_FLAGS = {
    "awq_decode.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=16"],
}


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = ([hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + COMMON_FLAGS +
           FILE_FLAGS.get(src, []) + extra)
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

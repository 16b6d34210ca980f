"""Build libsparse_kv.so (all HIP sources, gfx950) in-tree with hipcc.

Usage: python -m sparse_kv_amd.build   (or call build()).
Objects go to sparse_kv_amd/_build/, the library to sparse_kv_amd/libsparse_kv.so.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc")
INC = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsparse_kv.so")
SOURCES = ["api.hip", "decode.hip", "merge.hip", "select.hip", "art.hip"]
# the benchmark's streaming-read probe, a library of its own
BENCH_LIB = os.path.join(HERE, "libsparse_kv_bench.so")
BENCH_SOURCES = ["bench_read.hip"]
ARCH = "gfx950"

# Packed fp32 VALU ops are kept out of the generated code on purpose.
CFLAGS = [
    "-O3", f"--offload-arch={ARCH}", "-fPIC", "-fvisibility=hidden", "-std=c++17", "-Wall", "-Werror",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INC, "-I", SRC,
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    srcs = SOURCES + BENCH_SOURCES
    objs = [os.path.join(BUILD, s.replace(".hip", ".o")) for s in srcs]

    def compile_one(i):
        out = _run([cc, *CFLAGS, "-c", os.path.join(SRC, srcs[i]), "-o", objs[i]])
        if verbose and out.strip():
            print(out)

    jobs = jobs or min(len(srcs), os.cpu_count() or 1, 16)
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(compile_one, range(len(srcs))))
    for lib, n in ((LIB, len(SOURCES)), (BENCH_LIB, len(BENCH_SOURCES))):
        tmp = lib + ".tmp"
        part = objs[:n] if lib == LIB else objs[len(SOURCES):]
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *part, "-o", tmp])
        os.replace(tmp, lib)
        if verbose:
            print("built", lib)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)

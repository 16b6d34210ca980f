"""The benchmark's probe library (streaming read, empty launch) loads, exports what
include/sparse_kv_bench.h declares, and rejects bad arguments on the host
(CPU only: no call here reaches a launch)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_kv_bench.h")


@pytest.fixture(scope="module")
def blib():
    from sparse_kv_amd import build

    if not os.path.exists(build.BENCH_LIB):
        build.build()
    return ctypes.CDLL(build.BENCH_LIB)


def test_exports_and_validation(blib):
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    names = set(re.findall(r"^\s*int\s+(skv_[a-z_]+)\s*\(", text, flags=re.M))
    assert names == {"skv_bench_stream_read", "skv_bench_empty", "skv_bench_store"}
    st = blib.skv_bench_store
    st.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    st.restype = ctypes.c_int
    assert st(256, None, None) == -1
    assert st(0, ctypes.c_void_p(0x1000), None) == -1
    e = blib.skv_bench_empty
    e.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    e.restype = ctypes.c_int
    assert e(256, None, None) == -1
    assert e(0, ctypes.c_void_p(0x1000), None) == -1
    f = blib.skv_bench_stream_read
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    fake = ctypes.c_void_p(0x1000)
    assert f(None, 1 << 20, 16, fake, None) == -1
    assert f(fake, 1 << 20, 16, None, None) == -1
    assert f(fake, 1 << 20, 0, fake, None) == -1
    assert f(fake, (1 << 20) + 16, 16, fake, None) == -1  # slices must be whole 64 KiB steps
    assert f(fake, 1 << 34, 4, fake, None) == -1  # a slice of 4 GiB is over the 2 GiB range

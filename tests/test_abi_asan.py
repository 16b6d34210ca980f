"""The C-ABI layer (sparse_kv_amd/csrc/api.hip: argument checks, workspace
layouts, the routed layer loop, the static scratch of the workspace-free
routed call) built for the host with the address and undefined-behaviour
sanitizers, linked against recording stand-ins of the kernel launchers
(tests/c/launch_stubs.cpp) and driven from C (tests/c/abi_asan.c).  CPU only."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM_INC = "/opt/rocm/include"


def test_abi_layer_under_host_sanitizers(tmp_path):
    cxx, cc = shutil.which("g++"), shutil.which("gcc")
    if not cxx or not cc or not os.path.isdir(ROCM_INC):
        pytest.skip("needs g++, gcc and the ROCm headers")
    # the layer is plain host code apart from the scratch array's declaration;
    # it is compiled as C++ from a copy named .cpp
    src = tmp_path / "api_host.cpp"
    shutil.copyfile(os.path.join(ROOT, "sparse_kv_amd", "csrc", "api.hip"), src)
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "sparse_kv_amd", "csrc"), "-I", ROCM_INC,
           "-D__HIP_PLATFORM_AMD__", "-D__align__(x)=__attribute__((aligned(x)))", "-DHIP_SYMBOL(x)=x"]
    objs = []
    for name, path in (("api", str(src)), ("stubs", os.path.join(ROOT, "tests", "c", "launch_stubs.cpp"))):
        obj = str(tmp_path / f"{name}.o")
        subprocess.run([cxx, "-std=c++17", "-Wall", "-Werror", *san, *inc, "-c", path, "-o", obj], check=True)
        objs.append(obj)
    main_o = str(tmp_path / "main.o")
    subprocess.run([cc, "-std=c99", "-Wall", "-Werror", *san, "-I", os.path.join(ROOT, "include"), "-c",
                    os.path.join(ROOT, "tests", "c", "abi_asan.c"), "-o", main_o], check=True)
    exe = str(tmp_path / "abi_asan")
    subprocess.run([cxx, *san, main_o, *objs, "-o", exe, "-lpthread"], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip() == "ok", r.stdout + r.stderr

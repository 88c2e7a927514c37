"""The C ABI is usable from plain C: include/moe_ep.h (and the benchmark's
include/moe_streams.h) compile as C99 with warnings as errors, and a C
program linked to the libraries gets the sizes and host-side rejections the
headers document (no GPU needed)."""
import os
import shutil
import subprocess

import pytest

import combine_lds_atomic_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_c_program_against_the_header(tmp_path):
    exe = tmp_path / "c_abi_check"
    libdir = os.path.dirname(moe.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_abi_check.c"), "-o", str(exe), f"-L{libdir}", "-lmoe_ep", "-lmoe_streams",
           f"-Wl,-rpath,{libdir}", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "c abi ok" in r.stdout, r.stdout + r.stderr


@pytest.mark.gpu
@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_c_program_dispatch_and_combine_on_the_gpu(tmp_path):
    """A C program with hipMalloc'd memory runs the four core calls and
    checks the layout, the fp8 round trip and an exactly known combine."""
    exe = tmp_path / "c_abi_gpu"
    libdir = os.path.dirname(moe.LIB_PATH)
    # HIP's own headers are not -pedantic clean in C, so this one goes without it.
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi_gpu.c"), "-o", str(exe),
           f"-L{libdir}", "-lmoe_ep", "-L/opt/rocm/lib", "-lamdhip64", "-lm", f"-Wl,-rpath,{libdir}",
           "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    print("running the C program", flush=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "c abi gpu ok" in r.stdout, r.stdout + r.stderr

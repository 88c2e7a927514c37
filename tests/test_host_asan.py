"""The libraries' host code under AddressSanitizer (no GPU needed): every
source is rebuilt with the host half instrumented (the device code is
built as usual), and the plain-C ABI check (tests/c_abi_check.c: shape
sizing, workspace sizes, argument rejections of every entry point) runs
against those libraries in a program linked with clang's ASan runtime.  Any
out-of-bounds or use-after-free in that host code ends the run with a
report."""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "combine_lds_atomic_amd"))
import build as B  # noqa: E402

CLANG = "/opt/rocm/llvm/bin/clang"
# Host half only: each sanitizer flag follows -Xarch_host.
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not os.path.exists(CLANG) or shutil.which(B.hipcc()) is None and not os.path.exists(B.hipcc()),
                    reason="ROCm clang / hipcc not found")
def test_c_abi_check_under_address_sanitizer(tmp_path):
    cc = B.hipcc()

    def compile_one(src):
        obj = str(tmp_path / src.replace(".hip", ".o"))
        r = subprocess.run([cc, *B.HIPCC_FLAGS, *HOST_ASAN, "-c", os.path.join(B.CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return obj

    with ThreadPoolExecutor(max_workers=5) as ex:
        objs = dict(zip(B.SOURCES + B.STREAMS_SOURCES, ex.map(compile_one, B.SOURCES + B.STREAMS_SOURCES)))
    for name, srcs in (("libmoe_ep.so", B.SOURCES), ("libmoe_streams.so", B.STREAMS_SOURCES)):
        r = subprocess.run([cc, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *[objs[s] for s in srcs], "-o",
                            str(tmp_path / name)], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
    nm = subprocess.run(["nm", "-D", str(tmp_path / "libmoe_ep.so")], capture_output=True, text=True)
    assert "__asan_" in nm.stdout   # the host code is instrumented
    exe = str(tmp_path / "c_abi_check")
    r = subprocess.run([CLANG, "-std=c99", "-Wall", "-Werror", "-fsanitize=address", "-fno-omit-frame-pointer",
                        "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi_check.c"), "-o", exe,
                        f"-L{tmp_path}", "-lmoe_ep", "-lmoe_streams", f"-Wl,-rpath,{tmp_path}",
                        "-Wl,-rpath,/opt/rocm/lib"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    # Leak checking is off: the HIP runtime's own allocations at exit are not this library's.
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=23")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and "c abi ok" in r.stdout, r.stdout + r.stderr[-3000:]
    assert "AddressSanitizer" not in r.stderr, r.stderr[-3000:]

"""Build libmoe_ep.so and libmoe_streams.so (HIP, gfx950) in-tree with hipcc.

Each .hip source is compiled to an object in parallel, then linked into
``combine_lds_atomic_amd/libmoe_ep.so`` (dispatch / combine, include/moe_ep.h)
and ``combine_lds_atomic_amd/libmoe_streams.so`` (the benchmark's plain
streams, include/moe_streams.h).  Usage: ``python
combine_lds_atomic_amd/build.py`` (or ``__graft_entry__.build()``); run it by
path, since importing the package needs a library that exports every
declared symbol.
"""
from __future__ import annotations

import hashlib
import json
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmoe_ep.so")
STREAMS_LIB = os.path.join(PKG, "libmoe_streams.so")
SOURCES = ["abi.hip", "layout.hip", "dispatch.hip", "combine.hip"]
STREAMS_SOURCES = ["streams.hip"]
ARCH = "gfx950"

# -packed-fp32-ops keeps the compiler from emitting packed fp32 VALU ops.
# Code object v5: the HIP runtime that ships with PyTorch (ROCm 7.0) is the one
# loaded in the process, so the device code must be in a version it accepts.
HIPCC_FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-command-line-argument",
               "-mcode-object-version=5",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", f"-I{INCLUDE}", f"-I{CSRC}"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libmoe_ep")


BUILD_INFO = os.path.join(PKG, "build_info.json")


def build(verbose: bool = False, out: str = LIB, extra_flags: list[str] | None = None) -> str:
    """Build libmoe_ep.so at `out` and, beside the default one, libmoe_streams.so
    and build_info.json (the commit and the kernel sources the libraries were
    built from, for the benchmark's record)."""
    lib = _build_lib(SOURCES, out, "obj", verbose, extra_flags)
    if out == LIB:
        _build_lib(STREAMS_SOURCES, STREAMS_LIB, "obj_streams", verbose, extra_flags)
        _write_build_info()
    return lib


def sources_digest() -> str:
    """First 16 hex digits of the SHA-256 of the kernel sources (csrc/, in name order)."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _write_build_info() -> None:
    def git(*args):
        r = subprocess.run(["git", *args], cwd=ROOT, capture_output=True, text=True)
        return r.stdout.strip() if r.returncode == 0 else None
    sha = git("rev-parse", "HEAD")
    status = git("status", "--porcelain", "--", "combine_lds_atomic_amd/csrc", "include")
    info = {"git_sha": sha, "kernel_sources_modified": bool(status) if status is not None else None,
            "sources_digest": sources_digest()}
    with open(BUILD_INFO, "w") as fh:
        json.dump(info, fh)


def _build_lib(sources: list[str], out: str, objsub: str, verbose: bool, extra_flags: list[str] | None) -> str:
    cc = hipcc()
    objdir = os.path.join(ROOT, "_build", objsub)
    os.makedirs(objdir, exist_ok=True)
    flags = HIPCC_FLAGS + list(extra_flags or [])

    def compile_one(src: str) -> str:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [cc, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        objs = list(ex.map(compile_one, sources))
    tmp = out + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

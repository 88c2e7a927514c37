"""Every 16-byte global access of the bulk row kernels is non-temporal.

The row kernels move gigabytes once, and their 16-byte loads and stores are
written with __builtin_nontemporal_load / _store (plain stores measured 3-8%
slower).  The compiler can drop the non-temporal mark when it reshapes the
code around a store (a loop that exits early did this to the receive sum's
output store), so this test compiles the kernel sources to gfx950 assembly
and checks the `nt` bit on every global_load_dwordx4 / global_store_dwordx4 of
every kernel except the routing kernels (tables, not bulk data).  No GPU is
needed."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "combine_lds_atomic_amd"))
import build  # noqa: E402


def _assembly(src: str, out: str) -> str:
    flags = [f for f in build.HIPCC_FLAGS if f != "-fPIC"]
    r = subprocess.run([build.hipcc(), *flags, "--cuda-device-only", "-S", os.path.join(build.CSRC, src), "-o", out],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


@pytest.mark.parametrize("src", ["dispatch.hip", "combine.hip", "streams.hip"])
def test_bulk_accesses_are_nontemporal(src, tmp_path):
    try:
        build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    s = _assembly(src, str(tmp_path / (src + ".s")))
    kernels = 0
    for m in re.finditer(r"^(_ZN\w+): ;", s, re.M):
        name = m.group(1)
        if "k_route_" in name:
            continue
        body = s[m.end():s.index("s_endpgm", m.end())]
        acc = re.findall(r"^\s*(global_(?:load|store)_dwordx4[^\n;]*)", body, re.M)
        plain = [a.strip() for a in acc if not re.search(r"\bnt\b", a)]
        assert not plain, f"{name}: {plain}"
        kernels += 1
    assert kernels >= 3

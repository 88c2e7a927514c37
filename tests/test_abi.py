"""The C-ABI library loads, exports every symbol include/moe_ep.h declares,
and rejects bad arguments on the host (no GPU needed: nothing is launched)."""
import ctypes
import re
import subprocess

import pytest

import combine_lds_atomic_amd as moe


def test_exports_every_declared_symbol():
    declared = moe.declared_symbols()
    assert {"moe_dispatch_send", "moe_dispatch_send_ll", "moe_dispatch_direct", "moe_dispatch_direct_ll", "moe_dispatch_recv", "moe_combine_send",
            "moe_combine_recv", "moe_combine_pull"} <= set(declared)
    for name in declared:
        assert hasattr(moe.lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in nm.splitlines() if " T " in ln}
    assert set(declared) <= exported
    assert not [s for s in exported if s.startswith("moe_") and s not in declared]


def test_library_is_gfx950_code():
    blob = open(moe.LIB_PATH, "rb").read()
    ids = set(re.findall(rb"amdgcn-amd-amdhsa--(gfx\w+)", blob))
    assert ids == {b"gfx950"}, ids


def test_sizes():
    s = moe.shape(16, 128, 2048, 128, 8)
    assert moe.moe_recv_rows(s) == 16 * 128 * 8
    assert moe.moe_recv_rows(moe.shape(16, 128, 2048, 128, 8, region_rows=1000)) == 16000
    ws = moe.moe_workspace_bytes(s)
    assert ws >= 4 * (16 * 128 + 16 * 129 + 16 * 17 + 17 * 128) and ws % 256 == 0
    assert moe.moe_workspace_bytes(moe.shape(8, 0, 128, 8, 1)) > 0


@pytest.mark.parametrize("args,rc", [
    ((0, 128, 2048, 128, 8), -1),        # N < 1
    ((257, 1, 128, 257, 1), -1),          # N above the maximum
    ((16, -1, 2048, 128, 8), -1),         # T < 0
    ((16, 128, 2000, 128, 8), -1),        # H not a multiple of 128
    ((16, 128, 65536, 128, 8), -1),       # H too large
    ((16, 128, 2048, 120, 8), -1),        # E not a multiple of N
    ((16, 128, 2048, 2048, 8), -1),       # E too large
    ((16, 128, 2048, 128, 0), -1),        # k < 1
    ((2, 128, 2048, 4, 5), -1),           # k > E
    ((256, 1 << 20, 128, 256, 16), -4),   # N*T*k overflows int32
])
def test_shape_rejections(args, rc):
    assert moe.lib.moe_recv_rows(ctypes.byref(moe.shape(*args))) == rc


def test_region_rows_rejections():
    assert moe.lib.moe_recv_rows(ctypes.byref(moe.shape(16, 128, 2048, 128, 8, region_rows=-1))) == -1
    assert moe.lib.moe_recv_rows(ctypes.byref(moe.shape(16, 128, 2048, 128, 8, region_rows=1 << 28))) == -4
    bad = moe.shape(16, 128, 2048, 128, 8)
    bad.early_rows = 1                     # early rows need fixed regions
    assert moe.lib.moe_recv_rows(ctypes.byref(bad)) == -1
    assert moe.lib.moe_recv_rows(ctypes.byref(moe.shape(16, 128, 2048, 128, 8, 100, -1))) == -1
    assert moe.lib.moe_recv_rows(ctypes.byref(moe.shape(16, 128, 2048, 128, 8, 100, 7))) == -1   # N*C > R
    assert moe.lib.moe_recv_rows(ctypes.byref(moe.shape(16, 128, 2048, 128, 8, 112, 7))) == 16 * 112


def _p(v):
    return ctypes.c_void_p(v)


def test_null_and_alignment_rejections_happen_on_the_host():
    s = ctypes.byref(moe.shape(4, 8, 256, 8, 2))
    A = 0x10000000   # never dereferenced: every call below fails its host checks first
    lib = moe.lib
    assert lib.moe_dispatch_send(s, _p(A), _p(A), _p(A), _p(A), _p(A), None, None) == -2          # no ws
    assert lib.moe_dispatch_send(s, _p(A), None, _p(A), _p(A), _p(A), _p(A), None) == -2          # no ids
    assert lib.moe_dispatch_send(s, _p(A), _p(A), None, _p(A), _p(A), _p(A), None) == -2          # tokens w/o recv
    assert lib.moe_dispatch_send(s, _p(A + 8), _p(A), _p(A), _p(A), _p(A), _p(A), None) == -3     # tokens not 16-B
    assert lib.moe_dispatch_send(s, _p(A), _p(A), _p(A), _p(A), _p(A), _p(A + 16), None) == -3    # ws not 256-B
    assert lib.moe_dispatch_send_ll(s, _p(A), _p(A), _p(A), _p(A), _p(A), None, None) == -2       # no ws
    assert lib.moe_dispatch_send_ll(s, _p(A), _p(A), None, _p(A), _p(A), _p(A), None) == -2       # tokens w/o recv
    assert lib.moe_dispatch_send_ll(s, _p(A + 8), _p(A), _p(A), _p(A), _p(A), _p(A), None) == -3  # tokens not 16-B
    big = ctypes.byref(moe.shape(2, 513, 256, 8, 8))   # T*k = 4104: more than one routing chunk per rank
    assert lib.moe_dispatch_send_ll(big, _p(A), _p(A), _p(A), _p(A), _p(A), _p(A), None) == -1
    assert lib.moe_dispatch_direct(s, _p(A), _p(A), _p(A), _p(A), _p(A), _p(A), _p(A), None, None) == -2  # no ws
    assert lib.moe_dispatch_direct(s, _p(A), _p(A), _p(A), _p(A), _p(A), None, _p(A), _p(A), None) == -2  # no exp_off
    assert lib.moe_dispatch_direct(s, _p(A), _p(A), _p(A), _p(A), _p(A), _p(A), None, _p(A), None) == -2  # no row_src
    assert lib.moe_dispatch_direct(s, _p(A), _p(A), None, _p(A), _p(A), _p(A), _p(A), _p(A), None) == -2  # tokens w/o x_q
    assert lib.moe_dispatch_direct(s, _p(A + 8), _p(A), _p(A), _p(A), _p(A), _p(A), _p(A), _p(A), None) == -3
    assert lib.moe_dispatch_direct(s, _p(A), _p(A), _p(A + 8), _p(A), _p(A), _p(A), _p(A), _p(A), None) == -3
    assert lib.moe_dispatch_direct(s, _p(A), _p(A), _p(A), _p(A), _p(A), _p(A), _p(A), _p(A + 16), None) == -3
    assert lib.moe_dispatch_direct_ll(s, _p(A), _p(A), _p(A), _p(A), _p(A), _p(A), _p(A), None, None) == -2
    assert lib.moe_dispatch_direct_ll(s, _p(A), _p(A), _p(A), _p(A), _p(A), _p(A), None, _p(A), None) == -2
    assert lib.moe_dispatch_direct_ll(s, _p(A + 8), _p(A), _p(A), _p(A), _p(A), _p(A), _p(A), _p(A), None) == -3
    assert lib.moe_dispatch_direct_ll(big, _p(A), _p(A), _p(A), _p(A), _p(A), _p(A), _p(A), _p(A), None) == -1
    assert lib.moe_dispatch_recv(s, _p(A), _p(A), _p(A), None, _p(A), _p(A), _p(A), None) == -2  # partial payload
    assert lib.moe_dispatch_recv(s, _p(A), _p(A), _p(A), _p(A + 4), _p(A), _p(A), _p(A), None) == -3
    assert lib.moe_combine_send(s, _p(A), _p(A), _p(A), None, None) == -2
    assert lib.moe_combine_send(s, _p(A + 2), _p(A), _p(A), _p(A), None) == -3
    assert lib.moe_combine_recv(s, _p(A), _p(A), None, _p(A), None) == -2
    assert lib.moe_combine_recv(s, _p(A), _p(A), _p(A), _p(A + 8), None) == -3
    assert lib.moe_combine_pull(s, _p(A), _p(A), _p(A), _p(A), None, _p(A), None) == -2     # no ws
    assert lib.moe_combine_pull(s, _p(A), None, _p(A), _p(A), _p(A), _p(A), None) == -2     # no ids
    assert lib.moe_combine_pull(s, _p(A + 8), _p(A), _p(A), _p(A), _p(A), _p(A), None) == -3
    assert lib.moe_combine_send_partial(s, _p(A), _p(A), _p(A), _p(A), None, _p(A), None) == -2   # no ws
    assert lib.moe_combine_send_partial(s, _p(A), _p(A), _p(A), None, _p(A), _p(A), None) == -2   # no weights
    assert lib.moe_combine_send_partial(s, _p(A), _p(A), _p(A), _p(A), _p(A), _p(A + 8), None) == -3
    assert lib.moe_combine_recv_partial(s, _p(A), _p(A), _p(A), None, _p(A), None) == -2          # no ws
    assert lib.moe_combine_recv_partial(s, _p(A), None, _p(A), _p(A), _p(A), None) == -2          # no ids
    assert lib.moe_combine_recv_partial(s, _p(A), _p(A), _p(A), _p(A), _p(A + 2), None) == -3
    fl = ctypes.c_uint32()
    assert lib.moe_status(None, None, ctypes.byref(fl)) == -2
    assert lib.moe_status(_p(A + 4), None, ctypes.byref(fl)) == -3
    assert lib.moe_layout_export(s, None, None, None, None, None, None, None) == -2


def test_streams_library_exports_and_rejections():
    """libmoe_streams (include/moe_streams.h), the benchmark's plain streams,
    is a library of its own: it exports what its header declares, and
    libmoe_ep exports none of it."""
    from combine_lds_atomic_amd import streams as S
    txt = open(S.HEADER).read()
    declared = set(re.findall(r"^\s*int\s+(moe_\w+)\s*\(", txt, re.M))
    assert declared == {"moe_copy", "moe_stream"}
    nm = subprocess.run(["nm", "-D", "--defined-only", S.LIB_PATH], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in nm.splitlines() if " T " in ln}
    assert declared <= exported and not [x for x in exported if x.startswith("moe_") and x not in declared]
    assert not declared & set(moe.declared_symbols())
    A = 0x10000000
    lib = S.lib
    assert lib.moe_copy(_p(A), _p(A), 17, None) == -1
    assert lib.moe_copy(_p(A + 1), _p(A), 16, None) == -3
    assert lib.moe_stream(4, 8, _p(A), _p(A), 16, None) == -1          # no such pattern
    assert lib.moe_stream(0, 8, _p(A), _p(A), 16, None) == -1
    assert lib.moe_stream(1, 0, _p(A), _p(A), 16, None) == -1          # k outside [1, 8]
    assert lib.moe_stream(2, 9, _p(A), _p(A), 16, None) == -1
    assert lib.moe_stream(2, 8, _p(A), _p(A), -1, None) == -1          # negative count
    assert lib.moe_stream(2, 8, _p(A), _p(A), (1 << 40) + 1, None) == -4   # above 2^40 units
    assert lib.moe_stream(1, 8, None, _p(A), 16, None) == -2
    assert lib.moe_stream(1, 8, _p(A), _p(A + 8), 16, None) == -3


def test_noalloc_rejects_shapes_beyond_its_scratch_on_the_host():
    """The no-allocation direct dispatch refuses a shape whose routing tables
    exceed its 32 MiB device array before touching the GPU."""
    A = 0x10000000
    big = moe.shape(256, 16384, 128, 1024, 8)          # 33.5M slots: 4 bytes each of in-chunk ranks alone
    args = [_p(A)] * 7 + [_p(A), None]
    assert moe.lib.moe_dispatch_direct_noalloc(ctypes.byref(big), *args) == -4
    small = moe.shape(4, 8, 256, 8, 2)
    assert moe.lib.moe_dispatch_direct_noalloc(ctypes.byref(small), *([_p(A)] * 7), None, None) == -2   # no flags
    assert moe.lib.moe_dispatch_direct_noalloc(ctypes.byref(small), *([_p(A)] * 7), _p(A + 2), None) == -3

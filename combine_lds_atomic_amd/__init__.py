"""Python binding of libmoe_ep (MoE expert-parallel dispatch / combine on one
MI355X).  Argument marshalling only: every function forwards torch tensors'
device pointers and the current HIP stream to the C ABI of
``include/moe_ep.h`` under the same name; all computation happens in the HIP
kernels.  Importing this module fails loudly if the library is not built.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_EP_LIB selects another build of the same library (e.g. a tuning variant).
LIB_PATH = os.environ.get("MOE_EP_LIB") or os.path.join(PKG, "libmoe_ep.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "moe_ep.h")

MOE_OK = 0
ERRORS = {-1: "MOE_EINVAL", -2: "MOE_ENULL", -3: "MOE_EALIGN", -4: "MOE_ERANGE", -5: "MOE_EHIP"}
FLAG_BADID, FLAG_OVERFLOW, FLAG_BOUND, FLAG_TIMEOUT = 1, 2, 4, 8


class MoeError(RuntimeError):
    def __init__(self, fn: str, rc: int):
        super().__init__(f"{fn} returned {rc} ({ERRORS.get(rc, 'unknown')})")
        self.rc = rc


class moe_shape(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("early_rows", ctypes.c_int32), ("region_rows", ctypes.c_int64)]

    def __repr__(self):
        return (f"moe_shape(N={self.N}, T={self.T}, H={self.H}, E={self.E}, k={self.k}, "
                f"region_rows={self.region_rows}, early_rows={self.early_rows})")


def shape(N: int, T: int, H: int, E: int, k: int, region_rows: int = 0, early_rows: int = 0) -> moe_shape:
    return moe_shape(N, T, H, E, k, early_rows, region_rows)


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python combine_lds_atomic_amd/build.py` "
                      "(or __graft_entry__.build()) first")

# torch ships its own HIP runtime.  It must be in the process before the
# library is opened, so that the library's libamdhip64.so.7 dependency binds to
# that same runtime (by soname) instead of loading a second one: with two
# runtimes the library sees no device and torch's streams mean nothing to it.
import torch  # noqa: E402,F401

lib = ctypes.CDLL(LIB_PATH)


def _hip_runtimes() -> set[str]:
    try:
        maps = open("/proc/self/maps").read()
    except OSError:  # pragma: no cover
        return set()
    return {ln.split()[-1] for ln in maps.splitlines() if "libamdhip64" in ln}


if len(_hip_runtimes()) > 1:
    raise ImportError(f"two HIP runtimes are loaded ({sorted(_hip_runtimes())}); import torch before anything "
                      "that links /opt/rocm's libamdhip64")

_P = ctypes.c_void_p
_S = ctypes.POINTER(moe_shape)
_SIG = {
    "moe_recv_rows": (ctypes.c_int64, [_S]),
    "moe_workspace_bytes": (ctypes.c_int64, [_S]),
    "moe_workspace_init": (ctypes.c_int, [_S, _P, _P]),
    "moe_dispatch_send": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _P]),
    "moe_dispatch_send_ll": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _P]),
    "moe_dispatch_direct": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_dispatch_direct_ll": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_dispatch_direct_noalloc": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_dispatch_recv": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_combine_send": (ctypes.c_int, [_S, _P, _P, _P, _P, _P]),
    "moe_combine_recv": (ctypes.c_int, [_S, _P, _P, _P, _P, _P]),
    "moe_combine_pull": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _P]),
    "moe_combine_send_partial": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _P]),
    "moe_combine_recv_partial": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P]),
    "moe_status": (ctypes.c_int, [_P, _P, ctypes.POINTER(ctypes.c_uint32)]),
    "moe_layout_export": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _P]),
}
for _name, (_res, _args) in _SIG.items():
    _f = getattr(lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def declared_symbols() -> list[str]:
    """Function names declared in include/moe_ep.h."""
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|int64_t)\s+(moe_\w+)\s*\(", txt, re.M)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn: str, rc: int) -> None:
    if rc != MOE_OK:
        raise MoeError(fn, rc)


# --------------------------------------------------------------- sizes

def moe_recv_rows(sh: moe_shape) -> int:
    r = lib.moe_recv_rows(ctypes.byref(sh))
    _check("moe_recv_rows", r if r < 0 else 0)
    return int(r)


def moe_workspace_bytes(sh: moe_shape) -> int:
    r = lib.moe_workspace_bytes(ctypes.byref(sh))
    _check("moe_workspace_bytes", r if r < 0 else 0)
    return int(r)


# --------------------------------------------------------------- entry points

def moe_workspace_init(sh, ws, stream=None):
    _check("moe_workspace_init", lib.moe_workspace_init(ctypes.byref(sh), _ptr(ws), _stream(stream)))


def moe_dispatch_send(sh, tokens, topk_idx, recv_q, recv_s, send_pos, ws, stream=None):
    _check("moe_dispatch_send", lib.moe_dispatch_send(ctypes.byref(sh), _ptr(tokens), _ptr(topk_idx), _ptr(recv_q),
                                                      _ptr(recv_s), _ptr(send_pos), _ptr(ws), _stream(stream)))


def moe_dispatch_send_ll(sh, tokens, topk_idx, recv_q, recv_s, send_pos, ws, stream=None):
    _check("moe_dispatch_send_ll", lib.moe_dispatch_send_ll(ctypes.byref(sh), _ptr(tokens), _ptr(topk_idx),
                                                            _ptr(recv_q), _ptr(recv_s), _ptr(send_pos), _ptr(ws),
                                                            _stream(stream)))


def moe_dispatch_direct(sh, tokens, topk_idx, x_q, x_s, send_pos, exp_off, row_src, ws, stream=None):
    _check("moe_dispatch_direct", lib.moe_dispatch_direct(ctypes.byref(sh), _ptr(tokens), _ptr(topk_idx), _ptr(x_q),
                                                          _ptr(x_s), _ptr(send_pos), _ptr(exp_off), _ptr(row_src),
                                                          _ptr(ws), _stream(stream)))


def moe_dispatch_direct_ll(sh, tokens, topk_idx, x_q, x_s, send_pos, exp_off, row_src, ws, stream=None):
    _check("moe_dispatch_direct_ll", lib.moe_dispatch_direct_ll(ctypes.byref(sh), _ptr(tokens), _ptr(topk_idx),
                                                                _ptr(x_q), _ptr(x_s), _ptr(send_pos), _ptr(exp_off),
                                                                _ptr(row_src), _ptr(ws), _stream(stream)))


def moe_dispatch_direct_noalloc(sh, tokens, topk_idx, x_q, x_s, send_pos, exp_off, row_src, flags, stream=None):
    _check("moe_dispatch_direct_noalloc", lib.moe_dispatch_direct_noalloc(
        ctypes.byref(sh), _ptr(tokens), _ptr(topk_idx), _ptr(x_q), _ptr(x_s), _ptr(send_pos), _ptr(exp_off),
        _ptr(row_src), _ptr(flags), _stream(stream)))


def moe_dispatch_recv(sh, recv_q, recv_s, ws, x_q, x_s, exp_off, row_src, stream=None):
    _check("moe_dispatch_recv", lib.moe_dispatch_recv(ctypes.byref(sh), _ptr(recv_q), _ptr(recv_s), _ptr(ws),
                                                      _ptr(x_q), _ptr(x_s), _ptr(exp_off), _ptr(row_src),
                                                      _stream(stream)))


def moe_combine_send(sh, y_em, row_src, ws, comb, stream=None):
    _check("moe_combine_send", lib.moe_combine_send(ctypes.byref(sh), _ptr(y_em), _ptr(row_src), _ptr(ws),
                                                    _ptr(comb), _stream(stream)))


def moe_combine_recv(sh, comb, send_pos, topk_w, out, stream=None):
    _check("moe_combine_recv", lib.moe_combine_recv(ctypes.byref(sh), _ptr(comb), _ptr(send_pos), _ptr(topk_w),
                                                    _ptr(out), _stream(stream)))


def moe_combine_pull(sh, y_em, topk_idx, send_pos, topk_w, ws, out, stream=None):
    _check("moe_combine_pull", lib.moe_combine_pull(ctypes.byref(sh), _ptr(y_em), _ptr(topk_idx), _ptr(send_pos),
                                                    _ptr(topk_w), _ptr(ws), _ptr(out), _stream(stream)))


def moe_combine_send_partial(sh, y_em, topk_idx, send_pos, topk_w, ws, comb, stream=None):
    _check("moe_combine_send_partial", lib.moe_combine_send_partial(ctypes.byref(sh), _ptr(y_em), _ptr(topk_idx),
                                                                    _ptr(send_pos), _ptr(topk_w), _ptr(ws),
                                                                    _ptr(comb), _stream(stream)))


def moe_combine_recv_partial(sh, comb, topk_idx, send_pos, ws, out, stream=None):
    _check("moe_combine_recv_partial", lib.moe_combine_recv_partial(ctypes.byref(sh), _ptr(comb), _ptr(topk_idx),
                                                                    _ptr(send_pos), _ptr(ws), _ptr(out),
                                                                    _stream(stream)))


def moe_status(ws, stream=None) -> int:
    fl = ctypes.c_uint32(0)
    _check("moe_status", lib.moe_status(_ptr(ws), _stream(stream), ctypes.byref(fl)))
    return int(fl.value)


def moe_layout_export(sh, ws, cnt=None, send_off=None, recv_off=None, recv_total=None, base=None, stream=None):
    _check("moe_layout_export", lib.moe_layout_export(ctypes.byref(sh), _ptr(ws), _ptr(cnt), _ptr(send_off),
                                                      _ptr(recv_off), _ptr(recv_total), _ptr(base), _stream(stream)))


from .buffers import Buffers, allocate  # noqa: E402  (device-memory plumbing)

"""Binding of libmoe_streams (include/moe_streams.h): the plain streaming
kernels the benchmark times as each phase's achievable rate.  Not part of
dispatch / combine; argument marshalling only."""
from __future__ import annotations

import ctypes
import os

from . import PKG, _check, _ptr, _stream   # torch and the HIP runtime are loaded by the package

LIB_PATH = os.path.join(PKG, "libmoe_streams.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "moe_streams.h")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python combine_lds_atomic_amd/build.py` first")
lib = ctypes.CDLL(LIB_PATH)
lib.moe_copy.restype = ctypes.c_int
lib.moe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
lib.moe_stream.restype = ctypes.c_int
lib.moe_stream.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                           ctypes.c_void_p]

STREAM_FANOUT, STREAM_REDUCE, STREAM_FANOUT_ONESHOT = 1, 2, 3


def moe_copy(dst, src, nbytes: int, stream=None):
    _check("moe_copy", lib.moe_copy(_ptr(dst), _ptr(src), int(nbytes), _stream(stream)))


def moe_stream(pattern: int, k: int, dst, src, n16: int, stream=None):
    _check("moe_stream", lib.moe_stream(int(pattern), int(k), _ptr(dst), _ptr(src), int(n16), _stream(stream)))

"""moe_dispatch_direct_noalloc, the direct dispatch whose routing tables live
in the library's own device array instead of a caller workspace, called
through the C ABI and compared bit for bit with moe_dispatch_direct on the
same inputs: two calls in a row, the second on a smaller problem (the array
keeps the first call's tables), then the full combine-heavy size."""
import ctypes

import numpy as np
import pytest
import torch

import combine_lds_atomic_amd as moe
import workloads as W

pytestmark = pytest.mark.gpu

from gpu_harness import log  # noqa: E402


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t


def _compare(cfg, T, bad_ids=False):
    log(f"noalloc vs direct: {cfg.name} N={cfg.N} T={T} H={cfg.H} E={cfg.E} k={cfg.k} bad_ids={bad_ids}")
    sh = moe.shape(cfg.N, T, cfg.H, cfg.E, cfg.k)
    idx, _ = W.routing(cfg, T)
    if bad_ids:
        idx = idx.copy()
        idx[0, 0, 0] = cfg.E
        idx[cfg.N - 1, T - 1, cfg.k - 1] = -3
    idx_d = torch.from_numpy(idx).cuda()
    x = W.tokens(cfg, "cuda", T)
    ref = moe.allocate(sh, "cuda", combine=False, fill_rows=0x5A)
    moe.moe_dispatch_direct(sh, x, idx_d, ref.x_q, ref.x_s, ref.send_pos, ref.exp_off, ref.row_src, ref.ws)
    ref_flags = moe.moe_status(ref.ws)
    got = moe.allocate(sh, "cuda", combine=False, fill_rows=0x5A)
    flags = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = moe.lib.moe_dispatch_direct_noalloc(ctypes.byref(sh), _p(x), _p(idx_d), _p(got.x_q), _p(got.x_s),
                                             _p(got.send_pos), _p(got.exp_off), _p(got.row_src), _p(flags), st)
    assert rc == 0, rc
    torch.cuda.synchronize()
    for f in ("send_pos", "exp_off", "row_src", "x_q", "x_s"):
        assert torch.equal(_bits(getattr(ref, f)), _bits(getattr(got, f))), f
    assert int(flags.item()) == ref_flags
    assert bool(ref_flags & moe.FLAG_BADID) == bad_ids
    return ref_flags


def test_two_calls_then_full_size():
    big = W.Config("noalloc_big", N=8, T=600, H=1024, E=64, k=8, seed=11)     # T*k = 4800: two routing chunks
    small = W.Config("noalloc_small", N=4, T=50, H=256, E=16, k=4, seed=12)
    _compare(big, big.T, bad_ids=True)
    _compare(small, small.T)                   # smaller, and its error word starts clean
    cfg = W.CONFIGS["combine_heavy"]
    _compare(cfg, cfg.T)


def test_layout_only_and_empty():
    cfg = W.Config("noalloc_layout", N=4, T=33, H=256, E=16, k=4, seed=13)
    sh = moe.shape(cfg.N, cfg.T, cfg.H, cfg.E, cfg.k)
    idx, _ = W.routing(cfg)
    idx_d = torch.from_numpy(idx).cuda()
    ref = moe.allocate(sh, "cuda", payload=False, combine=False, fill_rows=-7)
    got = moe.allocate(sh, "cuda", payload=False, combine=False, fill_rows=-7)
    moe.moe_dispatch_direct(sh, None, idx_d, None, None, ref.send_pos, ref.exp_off, ref.row_src, ref.ws)
    flags = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    moe.moe_dispatch_direct_noalloc(sh, None, idx_d, None, None, got.send_pos, got.exp_off, got.row_src, flags)
    torch.cuda.synchronize()
    for f in ("send_pos", "exp_off", "row_src"):
        assert torch.equal(getattr(ref, f), getattr(got, f)), f
    assert int(flags.item()) == moe.moe_status(ref.ws) == 0
    empty = moe.shape(4, 0, 256, 16, 4)
    eo = torch.full((4, 5), -7, dtype=torch.int32, device="cuda")
    moe.moe_dispatch_direct_noalloc(empty, None, None, None, None, None, eo, None, flags)
    torch.cuda.synchronize()
    assert (eo.cpu() == 0).all() and int(flags.item()) == 0

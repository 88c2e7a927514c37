"""GPU parity of the direct dispatch (moe_dispatch_direct, and its single
launch moe_dispatch_direct_ll: each row stored once, straight at its
expert-major row) against the oracle, and against the two-call dispatch
(moe_dispatch_send + moe_dispatch_recv) bit for bit.

Small shapes compare every element: send_pos, exp_off, the exported tables,
row_src and the whole x_q / x_s arrays, including the rows nobody writes
(they keep the fill pattern).  The full-size workloads compare the integer
outputs and whole arrays with the two-call path, and a sample of rows with
the oracle."""
import zlib

import numpy as np
import pytest
import torch

import combine_lds_atomic_amd as moe
import workloads as W
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

from gpu_harness import (DIRECT_CALLS, check_dispatch_full_size, check_layout, check_same_as_two_calls, log, run_all,  # noqa: E402
                         run_direct)

FILL = 0x5A


@pytest.fixture(autouse=True)
def _announce(request):
    log(f"\n[gpu] {request.node.name}")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _cfg(name, **kw):
    return W.Config(name, seed=zlib.crc32(name.encode()), **kw)


CALLS = DIRECT_CALLS


@pytest.fixture(params=list(CALLS))
def call(request):
    return request.param


def _fits_ll(T, k):
    return T * k <= 4096


def _direct(r, payload=True, fill=FILL, call="direct", B=None):
    return run_direct(r, call, payload, fill, B)


_same_as_two_calls = check_same_as_two_calls


def _check_oracle(r, B2, lay):
    """Every element against the oracle (small shapes)."""
    check_layout(dict(r, B=B2), lay)
    if B2.x_q is None:
        return
    rq, rs = O.dispatch_send(r["x"].float().cpu().numpy(), lay)
    xq, xs, _ = O.dispatch_recv(rq, rs, lay)
    got_q, got_s = B2.x_q.cpu().numpy(), B2.x_s.cpu().numpy()
    erow = lay.em_row[lay.em_row >= 0]
    assert (got_q[erow] == xq[erow]).all(), "x_q"
    assert (got_s[erow].view(np.uint32) == xs[erow].view(np.uint32)).all(), "x_s"
    untouched = np.setdiff1d(np.arange(B2.rows), erow)
    assert (got_q[untouched] == FILL).all(), "x_q rows without a slot were written"
    assert (got_s[untouched] == float(FILL)).all(), "x_s rows without a slot were written"


def _case(cfg, T, region_rows=0, idx=None, w=None, early_rows=0, payload=True, call="direct"):
    if call == "direct_ll" and not _fits_ll(T, cfg.k):
        pytest.skip("the single launch needs T*k <= 4096")
    r = run_all(cfg, T, region_rows, idx=idx, w=w, payload=payload, combine=False, early_rows=early_rows)
    B2 = _direct(r, payload, call=call)
    flags = _same_as_two_calls(r, B2)
    lay = O.layout(r["idx"], cfg.E, cfg.N, region_rows, early_rows)
    _check_oracle(r, B2, lay)
    return r, B2, lay, flags


def test_tiny_config(call):
    _case(W.CONFIGS["tiny"], 128, call=call)


def test_tiny_config_fixed_regions(call):
    cfg = W.CONFIGS["tiny"]
    idx, w = W.routing(cfg, 128)
    R = int(O.layout(idx, cfg.E, cfg.N).recv_total.max()) + 17
    _case(cfg, 128, R, idx=idx, w=w, call=call)


def test_layout_only(call):
    _case(W.CONFIGS["tiny"], 128, payload=False, call=call)


@pytest.mark.parametrize("N,T,H,E,k", [
    (8, 33, 256, 16, 8),        # k = E/N
    (5, 77, 1152, 40, 6),       # 9 scale blocks per row (not whole 16-byte units), ragged
    (4, 20, 256, 64, 12),       # k > 8
    (2, 5, 128, 4, 1),          # one slot per token
    (16, 9, 384, 16, 4),        # one expert per rank
    (3, 1500, 384, 12, 3),      # many tokens, ragged workgroup ranges
    (6, 40, 9216, 24, 4),       # long rows: the pack splits tokens into slices
])
def test_shapes(N, T, H, E, k, call):
    _case(_cfg(f"dd{N}_{T}_{H}_{E}_{k}", N=N, T=T, H=H, E=E, k=k), T, call=call)


def test_bad_ids(call):
    cfg = _cfg("dd_badid", N=4, T=40, H=256, E=16, k=4)
    idx, w = W.routing(cfg, 40)
    idx = idx.copy()
    idx[0, 3, 1] = 16
    idx[2, 7, 0] = -1
    idx[3, 39, 3] = 1 << 30
    flags = _case(cfg, 40, idx=idx, w=w, call=call)[3]
    assert flags & O.FLAG_BADID


def test_fixed_region_overflow(call):
    """The fullest regions drop rows: the same rows are dropped (and the same
    row_src holes left) as by the two-call path."""
    cfg = _cfg("dd_ovf", N=4, T=64, H=256, E=8, k=3)
    idx, w = W.routing(cfg, 64)
    idx = idx.copy()
    idx[:, :, 0] = 0
    R = int(O.layout(idx, cfg.E, cfg.N).recv_total.max()) - 9
    r, B2, lay, flags = _case(cfg, 64, R, idx=idx, w=w, call=call)
    assert flags & O.FLAG_OVERFLOW
    assert ((lay.em_row < 0) & lay.slot_valid).any()


@pytest.mark.parametrize("C,slack", [(20, 40), (20, -3), (56, -2)])
def test_early_rows(C, slack, call):
    """Early rows.  With C = 56 some sources leave early rows unused, so the
    fullest region drops source-major rows while every expert-major row still
    fits: those rows exist with row_src -1 and keep their fill."""
    cfg = _cfg("dd_early", N=8, T=64, H=256, E=32, k=6)
    idx, w = W.routing(cfg, 64)
    over = O.layout(idx, cfg.E, cfg.N, cfg.N * C + 10 ** 6, C).recv_off[:, cfg.N]
    R = int(cfg.N * C + over.max() + slack)
    r, B2, lay, flags = _case(cfg, 64, R, idx=idx, w=w, early_rows=C, call=call)
    if slack < 0:
        assert flags & O.FLAG_OVERFLOW
    if C == 56:
        assert (B2.row_src.cpu().numpy() == -1).sum() == 3


def test_empty_batch(call):
    sh = moe.shape(4, 0, 256, 16, 2)
    B = moe.allocate(sh, "cuda", combine=False)
    B.exp_off.fill_(-5)
    empty_i = torch.empty((4, 0, 2), dtype=torch.int32, device="cuda")
    CALLS[call](sh, None, empty_i, None, None, None, B.exp_off, None, B.ws)
    torch.cuda.synchronize()
    assert (B.exp_off.cpu().numpy() == 0).all()
    assert moe.moe_status(B.ws) == 0


def test_then_combine(call):
    """The direct dispatch's row_src drives the combine exactly as the
    two-call path's does."""
    cfg = W.CONFIGS["tiny"]
    r = run_all(cfg, 128)
    B2 = _direct(r, call=call)
    comb = torch.empty_like(r["B"].comb)
    out = torch.empty_like(r["B"].out)
    comb.view(torch.int16).fill_(0x3F00)
    w_d = torch.from_numpy(np.ascontiguousarray(r["w"], np.float32)).cuda()
    moe.moe_combine_send(r["sh"], r["y"], B2.row_src, B2.ws, comb)
    moe.moe_combine_recv(r["sh"], comb, B2.send_pos, w_d, out)
    torch.cuda.synchronize()
    assert torch.equal(comb.view(torch.int16), r["B"].comb.view(torch.int16))
    assert torch.equal(out.view(torch.int16), r["B"].out.view(torch.int16))


def test_single_launch_workspace_reuse():
    """One workspace through direct_ll, send_ll and direct_ll again with a
    new routing (each call advances the workspace's call number): every
    result equals a fresh workspace's."""
    cfg = _cfg("dd_reuse", N=8, T=96, H=512, E=64, k=6)
    sh = moe.shape(cfg.N, 96, cfg.H, cfg.E, cfg.k)
    Bs = moe.allocate(sh, "cuda", combine=False, fill_rows=FILL)
    for rnd, call in enumerate(["direct_ll", "send_ll", "direct_ll", "direct_ll"]):
        idx, w = W.routing(cfg.with_(seed=cfg.seed + rnd), 96)
        r = run_all(cfg, 96, idx=idx, w=w, combine=False)
        if call == "send_ll":
            idx_d = torch.from_numpy(np.ascontiguousarray(idx, np.int32)).cuda()
            moe.moe_dispatch_send_ll(sh, r["x"], idx_d, Bs.recv_q, Bs.recv_s, Bs.send_pos, Bs.ws)
            torch.cuda.synchronize()
            assert torch.equal(Bs.send_pos, r["B"].send_pos)
            assert torch.equal(Bs.recv_q, r["B"].recv_q)
            assert moe.moe_status(Bs.ws) == 0
            continue
        Bs.x_q.fill_(FILL)
        Bs.x_s.fill_(float(FILL))
        Bs.row_src.fill_(FILL)
        _direct(r, call=call, B=Bs)
        _same_as_two_calls(r, Bs)


# ------------------------------------------------------------------ full size

def _need(gib):
    free, _ = torch.cuda.mem_get_info()
    if free < gib * 2 ** 30:
        pytest.skip(f"needs {gib} GiB of free device memory, {free / 2**30:.0f} GiB free")


def _full(cfg, T, call="direct"):
    """Bit for bit against the two-call path, and every expert-major row
    against the oracle (chunk by chunk on the host)."""
    if call == "direct_ll" and not _fits_ll(T, cfg.k):
        pytest.skip("the single launch needs T*k <= 4096")
    r = run_all(cfg, T, combine=False)
    B2 = _direct(r, call=call)
    _same_as_two_calls(r, B2)
    sh = r["sh"]
    lay = O.layout(r["idx"], sh.E, sh.N)
    check_layout(dict(r, B=B2), lay)
    B2.recv_q = B2.recv_s = None
    check_dispatch_full_size(r, lay, B=B2)


def test_dsv3_decode_full_size(call):
    cfg = W.CONFIGS["dsv3_decode"]
    _full(cfg, cfg.T, call=call)


def test_kimi_dispatch_full_size(call):
    cfg = W.CONFIGS["kimi_skewed"]
    _full(cfg, cfg.T, call=call)


def test_combine_heavy_full_size():
    _need(30)
    cfg = W.CONFIGS["combine_heavy"]
    _full(cfg, cfg.T)


def test_prefill_literal_bound_regions():
    """The prefill chunk with regions of the literal worst-case size N*T*max(k,
    E/N) = 4,194,304 rows each ("Send and receive buffers": the receive
    buffer is sized to that bound), through the direct dispatch, which writes
    the expert-major rows only: 8 such regions of fp8 rows are 240 GB, which
    the two-call path (receive regions and expert-major rows) cannot hold in
    288 GB.  Every integer output and every written row against the oracle."""
    cfg = W.CONFIGS["prefill"]
    N, T, H, E, k = cfg.N, cfg.T, cfg.H, cfg.E, cfg.k
    R = N * T * max(k, cfg.L)
    sh = moe.shape(N, T, H, E, k, R)
    rows = moe.moe_recv_rows(sh)
    need = rows * H + rows * (H // 128) * 4 + rows * 4 + moe.moe_workspace_bytes(sh) + N * T * H * 2
    free, _ = torch.cuda.mem_get_info()
    if free < need + (2 << 30):
        pytest.skip(f"literal-bound regions need {need / 2**30:.1f} GiB of device memory plus 2 GiB of slack, "
                    f"{free / 2**30:.1f} GiB free")
    idx, w = W.routing(cfg, T)
    x = W.tokens(cfg, "cuda", T)
    B = moe.allocate(sh, "cuda", payload=False, combine=False, fill_rows=-7)
    B.x_q = torch.empty((rows, H), dtype=torch.uint8, device="cuda")
    B.x_s = torch.empty((rows, H // 128), dtype=torch.float32, device="cuda")
    idx_d = torch.from_numpy(idx).cuda()
    moe.moe_dispatch_direct(sh, x, idx_d, B.x_q, B.x_s, B.send_pos, B.exp_off, B.row_src, B.ws)
    flags = moe.moe_status(B.ws)
    lay = O.layout(idx, E, N, R)
    assert flags == lay.flags == 0
    assert lay.recv_total.max() <= R
    r = dict(sh=sh, idx=idx, w=w, x=x, B=B)
    check_layout(r, lay)
    check_dispatch_full_size(r, lay)

"""GPU parity of the single-launch dispatch (moe_dispatch_send_ll).

Every case runs the send half in one launch, then the same receive half and
combine as the other parity tests, and is checked twice:
  - against the CPU oracle, every element (bit-exact layout, fp8 bytes and
    scales; combine within the stated tolerance, and bit-exact);
  - bit for bit against the multi-launch moe_dispatch_send on the same
    inputs, including every routing table left in the workspace.
Further cases reuse one workspace across calls with different routings (the
per-call tags must keep every stale value out), re-initialise a workspace for
another shape, and check the host-side rejection of shapes with more than one
routing chunk per rank."""
import zlib

import numpy as np
import pytest
import torch

import combine_lds_atomic_amd as moe
import workloads as W
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

from gpu_harness import check_full, export_layout, log, run_all  # noqa: E402

OUTS = ("send_pos", "recv_q", "recv_s", "x_q", "x_s", "exp_off", "row_src", "comb", "out")


@pytest.fixture(autouse=True)
def _announce(request):
    log(f"\n[gpu] {request.node.name}")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _cfg(name, **kw):
    return W.Config(name, seed=zlib.crc32(name.encode()), **kw)


def _same(a, b, f):
    ta, tb = getattr(a["B"], f), getattr(b["B"], f)
    if ta is None:
        return
    va = ta.view(torch.uint8) if ta.dtype != torch.int32 else ta
    vb = tb.view(torch.uint8) if tb.dtype != torch.int32 else tb
    assert torch.equal(va, vb), f"single launch != multi launch: {f}"


def _case(cfg, T, region_rows=0, idx=None, w=None, full=True, early_rows=0):
    if idx is None:
        idx, w = W.routing(cfg, T)
    r = run_all(cfg, T, region_rows, idx=idx, w=w, single_launch=True, early_rows=early_rows)
    lay = O.layout(r["idx"], cfg.E, cfg.N, region_rows, early_rows)
    assert r["flags"] == lay.flags, (r["flags"], lay.flags)
    assert not r["flags"] & moe.FLAG_TIMEOUT
    if full:
        check_full(r, lay)
    m = run_all(cfg, T, region_rows, idx=r["idx"], w=r["w"], x=r["x"], y=r["y"], early_rows=early_rows)
    assert m["flags"] == r["flags"]
    for f in OUTS:
        _same(r, m, f)
    gl, gm = export_layout(r), export_layout(m)
    for k in gl:
        assert (gl[k] == gm[k]).all(), f"layout table {k}"
    return r, lay


def test_tiny_config():
    _case(W.CONFIGS["tiny"], 128)


def test_dsv3_decode_config():
    _case(W.CONFIGS["dsv3_decode"], 128)


def test_kimi_dispatch_config():
    _case(W.CONFIGS["kimi_skewed"], 128)


@pytest.mark.parametrize("N,T,H,E,k", [
    (8, 512, 640, 64, 8),       # T*k = 4096, the largest single-chunk rank
    (3, 37, 384, 12, 3),        # ragged everything; 3 scale blocks per row
    (1, 1, 128, 1, 1),          # one rank, one token, one expert
    (8, 33, 256, 16, 8),        # k > E/N
    (5, 77, 9216, 40, 6),       # rows longer than one 1024-element pass, ragged
    (256, 3, 128, 512, 4),      # the most ranks: cross-rank scans over 256 sources per column
    (64, 16, 256, 1024, 8),     # the most experts
])
def test_shapes(N, T, H, E, k):
    _case(_cfg(f"ll{N}_{T}_{H}_{E}_{k}", N=N, T=T, H=H, E=E, k=k), T)


def test_no_tokens():
    cfg = _cfg("ll_empty", N=2, T=0, H=256, E=8, k=2)
    r = run_all(cfg, 0, single_launch=True)
    assert r["flags"] == 0
    assert (r["B"].exp_off.cpu().numpy() == 0).all()


def test_skewed_small():
    _case(_cfg("ll_skew", N=8, T=500, H=256, E=48, k=8, skew=True), 500)


def test_all_to_rank0():
    cfg = _cfg("ll_forced", N=8, T=500, H=256, E=64, k=8, forced_rank0=True)
    _, lay = _case(cfg, 500)
    assert lay.recv_total[0] == 8 * 500 * 8


def test_fixed_regions():
    cfg = W.CONFIGS["tiny"]
    idx, w = W.routing(cfg, 128)
    R = int(O.layout(idx, cfg.E, cfg.N).recv_total.max()) + 37
    _case(cfg, 128, R, idx, w)


def test_fixed_region_overflow_matches_multi_launch():
    cfg = _cfg("ll_ovf", N=4, T=64, H=256, E=8, k=2)
    idx, w = W.routing(cfg, 64)
    idx = idx.copy()
    idx[:, :, 0] = 0                                   # everybody's slot 0 -> rank 0
    R = int(O.layout(idx, cfg.E, cfg.N).recv_total.max()) - 5
    r, lay = _case(cfg, 64, R, idx, w, full=False)
    assert r["flags"] & O.FLAG_OVERFLOW
    assert (r["B"].send_pos.cpu().numpy() == lay.send_pos).all()


def _early_region(idx, E, N, C, slack):
    over = O.layout(idx, E, N, N * C + 10 ** 6, C).recv_off[:, N]
    return int(N * C + over.max() + slack)


@pytest.mark.parametrize("name,C", [("tiny", 1), ("tiny", 48), ("tiny", 200), ("dsv3_decode", 40),
                                    ("kimi_skewed", 16)])
def test_early_rows(name, C):
    """Early rows: the packers of most rows need only their own rank's count."""
    cfg = W.CONFIGS[name]
    idx, w = W.routing(cfg, 128)
    _case(cfg, 128, _early_region(idx, cfg.E, cfg.N, C, 5), idx, w, early_rows=C)


def test_early_rows_overflow():
    cfg = _cfg("ll_early_ovf", N=4, T=64, H=256, E=8, k=2)
    idx, w = W.routing(cfg, 64)
    idx = idx.copy()
    idx[:, :, 0] = 0
    C = 8
    r, _ = _case(cfg, 64, _early_region(idx, cfg.E, cfg.N, C, -6), idx, w, full=False, early_rows=C)
    assert r["flags"] & O.FLAG_OVERFLOW


def test_bad_ids():
    cfg = _cfg("ll_badid", N=4, T=40, H=256, E=16, k=4)
    idx, w = W.routing(cfg, 40)
    idx = idx.copy()
    idx[0, 3, 1] = 16
    idx[2, 7, 0] = -1
    idx[3, 39, 3] = 1 << 30
    r, _ = _case(cfg, 40, idx=idx, w=w)
    assert r["flags"] & O.FLAG_BADID


def test_reused_workspace_takes_only_current_values():
    """One workspace, many calls: each call's routing differs, so a value left
    by an earlier call (an older tag) would show up as a wrong position."""
    cfg = _cfg("ll_reuse", N=8, T=96, H=512, E=32, k=4)
    sh = moe.shape(cfg.N, 96, cfg.H, cfg.E, cfg.k)
    B = moe.allocate(sh, "cuda", combine=False)
    x = W.tokens(cfg, "cuda", 96)
    cases = []
    for seed in range(3):
        c = cfg.with_(seed=cfg.seed + seed)
        idx, _ = W.routing(c, 96)
        lay = O.layout(idx, cfg.E, cfg.N)
        rq, rs = O.dispatch_send(x.float().cpu().numpy(), lay)
        cases.append((torch.from_numpy(idx).cuda(), lay, rq, rs))
    for call in range(9):
        idx_d, lay, rq, rs = cases[call % 3] if call % 4 != 3 else cases[(call + 1) % 3]
        send = moe.moe_dispatch_send if call == 4 else moe.moe_dispatch_send_ll   # mixed on one workspace
        B.recv_q.fill_(0x5A)
        send(sh, x, idx_d, B.recv_q, B.recv_s, B.send_pos, B.ws)
        moe.moe_dispatch_recv(sh, B.recv_q, B.recv_s, B.ws, B.x_q, B.x_s, B.exp_off, B.row_src)
        assert moe.moe_status(B.ws) == 0, call
        assert (B.send_pos.cpu().numpy() == lay.send_pos).all(), call
        rows = lay.recv_row[lay.recv_row >= 0]
        got = B.recv_q.cpu().numpy()
        assert (got[rows] == rq[rows]).all(), call
        assert (B.recv_s.cpu().numpy()[rows].view(np.uint32) == rs[rows].view(np.uint32)).all(), call
        assert (B.exp_off.cpu().numpy() == lay.exp_off).all(), call


def test_reinitialised_workspace_for_another_shape():
    big = moe.shape(8, 128, 256, 32, 8)
    small_cfg = _cfg("ll_small", N=4, T=50, H=256, E=16, k=3)
    ws = torch.empty(moe.moe_workspace_bytes(big), dtype=torch.uint8, device="cuda")
    moe.moe_workspace_init(big, ws)
    bcfg = _cfg("ll_big", N=8, T=128, H=256, E=32, k=8)
    Bb = moe.allocate(big, "cuda", combine=False)
    idx_b, _ = W.routing(bcfg, 128)
    xb = W.tokens(bcfg, "cuda", 128)
    moe.moe_dispatch_send_ll(big, xb, torch.from_numpy(idx_b).cuda(), Bb.recv_q, Bb.recv_s, Bb.send_pos, ws)
    assert moe.moe_status(ws) == 0
    small = moe.shape(4, 50, 256, 16, 3)
    assert moe.moe_workspace_bytes(small) <= ws.numel()
    moe.moe_workspace_init(small, ws)
    Bs = moe.allocate(small, "cuda", combine=False)
    idx_s, _ = W.routing(small_cfg, 50)
    xs = W.tokens(small_cfg, "cuda", 50)
    moe.moe_dispatch_send_ll(small, xs, torch.from_numpy(idx_s).cuda(), Bs.recv_q, Bs.recv_s, Bs.send_pos, ws)
    assert moe.moe_status(ws) == 0
    lay = O.layout(idx_s, 16, 4)
    assert (Bs.send_pos.cpu().numpy() == lay.send_pos).all()
    rq, rs = O.dispatch_send(xs.float().cpu().numpy(), lay)
    rows = lay.recv_row[lay.recv_row >= 0]
    assert (Bs.recv_q.cpu().numpy()[rows] == rq[rows]).all()


def test_more_than_one_chunk_per_rank_is_rejected():
    sh = moe.shape(2, 513, 256, 8, 8)       # T*k = 4104 > 4096
    B = moe.allocate(sh, "cuda", combine=False)
    idx = torch.zeros((2, 513, 8), dtype=torch.int32, device="cuda")
    x = torch.zeros((2, 513, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError) as e:
        moe.moe_dispatch_send_ll(sh, x, idx, B.recv_q, B.recv_s, B.send_pos, B.ws)
    assert e.value.rc == -1

"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every case compares every output element: small shapes whole arrays at once,
the full-size workloads (in the launch configuration the benchmark times)
chunk by chunk, with the oracle computing each chunk on the host as the test
runs.  Bar: counts, offsets, positions, row_src, fp8 bytes and
fp32 scales bit-exact; combine within 1 bf16 ulp and 2^-7*|ref| + 1e-3 (the
kernel also matches bit for bit)."""
import zlib

import numpy as np
import pytest
import torch

import workloads as W
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

from gpu_harness import (bf16_np, check_combine_full_size, check_combine_out, check_dispatch_full_size,  # noqa: E402
                         check_full, check_layout, log, run_all)


@pytest.fixture(autouse=True)
def _announce(request):
    log(f"\n[gpu] {request.node.name}")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _small(name, **kw):
    return W.Config(name, seed=zlib.crc32(name.encode()), **kw)


def _full_case(cfg, T, region_rows=0, idx=None, w=None, early_rows=0):
    r = run_all(cfg, T, region_rows, idx=idx, w=w, early_rows=early_rows)
    lay = O.layout(r["idx"], cfg.E, cfg.N, region_rows, early_rows)
    assert r["flags"] == lay.flags, (r["flags"], lay.flags)
    check_full(r, lay)
    return r, lay


# ------------------------------------------------------------------ small, whole-buffer parity

def test_tiny_config_packed():
    _full_case(W.CONFIGS["tiny"], 128)


def test_tiny_config_fixed_regions():
    cfg = W.CONFIGS["tiny"]
    idx, w = W.routing(cfg, 128)
    R = int(O.layout(idx, cfg.E, cfg.N).recv_total.max()) + 37
    _full_case(cfg, 128, R, idx, w)


def _early_region(idx, E, N, C, slack):
    """Fixed region rows for early rows C: every sender's early rows plus the
    largest region's further rows, plus `slack` (negative: too small)."""
    over = O.layout(idx, E, N, N * C + 10 ** 6, C).recv_off[:, N]
    return int(N * C + over.max() + slack)


@pytest.mark.parametrize("C", [1, 48, 200])
def test_tiny_config_early_rows(C):
    """Early (private per-sender) rows: C = 1 sends nearly everything through
    the common part, 200 holds every pair's rows privately."""
    cfg = W.CONFIGS["tiny"]
    idx, w = W.routing(cfg, 128)
    _full_case(cfg, 128, _early_region(idx, cfg.E, cfg.N, C, 17), idx, w, early_rows=C)


def test_early_rows_overflow_is_flagged_and_contained():
    cfg = _small("early_ovf", N=4, T=64, H=256, E=8, k=2)
    idx, w = W.routing(cfg, 64)
    idx = idx.copy()
    idx[:, :, 0] = 0                                   # everybody's slot 0 -> rank 0
    C = 8
    R = _early_region(idx, cfg.E, cfg.N, C, -6)
    r = run_all(cfg, 64, R, idx=idx, w=w, combine=False, early_rows=C)
    lay = O.layout(idx, cfg.E, cfg.N, R, C)
    assert r["flags"] & O.FLAG_OVERFLOW and r["flags"] == lay.flags
    B = r["B"]
    assert (B.send_pos.cpu().numpy() == lay.send_pos).all()
    got_rq = B.recv_q.cpu().numpy()
    x = r["x"].float().cpu().numpy()
    q, _ = O.quantize_rows(x.reshape(-1, cfg.H))
    tok = (np.arange(cfg.N)[:, None, None] * 64 + np.arange(64)[None, :, None]) + 0 * idx
    ok = lay.recv_row >= 0
    assert not ok.all()
    assert (got_rq[lay.recv_row[ok]] == q[tok[ok]]).all()
    rs = B.row_src.cpu().numpy()
    want = O.row_src(lay)
    used = O.region_rows_used(lay)
    for d in range(cfg.N):
        a = lay.base[d]
        assert (rs[a:a + used[d]] == want[a:a + used[d]]).all()


def test_literal_bound_regions():
    """Regions sized N*T*max(k, E/N) never overflow."""
    cfg = _small("bound", N=4, T=64, H=256, E=16, k=4)
    _full_case(cfg, 64, cfg.N * 64 * max(cfg.k, cfg.L))


@pytest.mark.parametrize("N,T,H,E,k", [
    (3, 1500, 384, 12, 3),      # 18 routing chunks, ragged last one; 3 scale blocks per row
    (8, 512, 640, 64, 8),       # T*k = 4096: whole chunks only
    (8, 513, 1152, 64, 8),      # 8 slots past whole chunks; 9 scale blocks
    (1, 1, 128, 1, 1),          # one rank, one token, one expert
    (4, 5, 128, 4, 1),          # E = N, k = 1
    (8, 33, 256, 16, 8),        # k > E/N: the bound uses k
    (2, 0, 256, 8, 2),          # no tokens
    (5, 77, 9216, 40, 6),       # H above one 1024-element wave pass, ragged
    (2, 20000, 128, 8, 8),      # 40 chunks of 4096 slots per rank
])
def test_shapes(N, T, H, E, k):
    cfg = _small(f"s{N}_{T}_{H}_{E}_{k}", N=N, T=T, H=H, E=E, k=k)
    _full_case(cfg, T)


@pytest.mark.parametrize("N,T,H,E,k,C", [
    (4, 4100, 1152, 32, 8, 0),   # 72 pieces per row, 56 tokens per chunk, ragged chunks
    (8, 2048, 384, 64, 6, 96),   # fixed regions with early rows
])
def test_large_token_counts(N, T, H, E, k, C):
    """Above 16384 tokens (where the combine kernels switch to their
    cooperative forms), every element checked, packed and with early rows."""
    cfg = _small(f"coop{N}_{T}_{H}", N=N, T=T, H=H, E=E, k=k)
    if C == 0:
        _full_case(cfg, T)
    else:
        idx, w = W.routing(cfg, T)
        _full_case(cfg, T, _early_region(idx, cfg.E, cfg.N, C, 17), idx, w, early_rows=C)


def test_skewed_small():
    cfg = _small("skew", N=8, T=600, H=256, E=48, k=8, skew=True)
    _full_case(cfg, 600)


def test_all_to_rank0_small():
    cfg = _small("forced", N=8, T=700, H=256, E=64, k=8, forced_rank0=True)
    r, lay = _full_case(cfg, 700)
    assert lay.recv_total[0] == 8 * 700 * 8 and (lay.recv_total[1:] == 0).all()


def test_dsv3_decode_config():
    _full_case(W.CONFIGS["dsv3_decode"], 128)


def test_kimi_dispatch_config():
    _full_case(W.CONFIGS["kimi_skewed"], 128)


def test_quantiser_edge_values():
    """All-zero and -0 blocks, bf16 subnormals, huge magnitudes, exact ties."""
    cfg = _small("edge", N=2, T=16, H=1024, E=4, k=2)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 16, 1024)).astype(np.float32)
    x[0, 0, :128] = 0.0
    x[0, 1, 128:256] = -0.0
    x[0, 2, :] = (2.0 ** -133) * rng.integers(-3, 4, 1024)      # subnormal bf16, tiny scale
    x[0, 3, :] = rng.standard_normal(1024) * 1e37                 # near the top of the range
    x[0, 4, :128] = 448.0 * np.arange(128) / 127.0
    x[0, 5, :] = 2.0 ** rng.integers(-130, 120, 1024)              # wide exponent spread
    x[1, 0, :] = np.float32(1.0)
    x[1, 1, :128] = np.float32(-3.0e-39)
    xb = torch.from_numpy(O.bf16_round(x)).to(torch.bfloat16).cuda()
    idx = np.stack([np.stack([rng.choice(4, 2, replace=False) for _ in range(16)]) for _ in range(2)])
    w = np.full((2, 16, 2), 0.5, np.float32)
    r = run_all(cfg, 16, idx=idx, w=w, x=xb)
    lay = O.layout(idx, 4, 2)
    check_full(r, lay)


def test_bad_ids_are_dropped_and_flagged():
    cfg = _small("badid", N=4, T=40, H=256, E=16, k=4)
    idx, w = W.routing(cfg, 40)
    idx = idx.copy()
    idx[0, 3, 1] = 16
    idx[2, 7, 0] = -1
    idx[3, 39, 3] = 1 << 30
    r = run_all(cfg, 40, idx=idx, w=w)
    lay = O.layout(idx, cfg.E, cfg.N)
    assert r["flags"] & O.FLAG_BADID and lay.flags & O.FLAG_BADID
    check_full(r, lay)


@pytest.mark.parametrize("tight", [False, True])
def test_many_rows_short_rows(tight):
    """More than 131072 expert-major rows with short rows: the size from
    which the row kernels switch to their large-problem forms, every element
    checked (with tight fixed regions, the overflow path of those forms)."""
    cfg = _small("many_rows", N=8, T=2100, H=256, E=64, k=8)
    idx, w = W.routing(cfg, 2100)
    R = int(O.layout(idx, cfg.E, cfg.N).recv_total.max()) - 40 if tight else 0
    r = run_all(cfg, 2100, R, idx=idx, w=w)
    lay = O.layout(idx, cfg.E, cfg.N, R)
    assert r["B"].rows >= 131072
    assert bool(r["flags"] & O.FLAG_OVERFLOW) == tight
    check_full(r, lay)


def test_bad_ids_with_several_routing_chunks():
    """T*k > 4096: positions come from chunk bases, and a dropped slot's
    send_pos is still -1."""
    cfg = _small("badid_chunks", N=2, T=700, H=256, E=16, k=8)
    idx, w = W.routing(cfg, 700)
    idx = idx.copy()
    idx[0, 3, 1] = 16
    idx[1, 650, 7] = -1
    idx[1, 699, 0] = 1 << 30
    r = run_all(cfg, 700, idx=idx, w=w)
    lay = O.layout(idx, cfg.E, cfg.N)
    assert r["flags"] & O.FLAG_BADID and lay.flags & O.FLAG_BADID
    assert (lay.send_pos[idx < 0] == -1).all()
    check_full(r, lay)


def test_fixed_region_overflow_is_flagged_and_contained():
    cfg = _small("ovf", N=4, T=64, H=256, E=8, k=2)
    idx, w = W.routing(cfg, 64)
    idx = idx.copy()
    idx[:, :, 0] = 0                                   # everybody's slot 0 -> rank 0
    full = O.layout(idx, cfg.E, cfg.N)
    R = int(full.recv_total.max()) - 5
    r = run_all(cfg, 64, R, idx=idx, w=w, combine=False)
    lay = O.layout(idx, cfg.E, cfg.N, R)
    assert r["flags"] & O.FLAG_OVERFLOW
    B = r["B"]
    # nothing outside [base[d], base[d] + R) -- the arrays hold exactly N*R rows, so
    # the checks are that every written row is where the oracle puts it and the
    # fitting regions are exact.
    got_rq = B.recv_q.cpu().numpy()
    x = r["x"].float().cpu().numpy()
    q, _ = O.quantize_rows(x.reshape(-1, cfg.H))
    tok = (np.arange(cfg.N)[:, None, None] * 64 + np.arange(64)[None, :, None]) + 0 * idx
    ok = lay.recv_row >= 0
    assert (got_rq[lay.recv_row[ok]] == q[tok[ok]]).all()
    fits = np.flatnonzero(full.recv_total <= R)
    gpos = B.send_pos.cpu().numpy()
    assert (gpos == lay.send_pos).all()
    rs = B.row_src.cpu().numpy()
    want = O.row_src(lay)
    for d in fits:
        a = lay.base[d]
        assert (rs[a:a + lay.recv_total[d]] == want[a:a + lay.recv_total[d]]).all()


def test_combine_sums_in_slot_order():
    """Rows of 2^24, 1 and -2^24 whose float32 sum depends on the order of the
    additions (tests/golden/combine_slot_order.json): combine send + recv and
    the pulling combine give the slot-order sums."""
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "combine_slot_order.json")) as f:
        g = json.load(f)
    idx = np.array(g["idx"], np.int32)
    w = np.array(g["w"], np.float32)
    cfg = _small("slot_order", N=g["N"], T=g["T"], H=g["H"], E=g["E"], k=g["k"])
    lay = O.layout(idx, cfg.E, cfg.N)
    vals = np.array(g["y_slot_values"], np.float32)
    y = np.zeros((lay.total_rows, cfg.H), np.float32)
    for s in range(cfg.N):
        for t in range(cfg.T):
            for j in range(cfg.k):
                y[lay.em_row[s, t, j]] = vals[s, t, j]
    y_d = torch.from_numpy(y).to(torch.bfloat16).cuda()
    r = run_all(cfg, cfg.T, idx=idx, w=w, y=y_d, payload=False)
    check_full(r, lay)
    got = O.bf16_from_bits(bf16_np(r["B"].out)).astype(np.float64)
    assert (got == np.array(g["out_slot_order"])[:, :, None]).all()


@pytest.mark.parametrize("region_rows", [0, 700])
def test_combine_reuses_dispatch_buffers(region_rows):
    """Buffers are reused between dispatch and combine: once moe_dispatch_recv
    has run, combine send writes `comb` into the memory that held the fp8
    receive regions, and combine recv writes `out` over the token rows."""
    import combine_lds_atomic_amd as moe
    cfg = _small("reuse", N=4, T=96, H=384, E=16, k=4)
    T = cfg.T
    idx, w = W.routing(cfg, T)
    lay = O.layout(idx, cfg.E, cfg.N, region_rows)
    sh = moe.shape(cfg.N, T, cfg.H, cfg.E, cfg.k, region_rows)
    B = moe.allocate(sh, "cuda", payload=True, combine=False, fill_rows=0x5A)
    rows = B.rows
    comb_bytes = cfg.N * T * cfg.k * cfg.H * 2
    pool = torch.full((max(rows * cfg.H, comb_bytes),), 0x5A, dtype=torch.uint8, device="cuda")
    recv_q = pool[:rows * cfg.H].view(rows, cfg.H)
    x = W.tokens(cfg, "cuda", T)
    x_host = x.float().cpu().numpy()
    idx_d, w_d = torch.from_numpy(idx).cuda(), torch.from_numpy(w).cuda()
    moe.moe_dispatch_send(sh, x, idx_d, recv_q, B.recv_s, B.send_pos, B.ws)
    moe.moe_dispatch_recv(sh, recv_q, B.recv_s, B.ws, B.x_q, B.x_s, B.exp_off, B.row_src)
    comb = pool[:comb_bytes].view(torch.bfloat16).view(cfg.N, T * cfg.k, cfg.H)   # recv_q's memory
    out = x                                                                          # the tokens' memory
    y = W.expert_outputs(cfg, rows, "cuda")
    moe.moe_combine_send(sh, y, B.row_src, B.ws, comb)
    moe.moe_combine_recv(sh, comb, B.send_pos, w_d, out)
    assert moe.moe_status(B.ws) == lay.flags
    rq, rs = O.dispatch_send(x_host, lay)
    xq, xs, rsrc = O.dispatch_recv(rq, rs, lay)
    erow = lay.em_row[lay.em_row >= 0]
    assert (B.x_q.cpu().numpy()[erow] == xq[erow]).all()
    assert (B.x_s.cpu().numpy()[erow].view(np.uint32) == xs[erow].view(np.uint32)).all()
    assert (B.row_src.cpu().numpy()[erow] == rsrc[erow]).all()
    yb = bf16_np(y)
    comb_o = O.combine_send(yb, rsrc, cfg.N, T, cfg.k)
    got_comb = bf16_np(comb).reshape(-1, cfg.H)
    wr = rsrc[rsrc >= 0]
    assert (got_comb[wr] == comb_o[wr]).all()
    check_combine_out(bf16_np(out), O.combine_recv(comb_o, lay.send_pos, w, T, cfg.k))


def test_repeat_runs_are_bitwise_identical():
    cfg = W.CONFIGS["tiny"]
    a = run_all(cfg, 128)
    b = run_all(cfg, 128, idx=a["idx"], w=a["w"], x=a["x"], y=a["y"])
    for f in ("send_pos", "recv_q", "recv_s", "x_q", "x_s", "row_src", "comb", "out"):
        ta, tb = getattr(a["B"], f), getattr(b["B"], f)
        assert torch.equal(ta.view(torch.uint8) if ta.dtype != torch.int32 else ta,
                           tb.view(torch.uint8) if tb.dtype != torch.int32 else tb), f


# ------------------------------------------------------------------ full size, every row

def _need(gib):
    free, _ = torch.cuda.mem_get_info()
    if free < gib * 2 ** 30:
        pytest.skip(f"needs {gib} GiB of free device memory, {free / 2**30:.0f} GiB free")


def _check_full_size(r, lay, payload=True):
    """Every integer output, every receive-region and expert-major row, every
    comb row and every output token, against the oracle computed chunk by
    chunk on the host."""
    check_layout(r, lay)
    log("  layout ok")
    if payload:
        check_dispatch_full_size(r, lay)
        log("  dispatch rows ok")
    check_combine_full_size(r, lay)
    log("  combine rows ok")
    assert torch.equal(r["out_pull"].view(torch.int16), r["B"].out.view(torch.int16)), "pull != send + recv"


def test_combine_heavy_full_size():
    """T=4096, H=7168, E=256, k=8, N=16, packed regions: the benchmarked launch."""
    _need(30)
    cfg = W.CONFIGS["combine_heavy"]
    r = run_all(cfg, cfg.T, fill=None)
    lay = O.layout(r["idx"], cfg.E, cfg.N)
    assert r["flags"] == 0
    _check_full_size(r, lay)


def test_kimi_combine_full_size():
    """Kimi-K2-shaped skew at combine batch 4096: layout-only dispatch, then
    combine; every comb row and output token of all 64 source ranks."""
    _need(70)
    cfg = W.CONFIGS["kimi_skewed"]
    r = run_all(cfg, cfg.Tc, payload=False, fill=None)
    lay = O.layout(r["idx"], cfg.E, cfg.N)
    assert r["flags"] == 0
    _check_full_size(r, lay, payload=False)


@pytest.mark.parametrize("name", ["prefill", "prefill_forced"])
def test_prefill_full_size(name):
    _need(55)
    cfg = W.CONFIGS[name]
    r = run_all(cfg, cfg.T, fill=None)
    lay = O.layout(r["idx"], cfg.E, cfg.N)
    assert r["flags"] == 0
    if cfg.forced_rank0:
        assert lay.recv_total[0] == cfg.N * cfg.T * cfg.k
    _check_full_size(r, lay)

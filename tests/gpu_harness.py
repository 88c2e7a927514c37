"""Helpers shared by the GPU tests: run the four C-ABI calls on seeded inputs
and compare with the oracle.  Nothing here computes expected values itself --
they come from ``oracle`` only."""
from __future__ import annotations

import sys

import numpy as np
import torch

import combine_lds_atomic_amd as moe
import workloads as W
from oracle import moe_oracle as O


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_np(t: torch.Tensor) -> np.ndarray:
    """bfloat16 tensor -> uint16 bit patterns on the host."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def run_all(cfg: W.Config, T: int, region_rows: int = 0, idx=None, w=None, x=None, y=None,
            payload: bool = True, combine: bool = True, fill: int | None = 0x5A, device="cuda",
            single_launch: bool = False, early_rows: int = 0):
    """Generate (or take) inputs and run dispatch send/recv and combine send/recv
    (single_launch: the send half through moe_dispatch_send_ll)."""
    sh = moe.shape(cfg.N, T, cfg.H, cfg.E, cfg.k, region_rows, early_rows)
    if idx is None:
        idx, w = W.routing(cfg, T)
    idx_d = torch.from_numpy(np.ascontiguousarray(idx, np.int32)).to(device)
    w_d = torch.from_numpy(np.ascontiguousarray(w, np.float32)).to(device)
    if x is None and payload:
        x = W.tokens(cfg, device, T)
    B = moe.allocate(sh, device, payload=payload, combine=combine, fill_rows=fill)
    send = moe.moe_dispatch_send_ll if single_launch else moe.moe_dispatch_send
    send(sh, x if payload else None, idx_d, B.recv_q, B.recv_s, B.send_pos, B.ws)
    moe.moe_dispatch_recv(sh, B.recv_q, B.recv_s, B.ws, B.x_q, B.x_s, B.exp_off, B.row_src)
    if combine:
        if y is None:
            y = W.expert_outputs(cfg, B.rows, device)
        if fill is not None:
            B.comb.view(torch.int16).fill_(0x3F00)
        moe.moe_combine_send(sh, y, B.row_src, B.ws, B.comb)
        moe.moe_combine_recv(sh, B.comb, B.send_pos, w_d, B.out)
        out_pull = torch.full_like(B.out, 7.0)
        moe.moe_combine_pull(sh, y, idx_d, B.send_pos, w_d, B.ws, out_pull)
    else:
        out_pull = None
    flags = moe.moe_status(B.ws)
    return dict(sh=sh, idx=np.asarray(idx), w=np.asarray(w), x=x, y=y, B=B, flags=flags, out_pull=out_pull)


def export_layout(r):
    sh, B = r["sh"], r["B"]
    N, E = sh.N, sh.E
    dev = B.ws.device
    t = dict(cnt=torch.empty((N, E), dtype=torch.int32, device=dev),
             send_off=torch.empty((N, E + 1), dtype=torch.int32, device=dev),
             recv_off=torch.empty((N, N + 1), dtype=torch.int32, device=dev),
             recv_total=torch.empty((N,), dtype=torch.int32, device=dev),
             base=torch.empty((N + 1,), dtype=torch.int32, device=dev))
    moe.moe_layout_export(sh, B.ws, **t)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in t.items()}


def check_layout(r, lay: O.Layout):
    """Counts, offsets, positions, exp_off and row_src: bit-exact."""
    g = export_layout(r)
    B = r["B"]
    assert (g["cnt"] == lay.cnt).all(), "cnt"
    assert (g["send_off"] == lay.send_off).all(), "send_off"
    assert (g["recv_off"] == lay.recv_off).all(), "recv_off"
    assert (g["recv_total"] == lay.recv_total).all(), "recv_total"
    assert (g["base"] == lay.base).all(), "base"
    assert (B.send_pos.cpu().numpy() == lay.send_pos).all(), "send_pos"
    assert (B.exp_off.cpu().numpy() == lay.exp_off).all(), "exp_off"
    rs = B.row_src.cpu().numpy()
    want = O.row_src(lay)
    used = O.region_rows_used(lay)
    for d in range(lay.N):
        a, b = lay.base[d], lay.base[d] + used[d]
        assert (rs[a:b] == want[a:b]).all(), f"row_src region {d}"


def check_full(r, lay: O.Layout, check_comb=True):
    """Whole-buffer parity against the oracle (small cases)."""
    check_layout(r, lay)
    B = r["B"]
    sh = r["sh"]
    N, T, H, k = sh.N, sh.T, sh.H, sh.k
    if B.recv_q is not None:
        x = r["x"].float().cpu().numpy()
        rq, rs = O.dispatch_send(x, lay)
        xq, xs, _ = O.dispatch_recv(rq, rs, lay)
        got_rq, got_rs = B.recv_q.cpu().numpy(), B.recv_s.cpu().numpy()
        got_xq, got_xs = B.x_q.cpu().numpy(), B.x_s.cpu().numpy()
        rrow = lay.recv_row[lay.recv_row >= 0]
        erow = lay.em_row[lay.em_row >= 0]
        assert (got_rq[rrow] == rq[rrow]).all(), "recv_q"
        assert (got_rs[rrow].view(np.uint32) == rs[rrow].view(np.uint32)).all(), "recv_s"
        assert (got_xq[erow] == xq[erow]).all(), "x_q"
        assert (got_xs[erow].view(np.uint32) == xs[erow].view(np.uint32)).all(), "x_s"
        # rows nobody writes keep the fill pattern
        untouched = np.setdiff1d(np.arange(B.rows), rrow)
        assert (got_rq[untouched] == 0x5A).all(), "recv_q rows outside the regions were written"
    if check_comb and B.comb is not None:
        y = bf16_np(r["y"])
        rsrc = O.row_src(lay)
        comb = O.combine_send(y, rsrc, N, T, k)
        got_comb = bf16_np(B.comb).reshape(N * T * k, H)
        wr = rsrc[rsrc >= 0]
        assert (got_comb[wr] == comb[wr]).all(), "comb"
        # a valid slot left without a row by a full fixed region: a zero row
        lost = lay.slot_valid & (lay.em_row < 0)
        if lost.any():
            s_, t_, j_ = np.nonzero(lost)
            assert (got_comb[s_ * T * k + lay.send_pos[s_, t_, j_]] == 0).all(), "comb rows of dropped slots"
        out = O.combine_recv(comb, lay.send_pos, r["w"], T, k)
        got_out = bf16_np(B.out)
        check_combine_out(got_out, out)
        check_combine_out(bf16_np(r["out_pull"]), out)     # the pulling combine gives the same bytes


def check_combine_out(got: np.ndarray, ref: np.ndarray):
    """bf16 combine output: the stated tolerance (1 bf16 ulp per element and
    |d| <= 2^-7 |ref| + 1e-3); the kernel also claims bit-exactness (same
    float32 operations in the same order, no FMA)."""
    g = O.bf16_from_bits(got).astype(np.float64)
    f = O.bf16_from_bits(ref).astype(np.float64)
    ulp = np.ldexp(1.0, np.frexp(np.abs(f))[1] - 8)
    d = np.abs(g - f)
    assert (d <= np.maximum(ulp, 2.0 ** -133)).all(), f"combine off by more than 1 ulp: max {d.max()}"
    assert (d <= 2.0 ** -7 * np.abs(f) + 1e-3).all(), "combine outside abs/rel tolerance"
    assert (got == ref).all(), f"combine not bit-exact at {np.count_nonzero(got != ref)} elements"


# ------------------------------------------------------------------ direct dispatch

DIRECT_CALLS = {"direct": moe.moe_dispatch_direct, "direct_ll": moe.moe_dispatch_direct_ll}


def run_direct(r, call="direct", payload=True, fill=0x5A, B=None):
    """The direct dispatch of run_all's inputs into buffers of its own (or B)."""
    sh = r["sh"]
    if B is None:
        B = moe.allocate(sh, r["B"].ws.device, payload=payload, combine=False, fill_rows=fill)
    idx_d = torch.from_numpy(np.ascontiguousarray(r["idx"], np.int32)).to(B.ws.device)
    DIRECT_CALLS[call](sh, r["x"] if payload else None, idx_d, B.x_q, B.x_s, B.send_pos, B.exp_off, B.row_src,
                       B.ws)
    torch.cuda.synchronize()
    return B


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t


def check_same_as_two_calls(r, B2):
    """Every output and workspace table of a direct dispatch (B2) equals the
    two-call path's (r["B"]) bit for bit; returns B2's status word."""
    B1 = r["B"]
    for f in ("send_pos", "exp_off", "row_src", "x_q", "x_s"):
        a, b = getattr(B1, f), getattr(B2, f)
        if a is None:
            assert b is None
            continue
        assert torch.equal(_bits(a), _bits(b)), f
    g1, g2 = export_layout(r), export_layout(dict(r, B=B2))
    for key in g1:
        assert (g1[key] == g2[key]).all(), key
    flags = moe.moe_status(B2.ws)   # read and cleared
    assert flags == r["flags"]
    return flags


# ------------------------------------------------------------------ send-side partial combine

PARTIAL_FILL = 0x3F00


def run_partial(r):
    """Both halves of the partial combine on the buffers of a run_all result."""
    sh, B = r["sh"], r["B"]
    dev = B.ws.device
    idx_d = torch.from_numpy(np.ascontiguousarray(r["idx"], np.int32)).to(dev)
    w_d = torch.from_numpy(np.ascontiguousarray(r["w"], np.float32)).to(dev)
    comb = torch.empty_like(B.comb)
    comb.view(torch.int16).fill_(PARTIAL_FILL)
    out = torch.full_like(B.out, 3.0)
    moe.moe_combine_send_partial(sh, r["y"], idx_d, B.send_pos, w_d, B.ws, comb)
    moe.moe_combine_recv_partial(sh, comb, idx_d, B.send_pos, B.ws, out)
    assert moe.moe_status(B.ws) & moe.FLAG_TIMEOUT == 0
    return comb, out


def partial_bound_check(out_bits, rows_by_slot, w_tok, group_rows):
    """The partial combine's tolerance against the float64 sum, one token."""
    o = O.bf16_from_bits(out_bits).astype(np.float64)
    ww = np.asarray(w_tok, np.float64)[:, None]
    exact = (ww * rows_by_slot).sum(axis=0)
    mag = (np.abs(ww) * np.abs(rows_by_slot)).sum(axis=0)
    pg = sum(np.abs(O.bf16_from_bits(p).astype(np.float64)) for p in group_rows) if group_rows else 0.0
    k = len(w_tok)
    lim = 2.0 ** -8 * (np.abs(o) + pg) + 2 * k * 2.0 ** -24 * mag + 2.0 ** -133
    assert (np.abs(o - exact) <= lim).all()


def check_partial_full(r, lay):
    """Whole-buffer parity of the partial combine against combine_partial:
    group rows at their leaders, untouched rows, the output, and the bound."""
    sh = r["sh"]
    N, T, H, k = sh.N, sh.T, sh.H, sh.k
    comb, out = run_partial(r)
    y = bf16_np(r["y"])
    comb_o, lead, out_o = O.combine_partial(y, r["idx"], lay, r["w"])
    got_comb = bf16_np(comb).reshape(N * T * k, H)
    led = np.zeros(N * T * k, bool)
    for s in range(N):
        for t in range(T):
            for j in np.flatnonzero(lead[s, t]):
                led[s * T * k + lay.send_pos[s, t, j]] = True
    assert (got_comb[led] == comb_o[led]).all(), "group rows"
    assert (got_comb[~led] == PARTIAL_FILL).all(), "rows no group leads were written"
    got_out = bf16_np(out)
    assert (got_out == out_o).all(), f"out differs at {np.count_nonzero(got_out != out_o)} elements"
    yv = O.bf16_from_bits(y).astype(np.float64)
    for s in range(N):
        for t in range(T):
            part = lay.em_row[s, t] >= 0
            rows = np.zeros((k, H))
            rows[part] = yv[lay.em_row[s, t][part]]
            grp = [comb_o[s * T * k + lay.send_pos[s, t, j]] for j in np.flatnonzero(lead[s, t])]
            partial_bound_check(got_out[s, t], rows, np.where(part, r["w"][s, t], 0.0), grp)
    return lead


# ------------------------------------------------------------------ full size, every row

def _workers(per_item_bytes: float) -> int:
    """Host threads for the chunked oracle checks: NumPy releases the GIL in
    its array loops, so the oracle's per-chunk work runs in parallel; bounded
    by the cores and by host memory (per_item_bytes each)."""
    import os
    try:
        import psutil
        avail = psutil.virtual_memory().available
    except Exception:  # pragma: no cover
        avail = 32e9
    budget = min(0.4 * avail, 100e9)
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, cores, int(budget // max(per_item_bytes, 1.0))))


def _pmap(fn, items, per_item_bytes):
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(_workers(per_item_bytes)) as ex:
        for _ in ex.map(fn, items):
            pass


def _rows(t: torch.Tensor, rows: np.ndarray) -> torch.Tensor:
    """Rows `rows` of a device array, gathered on the device and brought to
    the host."""
    return t[torch.from_numpy(np.ascontiguousarray(rows, np.int64)).to(t.device)].cpu()


def check_dispatch_full_size(r, lay: O.Layout, tok_chunk: int = 1024, B=None):
    """Every receive-region row (when B holds them) and every expert-major row
    (fp8 bytes and fp32 scales) against the oracle, chunk by chunk: the
    oracle quantises each chunk of tokens as the check runs (quantize_rows),
    and each quantised row must sit, bit for bit, at every row dispatch_send
    / dispatch_recv (or the direct dispatch) put it (recv_row, em_row of the
    oracle's layout)."""
    sh = r["sh"]
    B = r["B"] if B is None else B
    N, T, H, k = sh.N, sh.T, sh.H, sh.k
    x = r["x"]
    items = [(s, t0) for s in range(N) for t0 in range(0, T, tok_chunk)]
    arrays = [("x", lay.em_row, B.x_q, B.x_s)]
    if B.recv_q is not None:
        arrays.insert(0, ("recv", lay.recv_row, B.recv_q, B.recv_s))

    def one(item):
        s, t0 = item
        t1 = min(T, t0 + tok_chunk)
        q, sc = O.quantize_rows(x[s, t0:t1].float().cpu().numpy())
        for name, rows, gq, gs in arrays:
            rr = rows[s, t0:t1, :]
            ok = rr >= 0
            got_q = _rows(gq, rr[ok]).numpy()
            got_s = _rows(gs, rr[ok]).numpy()
            tok = np.broadcast_to(np.arange(t1 - t0)[:, None], rr.shape)[ok]
            assert (got_q == q[tok]).all(), f"{name}_q rank {s} tokens {t0}..{t1}"
            assert (got_s.view(np.uint32) == sc[tok].view(np.uint32)).all(), f"{name}_s rank {s} tokens {t0}..{t1}"

    _pmap(one, items, tok_chunk * H * (8 + 2 * k * 1.1) + 2 * tok_chunk * H * 8)


def check_combine_full_size(r, lay: O.Layout, ranks=None):
    """Every comb row and every output token of the source ranks `ranks` (all
    by default) against the oracle, one source rank at a time: the oracle's
    combine_send places the expert-major rows that return to rank s (those
    whose row_src falls in s's range), and its combine_recv sums them; comb,
    out and the pulling combine's output must match (comb bit for bit; out
    within the combine tolerance, and bit for bit)."""
    sh, B = r["sh"], r["B"]
    N, T, H, k = sh.N, sh.T, sh.H, sh.k
    rsrc = O.row_src(lay)
    w = np.asarray(r["w"], np.float32)
    y = r["y"]
    ranks = list(range(N)) if ranks is None else list(ranks)

    def one(s):
        sel = np.flatnonzero((rsrc >= s * T * k) & (rsrc < (s + 1) * T * k))
        y_sub = bf16_np(_rows(y, sel))
        comb = O.combine_send(y_sub, rsrc[sel] - s * T * k, 1, T, k)
        got = bf16_np(B.comb[s])
        wr = rsrc[sel] - s * T * k
        assert (got[wr] == comb[wr]).all(), f"comb rank {s}"
        del got
        out = O.combine_recv(comb, lay.send_pos[s:s + 1], w[s:s + 1], T, k)[0]
        check_combine_out(bf16_np(B.out[s]), out)
        if r.get("out_pull") is not None:
            check_combine_out(bf16_np(r["out_pull"][s]), out)

    _pmap(one, ranks, 6.0 * T * k * H * 2)


def check_partial_full_size(r, lay: O.Layout, ranks=None, bound_every: int = 16, tok_chunk: int = 256):
    """The send-side partial combine of the source ranks `ranks` (all by
    default), every token: each group row at its leader's position and the
    output bit for bit against the oracle's partial_token (run in worker
    processes, a chunk of tokens each), rows no group leads left untouched,
    and the mode's tolerance on every bound_every-th token."""
    import oracle_pool
    sh = r["sh"]
    N, T, H, k = sh.N, sh.T, sh.H, sh.k
    L = sh.E // N
    comb, out = run_partial(r)
    w = np.asarray(r["w"], np.float32)
    ranks = list(range(N)) if ranks is None else list(ranks)
    items = [(s, t0) for s in ranks for t0 in range(0, T, tok_chunk)]

    def inputs():
        for s, t0 in items:
            t1 = min(T, t0 + tok_chunk)
            em = lay.em_row[s, t0:t1]
            part = em >= 0
            rows = bf16_np(_rows(r["y"], np.where(part, em, 0).reshape(-1))).reshape(t1 - t0, k, H)
            rows[~part] = 0
            dest = np.where(lay.slot_valid[s, t0:t1], r["idx"][s, t0:t1], 0) // L
            yield rows, w[s, t0:t1], dest, part

    led = {s: np.zeros(T * k, bool) for s in ranks}
    got_out = {s: bf16_np(out[s]) for s in ranks}
    with oracle_pool.pool(oracle_pool.processes()) as pool:
        for (s, t0), res in zip(items, pool.imap(oracle_pool.partial_tokens, inputs())):
            pos = [lay.send_pos[s, t0 + i, j] for i, (groups, _) in enumerate(res) for j, _ in groups]
            got = bf16_np(_rows(comb[s], np.asarray(pos)))
            want = np.stack([p for groups, _ in res for _, p in groups])
            assert (got == want).all(), f"group rows, rank {s} tokens {t0}.."
            led[s][pos] = True
            for i, (groups, o) in enumerate(res):
                t = t0 + i
                assert (got_out[s][t] == o).all(), (s, t)
                if t % bound_every == 0:
                    part = lay.em_row[s, t] >= 0
                    rows_t = bf16_np(_rows(r["y"], np.where(part, lay.em_row[s, t], 0)))
                    rows_t[~part] = 0
                    partial_bound_check(got_out[s][t], O.bf16_from_bits(rows_t).astype(np.float64),
                                        np.where(part, w[s, t], 0.0), [p for _, p in groups])
    for s in ranks:
        assert (bf16_np(comb[s])[~led[s]] == PARTIAL_FILL).all(), f"rows no group leads were written (rank {s})"

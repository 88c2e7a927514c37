"""Benchmark: one MoE layer's dispatch + combine on one MI355X.

A step is the whole hot path over one batch: moe_dispatch_send (counts, scans,
positions, quantise + pack), moe_dispatch_recv (expert-major unpack),
moe_combine_send and moe_combine_recv, for all N logical ranks.  Inputs are
seeded synthetic tensors already resident in HBM.  Prints one JSON line.

The headline workload (default combine_heavy: T=4096, H=7168) gives the line's
value; every other workload is measured the same way in the same run and
reported under "workloads" (tiny, dsv3_decode, kimi_skewed, prefill,
prefill_forced).  Workloads whose combine batch differs from the dispatch
batch (the Kimi-K2 shape: dispatch 128, combine 4096 tokens per rank) time the
dispatch at the dispatch batch and the combine on the layout of an untimed,
payload-free dispatch at the combine batch.

Beside the step, on the same data: the pulling combine (moe_combine_pull), the
combine with send-side partial sums, the direct dispatch (moe_dispatch_direct)
and, when every rank's slots fit one routing chunk (T*k <= 4096), the single
launches (moe_dispatch_send_ll, also with early rows, and
moe_dispatch_direct_ll); the fastest composition of one layer as whole steps;
cold-cache phase times (1 GiB of scratch written before each call).  Each
phase's rate is also given as a fraction of two ceilings measured on the
phase's own buffers: the HIP runtime's own device-to-device copy
(hipMemcpyAsync) and fill (hipMemsetAsync, a write-only stream), and plain
streams of the phase's access pattern (libmoe_streams: a fan-out for the pack,
a copy for unpack and combine send, a reduction for the receive-side sum).
The CPU baselines (the oracle in one process, and in min(16, cores)
processes on independent problems) run first, before the GPU is touched.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--workloads all|none|a,b,...] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, published
PHASES = ["dispatch_send", "dispatch_recv", "combine_send", "combine_recv"]
# The kernel that moves each phase's bytes (dispatch send also runs the
# routing kernels, dispatch recv the row-map kernel k_unpack_index).
KERNEL_OF = {"dispatch_send": "k_pack_os", "dispatch_recv": "k_unpack_os", "combine_send": "k_comb_send_os",
             "combine_recv": "k_comb_recv_os"}
ALL_WORKLOADS = ["tiny", "dsv3_decode", "combine_heavy", "kimi_skewed", "prefill", "prefill_forced"]
DTYPE = "f32 arithmetic; e4m3fn payload with f32 block-128 scales (dispatch), bf16 (combine)"


def kernel_of(phase: str) -> str:
    return KERNEL_OF[phase]


def algorithmic_bytes(N, T, H, E, k, Tc=None, G=None):
    """Bytes each phase must move (inputs read once, outputs written once);
    Tc is the combine batch when it differs from the dispatch batch T; G the
    number of (token, destination rank) groups of the combine batch, which
    the send-side partial combine ships one row each."""
    Tc = T if Tc is None else Tc
    P, Pc = N * T * k, N * Tc * k
    G = Pc if G is None else G
    rowq = H + 4 * (H // 128)          # fp8 payload + fp32 scales
    rowb = 2 * H                       # bf16 row
    return {
        "combine_send_partial": Pc * rowb + G * rowb + 3 * N * Tc * k * 4,
        "combine_recv_partial": G * rowb + N * Tc * H * 2 + 2 * N * Tc * k * 4,
        "dispatch_send": N * T * 2 * H + P * rowq + 2 * N * T * k * 4 + N * E * 4,
        "dispatch_direct": N * T * 2 * H + P * rowq + 3 * N * T * k * 4 + N * E * 4,
        "dispatch_recv": 2 * P * rowq,
        "combine_send": 2 * Pc * rowb,
        "combine_recv": Pc * rowb + N * Tc * H * 2 + 2 * N * Tc * k * 4,
        "combine_pull": Pc * rowb + N * Tc * H * 2 + 3 * N * Tc * k * 4,
    }


def phase_read_write(N, T, H, E, k, Tc=None):
    """(read bytes, written bytes) of each of the four phases; their sums are
    algorithmic_bytes'.  The pack writes four times what it reads."""
    Tc = T if Tc is None else Tc
    P, Pc = N * T * k, N * Tc * k
    rowq, rowb = H + 4 * (H // 128), 2 * H
    return {"dispatch_send": (N * T * 2 * H + N * T * k * 4, P * rowq + N * T * k * 4 + N * E * 4),
            "dispatch_recv": (P * rowq, P * rowq),
            "combine_send": (Pc * rowb, Pc * rowb),
            "combine_recv": (Pc * rowb + 2 * N * Tc * k * 4, N * Tc * H * 2)}


def combine_groups(idx, L):
    """(token, destination rank) groups of a routing [N, T, k] with valid ids:
    the rows the send-side partial combine ships."""
    import numpy as np
    k = idx.shape[-1]
    ranks = np.sort(np.asarray(idx).reshape(-1, k) // L, axis=1)
    return int(ranks.shape[0] + np.count_nonzero(ranks[:, 1:] != ranks[:, :-1]))


def _kernel_sources_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "combine_lds_atomic_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def _build_info():
    """The commit the libraries were built from (written by build.py), if known."""
    p = os.path.join(ROOT, "combine_lds_atomic_amd", "build_info.json")
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        return json.load(fh)


def _traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("sources_digest") != _kernel_sources_digest():
        return None
    return d.get("hbm_bytes_per_launch")


def _oracle_run(cfg, T_sample: int, ready=None):
    """The oracle's four phases on seeded inputs of `cfg` with T_sample tokens
    per rank; input generation is not timed.  Returns (algorithmic bytes,
    seconds, start, end) with start/end on the monotonic clock.  `ready`, if
    given, is waited on once the inputs exist (a barrier across processes)."""
    import numpy as np
    import torch

    import workloads as W
    from oracle import moe_oracle as O

    idx, w = W.routing(cfg, T_sample)
    x = W.tokens(cfg, "cpu", T_sample).float().numpy()
    if ready is not None:
        ready.wait()
    t0 = time.monotonic()
    lay = O.layout(idx, cfg.E, cfg.N)
    rq, rs = O.dispatch_send(x, lay)
    xq, xs, rsrc = O.dispatch_recv(rq, rs, lay)
    t1 = time.monotonic()
    y = W.expert_outputs(cfg, lay.total_rows, "cpu").view(torch.int16).numpy().view(np.uint16)
    t2 = time.monotonic()
    comb = O.combine_send(y, rsrc, cfg.N, T_sample, cfg.k)
    O.combine_recv(comb, lay.send_pos, w, T_sample, cfg.k)
    t3 = time.monotonic()
    nb = algorithmic_bytes(cfg.N, T_sample, cfg.H, cfg.E, cfg.k)
    return sum(nb[p] for p in PHASES), (t1 - t0) + (t3 - t2), t0, t3


def note(msg: str) -> None:
    """Progress on stderr (stdout carries only the JSON line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_baseline(T_sample: int):
    """The oracle, as it stands, on a bounded sample of the same workload: the
    same N, H, E, k with T_sample tokens per rank; single-threaded NumPy."""
    import workloads as W
    cfg = W.CONFIGS["combine_heavy"]
    nbytes, sec, _, _ = _oracle_run(cfg, T_sample)
    return {"value": round(nbytes / sec / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "seconds": round(sec, 2),
            "sample": f"combine_heavy shape with T={T_sample} tokens/rank (N={cfg.N}, H={cfg.H}, E={cfg.E}, "
                      f"k={cfg.k}): all four phases, single-threaded NumPy, input generation excluded"}


def _oracle_proc(seed, T_sample, ready, out):
    import torch
    torch.set_num_threads(1)   # one core per process, input generation included
    import workloads as W
    out.put(_oracle_run(W.CONFIGS["combine_heavy"].with_(seed=seed), T_sample, ready))


def cpu_baseline_parallel(T_sample: int, procs: int):
    """The same oracle in `procs` processes at once, each on its own seeded
    sample of T_sample tokens per rank (independent problems, so the
    processes share nothing); throughput = all their bytes over the span from
    the first start to the last end.  Fresh interpreters ("spawn"), started
    before this process touches the GPU."""
    import multiprocessing as mp
    import workloads as W
    ctx = mp.get_context("spawn")
    ready, out = ctx.Barrier(procs), ctx.Queue()
    seed = W.CONFIGS["combine_heavy"].seed
    ps = [ctx.Process(target=_oracle_proc, args=(seed + 1 + i, T_sample, ready, out)) for i in range(procs)]
    for p in ps:
        p.start()
    res = [out.get() for _ in ps]
    for p in ps:
        p.join()
    nbytes = sum(r[0] for r in res)
    span = max(r[3] for r in res) - min(r[2] for r in res)
    cfg = W.CONFIGS["combine_heavy"]
    return {"value": round(nbytes / span / 1e9, 3), "unit": "GB/s", "cores": procs, "kind": "oracle",
            "seconds": round(span, 2),
            "sample": f"{procs} processes, each the combine_heavy shape with T={T_sample} tokens/rank "
                      f"(N={cfg.N}, H={cfg.H}, E={cfg.E}, k={cfg.k}) on its own seed: all four phases, "
                      f"NumPy, input generation excluded"}


class HipRuntime:
    """The HIP runtime torch has loaded (found by soname in the process map),
    for its own copy and fill: independent ceilings beside this repository's
    kernels."""
    MEMCPY_D2D = 3   # hipMemcpyDeviceToDevice

    def __init__(self):
        maps = open("/proc/self/maps").read()
        paths = sorted({ln.split()[-1] for ln in maps.splitlines() if "libamdhip64" in ln})
        if len(paths) != 1:
            raise RuntimeError(f"expected one HIP runtime in the process, found {paths}")
        self.lib = ctypes.CDLL(paths[0])
        self.lib.hipMemcpyAsync.restype = ctypes.c_int
        self.lib.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                            ctypes.c_void_p]
        self.lib.hipMemsetAsync.restype = ctypes.c_int
        self.lib.hipMemsetAsync.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p]

    def copy(self, dst, src, nbytes, stream):
        rc = self.lib.hipMemcpyAsync(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src.data_ptr()), nbytes,
                                     self.MEMCPY_D2D, ctypes.c_void_p(stream.cuda_stream))
        if rc:
            raise RuntimeError(f"hipMemcpyAsync returned {rc}")

    def fill(self, dst, nbytes, stream):
        rc = self.lib.hipMemsetAsync(ctypes.c_void_p(dst.data_ptr()), 0x5A, nbytes, ctypes.c_void_p(stream.cuda_stream))
        if rc:
            raise RuntimeError(f"hipMemsetAsync returned {rc}")


def measure(cfg, args, dev, stream, hip, sweep=False):
    """Every measurement of one workload; returns the result dict and the
    step's total algorithmic bytes and mean step time (ms)."""
    import numpy as np
    import torch

    import combine_lds_atomic_amd as moe
    from combine_lds_atomic_amd import streams as S
    import workloads as W

    T, Tc = cfg.T, cfg.Tc
    # Dispatch problem (timed) at batch T.
    sh = moe.shape(cfg.N, T, cfg.H, cfg.E, cfg.k)
    idx, w = W.routing(cfg, T)
    idx_d = torch.from_numpy(idx).to(dev)
    x = W.tokens(cfg, dev, T)
    B = moe.allocate(sh, dev, combine=(Tc == T))
    # Combine problem at batch Tc: the same buffers when Tc == T, otherwise the
    # layout of an untimed, payload-free dispatch at Tc.
    if Tc == T:
        shc, Bc, idxc_d, wc_d = sh, B, idx_d, torch.from_numpy(w).to(dev)
    else:
        shc = moe.shape(cfg.N, Tc, cfg.H, cfg.E, cfg.k)
        idxc, wc = W.routing(cfg, Tc)
        idxc_d, wc_d = torch.from_numpy(idxc).to(dev), torch.from_numpy(wc).to(dev)
        Bc = moe.allocate(shc, dev, payload=False)
        moe.moe_dispatch_send(shc, None, idxc_d, None, None, Bc.send_pos, Bc.ws)
        moe.moe_dispatch_recv(shc, None, None, Bc.ws, None, None, Bc.exp_off, Bc.row_src)
    y = W.expert_outputs(cfg, Bc.rows, dev)
    out_pull = torch.empty_like(Bc.out)
    G = combine_groups(idx if Tc == T else idxc, cfg.E // cfg.N)

    def step(ev=None, send=moe.moe_dispatch_send):
        if ev: ev[0].record(stream)
        send(sh, x, idx_d, B.recv_q, B.recv_s, B.send_pos, B.ws)
        if ev: ev[1].record(stream)
        moe.moe_dispatch_recv(sh, B.recv_q, B.recv_s, B.ws, B.x_q, B.x_s, B.exp_off, B.row_src)
        if ev: ev[2].record(stream)
        moe.moe_combine_send(shc, y, Bc.row_src, Bc.ws, Bc.comb)
        if ev: ev[3].record(stream)
        moe.moe_combine_recv(shc, Bc.comb, Bc.send_pos, wc_d, Bc.out)
        if ev: ev[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    flags = moe.moe_status(B.ws) | moe.moe_status(Bc.ws)
    if flags:
        raise SystemExit(f"device error flags {flags:#x} during warm-up ({cfg.name})")

    # Timed region: exactly K steps, synchronised on both sides.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = np.array([[evs[i][p].elapsed_time(evs[i][p + 1]) for p in range(4)] for i in range(args.steps)])
    per_phase_ms = ms.mean(axis=0)
    p90_ms = np.percentile(ms, 90, axis=0)
    step_ms = wall * 1e3 / args.steps
    nbytes = algorithmic_bytes(cfg.N, T, cfg.H, cfg.E, cfg.k, Tc, G)
    total = sum(nbytes[p] for p in PHASES)

    # The same step captured once in a HIP graph and replayed (no launch gaps).
    def graph_ms(send=None, fn=None):
        fn = fn or (lambda: step(send=send))
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            fn()
        stream.wait_stream(cap)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fn()
        torch.cuda.synchronize()
        graph.replay()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(args.steps):
            graph.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        del graph
        return g0.elapsed_time(g1) / args.steps

    graph_step_ms = graph_ms(moe.moe_dispatch_send)

    # The single-launch dispatch (moe_dispatch_send_ll, one routing chunk per
    # rank only) in the same step in place of moe_dispatch_send: its phase
    # time, the eager and graph-replayed step, and a bitwise comparison of its
    # outputs with the multi-launch call's.
    single = None
    if T * cfg.k <= 4096 and T > 0:
        note(f"{cfg.name}: single-launch dispatch")
        ref = {f: getattr(B, f).clone() for f in ("send_pos", "recv_q", "recv_s", "x_q", "x_s", "row_src")}
        for _ in range(args.warmup):
            step(send=moe.moe_dispatch_send_ll)
        evl = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(evl[i], send=moe.moe_dispatch_send_ll)
        torch.cuda.synchronize()
        wall_l = time.perf_counter() - t0
        same = all(torch.equal(getattr(B, f).view(torch.uint8) if ref[f].dtype != torch.int32 else getattr(B, f),
                               ref[f].view(torch.uint8) if ref[f].dtype != torch.int32 else ref[f]) for f in ref)
        ms_l = np.array([[evl[i][p].elapsed_time(evl[i][p + 1]) for p in range(4)] for i in range(args.steps)])
        single = {"call": "moe_dispatch_send_ll", "dispatch_send": None,
                  "step_us": round(wall_l * 1e6 / args.steps, 1),
                  "graph_step_us": round(graph_ms(moe.moe_dispatch_send_ll) * 1e3, 1),
                  "same_bytes_as_dispatch_send": bool(same)}
        single_ms = ms_l.mean(axis=0)[0]
        single_p90 = np.percentile(ms_l[:, 0], 90)
        del ref

        # The same with early rows: fixed regions that start with C private
        # rows per sender (C about 1.25x the mean rows of a rank pair), so
        # most packers need only their own rank's count.  Regions are sized
        # from the routing to hold everything.
        L = cfg.E // cfg.N
        C = max(1, int(np.ceil(1.25 * T * cfg.k / cfg.N)))
        pair = np.zeros((cfg.N, cfg.N), np.int64)
        for s_ in range(cfg.N):
            pair[s_] = np.bincount(idx[s_].reshape(-1) // L, minlength=cfg.N)
        R = int(cfg.N * C + np.maximum(pair - C, 0).sum(axis=0).max())
        she = moe.shape(cfg.N, T, cfg.H, cfg.E, cfg.k, R, C)
        Be = moe.allocate(she, dev, combine=False)
        ye = W.expert_outputs(cfg, Be.rows, dev)
        comb_e = torch.empty((cfg.N, T * cfg.k, cfg.H), dtype=torch.bfloat16, device=dev)
        out_e = torch.empty((cfg.N, T, cfg.H), dtype=torch.bfloat16, device=dev)
        w_d = torch.from_numpy(w).to(dev)       # weights of the dispatch batch

        def step_e(ev=None):
            if ev: ev[0].record(stream)
            moe.moe_dispatch_send_ll(she, x, idx_d, Be.recv_q, Be.recv_s, Be.send_pos, Be.ws)
            if ev: ev[1].record(stream)
            moe.moe_dispatch_recv(she, Be.recv_q, Be.recv_s, Be.ws, Be.x_q, Be.x_s, Be.exp_off, Be.row_src)
            if ev: ev[2].record(stream)
            moe.moe_combine_send(she, ye, Be.row_src, Be.ws, comb_e)
            if ev: ev[3].record(stream)
            moe.moe_combine_recv(she, comb_e, Be.send_pos, w_d, out_e)
            if ev: ev[4].record(stream)

        for _ in range(args.warmup):
            step_e()
        eve = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            step_e(eve[i])
        torch.cuda.synchronize()
        ms_e = np.array([[eve[i][p].elapsed_time(eve[i][p + 1]) for p in range(4)] for i in range(args.steps)])
        same_e = bool(torch.equal(Be.send_pos, B.send_pos))
        early_ms = ms_e.mean(axis=0)[0]
        single["early_rows"] = {"early_rows": C, "region_rows": R, "dispatch_send": None,
                                "same_send_pos": same_e}
        flags_e = moe.moe_status(Be.ws)
        if flags_e:
            raise SystemExit(f"device error flags {flags_e:#x} in the early-row steps ({cfg.name})")
        del Be, ye, comb_e, out_e

        # The routing alone: both sends without tokens compute only the
        # layout (send_pos and the tables).  The single launch then runs its
        # count and cross-rank workgroups only, so its time bounds from above
        # the routing its packers wait for before their first store (the
        # cross-rank workgroup's last step, the receive tables, comes after
        # the packers' signal); the multi-launch send runs its count and
        # cross-rank kernels.
        def time_layout(fn):
            for _ in range(max(args.warmup, 1)):
                fn(sh, None, idx_d, None, None, B.send_pos, B.ws)
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
            for i in range(args.steps):
                ev[i][0].record(stream)
                fn(sh, None, idx_d, None, None, B.send_pos, B.ws)
                ev[i][1].record(stream)
            torch.cuda.synchronize()
            t = np.array([e[0].elapsed_time(e[1]) for e in ev])
            return round(float(np.median(t)) * 1e3, 1)

        single["routing_only_median_us"] = {"moe_dispatch_send_ll": time_layout(moe.moe_dispatch_send_ll),
                                            "moe_dispatch_send": time_layout(moe.moe_dispatch_send)}

    note(f"{cfg.name}: direct dispatch")
    # The direct dispatch (moe_dispatch_direct: rows stored straight at their
    # expert-major rows, no receive regions, no unpack) on the same inputs
    # and buffers, compared bit for bit with the two-call path's outputs.
    # Its single launch (moe_dispatch_direct_ll) likewise where T*k <= 4096.
    ref = {f: getattr(B, f).clone() for f in ("send_pos", "x_q", "x_s", "exp_off", "row_src")}

    def time_direct(fn):
        for _ in range(max(args.warmup, 1)):
            fn(sh, x, idx_d, B.x_q, B.x_s, B.send_pos, B.exp_off, B.row_src, B.ws)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for i in range(args.steps):
            ev[i][0].record(stream)
            fn(sh, x, idx_d, B.x_q, B.x_s, B.send_pos, B.exp_off, B.row_src, B.ws)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        t = np.array([e[0].elapsed_time(e[1]) for e in ev])
        same = all(torch.equal(getattr(B, f).view(torch.uint8), ref[f].view(torch.uint8)) for f in ref)
        return t.mean(), np.percentile(t, 90), np.median(t), bool(same)

    direct_ms, direct_p90, direct_med, direct_same = time_direct(moe.moe_dispatch_direct)
    direct_ll = time_direct(moe.moe_dispatch_direct_ll) if T * cfg.k <= 4096 and T > 0 else None
    del ref

    note(f"{cfg.name}: pulling and partial combines")
    # The pulling combine on the same data (not part of the step).
    pull_ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    for _ in range(2):
        moe.moe_combine_pull(shc, y, idxc_d, Bc.send_pos, wc_d, Bc.ws, out_pull)
    pull_ev[0].record(stream)
    for i in range(args.steps):
        moe.moe_combine_pull(shc, y, idxc_d, Bc.send_pos, wc_d, Bc.ws, out_pull)
        pull_ev[i + 1].record(stream)
    torch.cuda.synchronize()
    pull_ms = np.array([pull_ev[i].elapsed_time(pull_ev[i + 1]) for i in range(args.steps)]).mean()
    pull_same = bool(torch.equal(out_pull.view(torch.int16), Bc.out.view(torch.int16)))

    # Combine with send-side partial sums (one row per token and destination
    # rank), on the same data, into its own buffers (not part of the step).
    comb_p = torch.empty_like(Bc.comb)
    out_p = torch.empty_like(Bc.out)
    for _ in range(2):
        moe.moe_combine_send_partial(shc, y, idxc_d, Bc.send_pos, wc_d, Bc.ws, comb_p)
        moe.moe_combine_recv_partial(shc, comb_p, idxc_d, Bc.send_pos, Bc.ws, out_p)
    part_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        part_ev[i][0].record(stream)
        moe.moe_combine_send_partial(shc, y, idxc_d, Bc.send_pos, wc_d, Bc.ws, comb_p)
        part_ev[i][1].record(stream)
        moe.moe_combine_recv_partial(shc, comb_p, idxc_d, Bc.send_pos, Bc.ws, out_p)
        part_ev[i][2].record(stream)
    torch.cuda.synchronize()
    part_ms = np.array([[part_ev[i][p].elapsed_time(part_ev[i][p + 1]) for p in range(2)]
                        for i in range(args.steps)]).mean(axis=0)
    part_diff = float((out_p.view(torch.int16) != Bc.out.view(torch.int16)).float().mean().item())
    del comb_p, out_p

    # Cold-cache phase times (secondary): before each phase call, 1 GiB of
    # scratch is written so that nothing of the previous phase's output (nor
    # of this phase's inputs) is left in the 256 MB Infinity Cache.
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    calls = [lambda: moe.moe_dispatch_send(sh, x, idx_d, B.recv_q, B.recv_s, B.send_pos, B.ws),
             lambda: moe.moe_dispatch_recv(sh, B.recv_q, B.recv_s, B.ws, B.x_q, B.x_s, B.exp_off, B.row_src),
             lambda: moe.moe_combine_send(shc, y, Bc.row_src, Bc.ws, Bc.comb),
             lambda: moe.moe_combine_recv(shc, Bc.comb, Bc.send_pos, wc_d, Bc.out)]
    cold = np.zeros((args.steps, 4))
    for i in range(args.steps):
        for p, fn in enumerate(calls):
            scratch.fill_(i & 0xFF)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            cold[i, p] = e0.elapsed_time(e1)
    del scratch

    # The fastest composition of one layer on one GPU: the faster dispatch --
    # the direct one, or the send (single launch with early rows where it
    # applies, else the multi-launch call) plus the unpack -- then the
    # pulling combine, timed as whole steps.
    fast = None
    if Tc == T:
        note(f"{cfg.name}: fastest layer")
        two_call_ms = (early_ms if single is not None else per_phase_ms[0]) + per_phase_ms[1]
        direct_f = moe.moe_dispatch_direct
        if direct_ll is not None and direct_ll[0] < direct_ms:
            direct_f = moe.moe_dispatch_direct_ll
        if min(direct_ms, direct_ll[0] if direct_ll else direct_ms) < two_call_ms:
            she_f, Bf, send_f = sh, B, None
        elif single is not None:
            she_f = moe.shape(cfg.N, T, cfg.H, cfg.E, cfg.k, single["early_rows"]["region_rows"],
                              single["early_rows"]["early_rows"])
            Bf = moe.allocate(she_f, dev, combine=False)
            send_f = moe.moe_dispatch_send_ll
        else:
            she_f, Bf, send_f = sh, B, moe.moe_dispatch_send
        yf = y if Bf is B else W.expert_outputs(cfg, Bf.rows, dev)
        out_f = torch.empty_like(Bc.out)
        w_f = torch.from_numpy(w).to(dev)

        def step_f(ev=None):
            if ev: ev[0].record(stream)
            if send_f is None:
                direct_f(she_f, x, idx_d, Bf.x_q, Bf.x_s, Bf.send_pos, Bf.exp_off, Bf.row_src, Bf.ws)
                if ev: ev[1].record(stream)
            else:
                send_f(she_f, x, idx_d, Bf.recv_q, Bf.recv_s, Bf.send_pos, Bf.ws)
                if ev: ev[1].record(stream)
                moe.moe_dispatch_recv(she_f, Bf.recv_q, Bf.recv_s, Bf.ws, Bf.x_q, Bf.x_s, Bf.exp_off, Bf.row_src)
            if ev: ev[2].record(stream)
            moe.moe_combine_pull(she_f, yf, idx_d, Bf.send_pos, w_f, Bf.ws, out_f)
            if ev: ev[3].record(stream)

        for _ in range(args.warmup):
            step_f()
        evf = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step_f(evf[i])
        torch.cuda.synchronize()
        wall_f = time.perf_counter() - t0
        ms_f = np.array([[evf[i][p].elapsed_time(evf[i][p + 1]) for p in range(3)] for i in range(args.steps)])
        fast = {"dispatch": direct_f.__name__ if send_f is None else f"{send_f.__name__} + moe_dispatch_recv",
                "early_rows": she_f.early_rows,
                "us": {n: round(v * 1e3, 1) for n, v in zip(
                    ("dispatch_direct", None, "combine_pull") if send_f is None else
                    ("dispatch_send", "dispatch_recv", "combine_pull"), ms_f.mean(axis=0)) if n},
                "step_us": round(wall_f * 1e6 / args.steps, 1),
                "graph_step_us": round(graph_ms(fn=step_f) * 1e3, 1)}
        if Bf is not B:
            flags_f = moe.moe_status(Bf.ws)
            if flags_f:
                raise SystemExit(f"device error flags {flags_f:#x} in the fastest-path steps ({cfg.name})")
            del Bf, yf
        del out_f

    flags = moe.moe_status(B.ws) | moe.moe_status(Bc.ws)
    if flags:
        raise SystemExit(f"device error flags {flags:#x} in the timed steps ({cfg.name})")

    # Ceilings on the phases' own buffers (where a buffer lands in memory moves
    # a stream's rate by up to ~20%), free of row lookups and arithmetic:
    #   - the HIP runtime's own device-to-device copy (hipMemcpyAsync, y ->
    #     comb, the dominant phase's bytes) and fill (hipMemsetAsync on comb,
    #     write-only), independent of this repository's kernels;
    #   - libmoe_streams' copy of the same bytes, and its streams with the
    #     pack's pattern (a bf16 token row read, k fp8 rows stored: tokens ->
    #     recv_q) and the receive-side sum's (k bf16 rows read, one stored:
    #     comb -> out).
    # They overwrite recv_q, comb and out, so they run after everything else.
    note(f"{cfg.name}: ceilings")
    dom = max(range(4), key=lambda p: per_phase_ms[p])
    copy_bytes = (nbytes[PHASES[dom]] // 2) // 16 * 16
    copy_bytes = min(copy_bytes, y.numel() * 2 // 16 * 16, Bc.comb.numel() * 2 // 16 * 16)

    def rate(fn, moved):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(5):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return moved * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9

    u_fan = cfg.N * T * cfg.H // 16            # one fp8 copy of every dispatched token, in 16-B units
    u_red = cfg.N * Tc * cfg.H * 2 // 16       # the bf16 combine output, in 16-B units
    assert 2 * u_fan * 16 == x.numel() * 2 and cfg.k * u_fan * 16 <= B.recv_q.numel()
    assert cfg.k * u_red * 16 == Bc.comb.numel() * 2 and u_red * 16 == Bc.out.numel() * 2
    vendor_copy = rate(lambda: hip.copy(Bc.comb, y, copy_bytes, stream), 2 * copy_bytes)
    vendor_fill = rate(lambda: hip.fill(Bc.comb, copy_bytes, stream), copy_bytes)
    copy_gbs = rate(lambda: S.moe_copy(Bc.comb, y, copy_bytes), 2 * copy_bytes)
    fan_chunked = rate(lambda: S.moe_stream(S.STREAM_FANOUT, cfg.k, B.recv_q, x, u_fan), (2 + cfg.k) * u_fan * 16)
    fan_oneshot = rate(lambda: S.moe_stream(S.STREAM_FANOUT_ONESHOT, cfg.k, B.recv_q, x, u_fan),
                       (2 + cfg.k) * u_fan * 16)
    fan_gbs = max(fan_chunked, fan_oneshot)    # the faster grid form of the fan-out
    red_gbs = rate(lambda: S.moe_stream(S.STREAM_REDUCE, cfg.k, Bc.out, Bc.comb, u_red), (cfg.k + 1) * u_red * 16)
    ceilings = {"dispatch_send": {"pattern": f"fan-out: 32 B read, 16 B stored to each of {cfg.k} arrays "
                                             "(the faster of two grid forms)",
                                  "GB/s": round(fan_gbs, 1), "chunked_GB/s": round(fan_chunked, 1),
                                  "one_shot_GB/s": round(fan_oneshot, 1)},
                "dispatch_recv": {"pattern": "copy", "GB/s": round(copy_gbs, 1)},
                "combine_send": {"pattern": "copy", "GB/s": round(copy_gbs, 1)},
                "combine_recv": {"pattern": f"reduction: {cfg.k} arrays read, one stored",
                                 "GB/s": round(red_gbs, 1)}}
    # The same two streams with fewer arrays (headline workload only): how
    # much of the fan-out's and the reduction's shortfall against the copy
    # comes from spreading the accesses over k arrays at once.
    by_k = None
    if sweep:
        by_k = {"fanout_chunked_GB/s": {}, "fanout_one_shot_GB/s": {}, "reduce_GB/s": {}}
        for kk in sorted({1, 2, 4, cfg.k}):
            for key, pat in (("fanout_chunked_GB/s", S.STREAM_FANOUT), ("fanout_one_shot_GB/s", S.STREAM_FANOUT_ONESHOT)):
                by_k[key][kk] = round(rate(lambda: S.moe_stream(pat, kk, B.recv_q, x, u_fan), (2 + kk) * u_fan * 16), 1)
            by_k["reduce_GB/s"][kk] = round(rate(lambda: S.moe_stream(S.STREAM_REDUCE, kk, Bc.out, Bc.comb, u_red),
                                                 (kk + 1) * u_red * 16), 1)
    vendor = {"copy_GB/s": round(vendor_copy, 1), "fill_GB/s": round(vendor_fill, 1),
              "bytes": int(copy_bytes),
              "what": "hipMemcpyAsync device-to-device y -> comb (GB/s counts bytes read + written) and "
                      "hipMemsetAsync on comb (bytes written), on the phases' own buffers"}

    def info(name, t_ms, t90=None, t50=None):
        """Mean time t_ms (the roofline uses the mean launch duration), with
        the p90 and median where given."""
        gbs = nbytes[name] / (t_ms * 1e-3) / 1e9
        d = {"us": round(t_ms * 1e3, 1), "alg_bytes": nbytes[name], "GB/s": round(gbs, 1),
             "frac": round(gbs / HBM_PEAK_GBS, 4)}
        if t50 is not None:
            d["median_us"] = round(t50 * 1e3, 1)
        if t90 is not None:
            d["p90_us"] = round(t90 * 1e3, 1)
        return d

    rw = phase_read_write(cfg.N, T, cfg.H, cfg.E, cfg.k, Tc)
    med_ms = np.median(ms, axis=0)
    phase_info = {name: info(name, per_phase_ms[p], p90_ms[p], med_ms[p]) for p, name in enumerate(PHASES)}
    for name, d in phase_info.items():
        d["of_pattern_ceiling"] = round(d["GB/s"] / ceilings[name]["GB/s"], 4)
        d["of_vendor_copy"] = round(d["GB/s"] / vendor_copy, 4)
        rb, wb = rw[name]
        d["read_write_bytes"] = [rb, wb]
    if single is not None:
        single["dispatch_send"] = info("dispatch_send", single_ms, single_p90)
        single["early_rows"]["dispatch_send"] = info("dispatch_send", early_ms)
    dom_name = PHASES[dom]
    achieved = nbytes[dom_name] / (per_phase_ms[dom] * 1e-3) / 1e9
    kernel = kernel_of(dom_name)
    batch = f"T={T}" if Tc == T else f"dispatch T={T}, combine T={Tc}"
    res = {
        "config": {"workload": f"{cfg.name}: {cfg.note}; packed receive regions", "N": cfg.N, "T": T, "T_comb": Tc,
                   "H": cfg.H, "E": cfg.E, "k": cfg.k, "region_rows": 0, "batch": batch, "seed": cfg.seed,
                   "payload": "bf16 in, e4m3fn+fp32 block-128 scales dispatched, bf16 combined with fp32 accumulation"},
        "phases": phase_info,
        "phases_cold_cache": {name: {"median_us": round(float(np.median(cold[:, p])) * 1e3, 1),
                                     "p90_us": round(float(np.percentile(cold[:, p], 90)) * 1e3, 1)}
                              for p, name in enumerate(PHASES)},
        "step_us": round(step_ms * 1e3, 1),
        "dispatch_us": round((per_phase_ms[0] + per_phase_ms[1]) * 1e3, 1),
        "combine_us": round((per_phase_ms[2] + per_phase_ms[3]) * 1e3, 1),
        "dispatch_frac": round((nbytes["dispatch_send"] + nbytes["dispatch_recv"]) /
                               ((per_phase_ms[0] + per_phase_ms[1]) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "combine_frac": round((nbytes["combine_send"] + nbytes["combine_recv"]) /
                              ((per_phase_ms[2] + per_phase_ms[3]) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "combine_pull": dict(info("combine_pull", pull_ms), same_bytes_as_send_recv=pull_same,
                             of_pattern_ceiling=round(nbytes["combine_pull"] / (pull_ms * 1e-3) / 1e9 / red_gbs, 4)),
        "dispatch_direct": dict(info("dispatch_direct", direct_ms, direct_p90, direct_med),
                                same_bytes_as_send_recv=bool(direct_same),
                                of_pattern_ceiling=round(nbytes["dispatch_direct"] / (direct_ms * 1e-3) / 1e9 / fan_gbs, 4),
                                single_launch=None if direct_ll is None else dict(
                                    info("dispatch_direct", *direct_ll[:3]), same_bytes_as_send_recv=direct_ll[3])),
        "combine_partial": {"groups_per_token": round(G / (cfg.N * Tc), 3),
                            "send": info("combine_send_partial", part_ms[0]),
                            "recv": info("combine_recv_partial", part_ms[1]),
                            "us": round((part_ms[0] + part_ms[1]) * 1e3, 1),
                            "elements_differing_from_send_recv": round(part_diff, 5)},
        "graph_step_us": round(graph_step_ms * 1e3, 1),
        "single_launch_dispatch": single,
        "fastest_layer": fast,
        "vendor_ceilings": vendor,
        "copy_ceiling_GB/s": round(copy_gbs, 1),
        "pattern_ceilings": ceilings,
        "pattern_ceilings_by_arrays": by_k,
        "roofline": {"bound": "hbm", "kernel": kernel, "phase": dom_name, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": _traffic(kernel, cfg.name)},
    }
    del B, Bc, x, y, out_pull
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res, total, step_ms


def summary(r):
    """The per-workload entry of the JSON line: phase medians and rates, the
    dispatch / combine fractions, the step, the fastest layer and the
    ceilings."""
    return {
        "config": r["config"]["workload"],
        "phases": {p: {k: v for k, v in d.items() if k in ("median_us", "us", "GB/s", "frac", "of_vendor_copy",
                                                               "of_pattern_ceiling")}
                   for p, d in r["phases"].items()},
        "dispatch_frac": r["dispatch_frac"], "combine_frac": r["combine_frac"],
        "dispatch_us": r["dispatch_us"], "combine_us": r["combine_us"],
        "step_us": r["step_us"], "graph_step_us": r["graph_step_us"],
        "fastest_layer": r["fastest_layer"],
        "combine_pull_us": r["combine_pull"]["us"],
        "dispatch_direct_us": r["dispatch_direct"]["us"],
        "dispatch_direct_ll_us": (r["dispatch_direct"]["single_launch"] or {}).get("us"),
        "dispatch_send_ll_us": ((r["single_launch_dispatch"] or {}).get("dispatch_send") or {}).get("us"),
        "dispatch_send_ll_early_rows_us": (((r["single_launch_dispatch"] or {}).get("early_rows") or {})
                                           .get("dispatch_send") or {}).get("us"),
        "routing_only_median_us": (r["single_launch_dispatch"] or {}).get("routing_only_median_us"),
        "combine_partial_us": r["combine_partial"]["us"],
        "vendor_ceilings": {k: v for k, v in r["vendor_ceilings"].items() if k.endswith("GB/s")},
        "pattern_ceilings_GB/s": {p: c["GB/s"] for p, c in r["pattern_ceilings"].items()},
        "roofline_kernel": r["roofline"]["kernel"], "roofline_frac": r["roofline"]["frac"],
    }


def latency_model(points):
    """Per phase, the fit t = alpha + bytes / beta over the workloads of one
    run (points: phase -> [(algorithmic bytes, us)]), least squares on the
    relative residuals so that the small workloads fix alpha (the fixed cost
    per call: launches, routing latency) and the large ones beta (the
    streaming rate).  Phases with fewer than three workloads are left out."""
    import numpy as np
    out = {}
    for phase, pts in points.items():
        if len(pts) < 3:
            continue
        b = np.array([p[0] for p in pts], dtype=np.float64) / 1e9   # GB
        t = np.array([p[1] for p in pts], dtype=np.float64)         # us
        A = np.stack([np.ones_like(b), b], axis=1) / t[:, None]
        (alpha, slope), *_ = np.linalg.lstsq(A, np.ones_like(t), rcond=None)
        fit = alpha + slope * b
        out[phase] = {"alpha_us": round(float(alpha), 2),
                      "beta_GB/s": round(float(1e6 / slope), 1) if slope > 0 else None,
                      "workloads": len(pts),
                      "max_rel_residual": round(float(np.max(np.abs(fit - t) / t)), 4)}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="combine_heavy", help="the headline workload")
    ap.add_argument("--workloads", default="all",
                    help="other workloads measured in the same run: all, none, or a comma-separated list")
    ap.add_argument("--shape", default=None,
                    help="N,T,H,E,k: time a uniformly routed workload of this shape as the headline instead")
    ap.add_argument("--seed", type=int, default=None, help="input seed of the headline workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=2048)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: all N logical EP ranks live in one MI355X's HBM, so --gpus {args.gpus} "
              "is not a configuration of this benchmark (the multi-GPU sharding is a design, not built).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads as W

    cfg = W.CONFIGS[args.workload]
    if args.shape:
        try:
            N, T, H, E, k = (int(v) for v in args.shape.split(","))
        except ValueError:
            raise SystemExit("--shape takes N,T,H,E,k")
        cfg = W.Config("custom", N=N, T=T, H=H, E=E, k=k, seed=0x7A11_00FF,
                       note=f"T={T}, H={H}, E={E}, k={k}, N={N}, uniform routing")
    if args.seed is not None:
        cfg = cfg.with_(seed=args.seed)
    others = [] if args.workloads == "none" else (
        [w for w in ALL_WORKLOADS if w != cfg.name] if args.workloads == "all" else
        [w for w in args.workloads.split(",") if w and w != cfg.name])
    for w in others:
        if w not in W.CONFIGS:
            raise SystemExit(f"unknown workload {w}")
    # The CPU baselines run first: the parallel one starts processes, which
    # should happen before this process initialises the GPU.
    cpu_single = cpu_par = None
    if not args.no_cpu_baseline:
        note("cpu baseline: the oracle, one process")
        cpu_single = cpu_baseline(args.cpu_sample_tokens)
        procs = min(16, len(os.sched_getaffinity(0)))
        note(f"cpu baseline: the oracle, {procs} processes")
        cpu_par = cpu_baseline_parallel(max(1, args.cpu_sample_tokens // 8), procs)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    import combine_lds_atomic_amd  # noqa: F401  (loads the library beside torch's HIP runtime)
    hip = HipRuntime()

    note(f"gpu: {cfg.name}, {args.warmup} warm-up and {args.steps} timed steps")
    res, total, step_ms = measure(cfg, args, dev, stream, hip, sweep=True)
    wl = {}
    points = {p: [(d["alg_bytes"], d["us"])] for p, d in res["phases"].items()}
    for name in others:
        note(f"gpu: {name}, {args.warmup} warm-up and {args.steps} timed steps")
        r, _, _ = measure(W.CONFIGS[name], args, dev, stream, hip)
        wl[name] = summary(r)
        for p, d in r["phases"].items():
            points[p].append((d["alg_bytes"], d["us"]))

    value = total / (step_ms * 1e-3) / 1e9
    line = {
        "metric": "dispatch / combine us per layer and effective HBM GB/s (% of ~8 TB/s peak)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE,
        "data": "synthetic",
        "sources_digest": _kernel_sources_digest(),
        "build": _build_info(),
    }
    line.update(res)
    line["workloads"] = wl
    line["latency_model"] = latency_model(points)
    line["cpu_baseline"] = cpu_single
    line["cpu_baseline_parallel"] = cpu_par
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""Two independent problems on two streams at once, each with its own
workspace: the library keeps no state outside the workspace (its only host
state is a per-device cache of CU and occupancy counts), so both must match
the oracle exactly as when run alone.  Both streams have the default
priority."""
import zlib

import numpy as np
import pytest
import torch

import combine_lds_atomic_amd as moe
import workloads as W
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

from gpu_harness import bf16_np, log  # noqa: E402


def _problem(name, N, T, H, E, k, single_launch):
    cfg = W.Config(name, seed=zlib.crc32(name.encode()), N=N, T=T, H=H, E=E, k=k)
    sh = moe.shape(N, T, H, E, k)
    idx, w = W.routing(cfg, T)
    B = moe.allocate(sh, "cuda")
    return dict(cfg=cfg, sh=sh, idx=idx, w=w, B=B, x=W.tokens(cfg, "cuda", T),
                y=W.expert_outputs(cfg, B.rows, "cuda"), idx_d=torch.from_numpy(idx).cuda(),
                w_d=torch.from_numpy(w).cuda(), single_launch=single_launch)


def _run(p, stream):
    sh, B = p["sh"], p["B"]
    send = moe.moe_dispatch_send_ll if p["single_launch"] else moe.moe_dispatch_send
    send(sh, p["x"], p["idx_d"], B.recv_q, B.recv_s, B.send_pos, B.ws, stream)
    moe.moe_dispatch_recv(sh, B.recv_q, B.recv_s, B.ws, B.x_q, B.x_s, B.exp_off, B.row_src, stream)
    moe.moe_combine_pull(sh, p["y"], p["idx_d"], B.send_pos, p["w_d"], B.ws, B.out, stream)


def _check(p):
    cfg, B = p["cfg"], p["B"]
    lay = O.layout(p["idx"], cfg.E, cfg.N)
    assert (B.send_pos.cpu().numpy() == lay.send_pos).all()
    rq, rs = O.dispatch_send(p["x"].float().cpu().numpy(), lay)
    xq, xs, rsrc = O.dispatch_recv(rq, rs, lay)
    assert (B.x_q.cpu().numpy() == xq).all() and (B.x_s.cpu().numpy().view(np.uint32) == xs.view(np.uint32)).all()
    assert (B.row_src.cpu().numpy() == rsrc).all()
    comb = O.combine_send(bf16_np(p["y"]), rsrc, cfg.N, cfg.T, cfg.k)
    out = O.combine_recv(comb, lay.send_pos, p["w"], cfg.T, cfg.k)
    assert (bf16_np(B.out) == out).all()
    assert moe.moe_status(B.ws) == 0


@pytest.mark.parametrize("single_launch", [False, True])
def test_two_streams_two_workspaces(single_launch):
    log(f"\n[gpu] two streams, single_launch={single_launch}")
    a = _problem("streams_a", 16, 128, 2048, 128, 8, single_launch)
    b = _problem("streams_b", 8, 96, 1152, 64, 6, single_launch)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(3):                      # interleave launches of both problems
        _run(a, s1)
        _run(b, s2)
    torch.cuda.synchronize()
    _check(a)
    _check(b)

"""The four calls (and the pulling combine, the single-launch dispatch and
the direct dispatch in both forms) are capturable in a HIP graph: no host
synchronisation, allocation or memset happens inside them.  A captured step is replayed several times, with eager
work and synchronisation between replays, and every replay must equal the
eager run bit for bit."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,T,single_launch", [("tiny", 128, False), ("dsv3_decode", 128, False),
                                                   ("tiny", 128, True), ("dsv3_decode", 128, True)])
def test_graph_replay_matches_eager(name, T, single_launch):
    _replay(name, T, "send_ll" if single_launch else "send")


@pytest.mark.parametrize("name,dispatch", [("tiny", "direct"), ("tiny", "direct_ll"), ("dsv3_decode", "direct_ll")])
def test_graph_replay_direct_dispatch(name, dispatch):
    _replay(name, 128, dispatch)


def _replay(name, T, dispatch):
    import combine_lds_atomic_amd as moe
    cfg = W.CONFIGS[name]
    sh = moe.shape(cfg.N, T, cfg.H, cfg.E, cfg.k)
    idx, w = W.routing(cfg, T)
    idx_d, w_d = torch.from_numpy(idx).cuda(), torch.from_numpy(w).cuda()
    x = W.tokens(cfg, "cuda", T)
    B = moe.allocate(sh, "cuda")
    y = W.expert_outputs(cfg, B.rows, "cuda")
    out_pull = torch.empty_like(B.out)

    def step():
        if dispatch in ("send", "send_ll"):
            send = moe.moe_dispatch_send_ll if dispatch == "send_ll" else moe.moe_dispatch_send
            send(sh, x, idx_d, B.recv_q, B.recv_s, B.send_pos, B.ws)
            moe.moe_dispatch_recv(sh, B.recv_q, B.recv_s, B.ws, B.x_q, B.x_s, B.exp_off, B.row_src)
        else:
            direct = moe.moe_dispatch_direct_ll if dispatch == "direct_ll" else moe.moe_dispatch_direct
            direct(sh, x, idx_d, B.x_q, B.x_s, B.send_pos, B.exp_off, B.row_src, B.ws)
        moe.moe_combine_send(sh, y, B.row_src, B.ws, B.comb)
        moe.moe_combine_recv(sh, B.comb, B.send_pos, w_d, B.out)
        moe.moe_combine_pull(sh, y, idx_d, B.send_pos, w_d, B.ws, out_pull)

    outs = ("send_pos", "x_q", "x_s", "exp_off", "row_src", "comb", "out")
    if dispatch in ("send", "send_ll"):
        outs += ("recv_q", "recv_s")

    def snapshot():
        return {f: getattr(B, f).clone() for f in outs} | {"pull": out_pull.clone()}

    step()
    torch.cuda.synchronize()
    ref = snapshot()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                      # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(4):
        for f in outs:              # eager work between replays: scribble over every output
            getattr(B, f).view(torch.uint8).fill_(0xA5 ^ rep)
        out_pull.view(torch.uint8).fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for f, t in ref.items():
            assert torch.equal(got[f].view(torch.uint8), t.view(torch.uint8)), (rep, f)
    assert moe.moe_status(B.ws) == 0
    del g

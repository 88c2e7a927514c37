"""GPU parity of the combine with send-side partial accumulation
(moe_combine_send_partial + moe_combine_recv_partial) against the oracle's
combine_partial.

Both halves are bit-exact against the oracle (the same float32 operations in
the same order, one bf16 rounding per group row and one for the result):
the group rows at their leaders' positions, the untouched rows of comb and
the output.  The output also meets this mode's own tolerance against the
exact sum, |out - sum_j w_j y_j| <= 2^-8 (|out| + sum_g |p_g|) +
2k 2^-24 sum_j |w_j y_j|.  Small shapes compare every element at once; the
full-size workloads every token of every source rank (eight whole source
ranks at the Kimi shape), rank by rank."""
import zlib

import numpy as np
import pytest
import torch

import workloads as W
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

from gpu_harness import (PARTIAL_FILL, bf16_np, check_partial_full, check_partial_full_size, log,  # noqa: E402
                         partial_bound_check, run_all, run_partial)

FILL = PARTIAL_FILL


@pytest.fixture(autouse=True)
def _announce(request):
    log(f"\n[gpu] {request.node.name}")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _cfg(name, **kw):
    return W.Config(name, seed=zlib.crc32(name.encode()), **kw)


_partial = run_partial
_bound_check = partial_bound_check


def _full_check(r, region_rows=0):
    sh = r["sh"]
    lay = O.layout(r["idx"], sh.E, sh.N, region_rows)
    return lay, check_partial_full(r, lay)


def test_tiny_config():
    _full_check(run_all(W.CONFIGS["tiny"], 128))


@pytest.mark.parametrize("N,T,H,E,k", [
    (8, 33, 256, 16, 8),        # k = E/N: tokens often keep two slots on one rank
    (5, 77, 9216, 40, 6),       # rows longer than 8 columns per lane, ragged
    (4, 20, 256, 64, 12),       # k > 8: groups taken one after another
    (2, 5, 128, 4, 1),          # one slot per token
    (16, 9, 384, 16, 4),        # one expert per rank: every slot its own group
    (3, 1500, 384, 12, 3),      # many tokens, ragged workgroup ranges
])
def test_shapes(N, T, H, E, k):
    _full_check(run_all(_cfg(f"cp{N}_{T}_{H}_{E}_{k}", N=N, T=T, H=H, E=E, k=k), T))


@pytest.mark.parametrize("N,T,H,E,k,tight", [
    (8, 2100, 256, 64, 8, False),    # k <= 8: every group formed from registers
    (4, 4100, 384, 64, 12, False),   # k > 8, ragged token chunks (170 tokens per chunk)
    (8, 2100, 256, 64, 8, True),     # fixed regions that overflow: dropped slots join no group
])
def test_many_tokens(N, T, H, E, k, tight):
    """At least 16384 tokens (N*T): the size from which the send half takes
    its large-problem form; every element checked."""
    cfg = _cfg(f"cp_many{N}_{k}_{tight}", N=N, T=T, H=H, E=E, k=k)
    idx, w = W.routing(cfg, T)
    R = int(O.layout(idx, E, N).recv_total.max()) - 40 if tight else 0
    r = run_all(cfg, T, R, idx=idx, w=w)
    assert N * T >= 16384
    assert bool(r["flags"] & O.FLAG_OVERFLOW) == tight
    _full_check(r, R)


def test_all_slots_on_one_rank_equals_plain_combine():
    cfg = _cfg("cp_forced", N=8, T=200, H=256, E=64, k=8, forced_rank0=True)
    r = run_all(cfg, 200)
    _, lead = _full_check(r)
    assert (lead.sum(axis=2) == 1).all()
    _, out = _partial(r)
    assert torch.equal(out.view(torch.int16), r["B"].out.view(torch.int16))


def test_bad_ids():
    cfg = _cfg("cp_badid", N=4, T=40, H=256, E=16, k=4)
    idx, w = W.routing(cfg, 40)
    idx = idx.copy()
    idx[0, 3, 1] = 16
    idx[2, 7, 0] = -1
    idx[3, 39, 3] = 1 << 30
    _full_check(run_all(cfg, 40, idx=idx, w=w))


def test_fixed_region_overflow():
    cfg = _cfg("cp_ovf", N=4, T=64, H=256, E=8, k=3)
    idx, w = W.routing(cfg, 64)
    idx = idx.copy()
    idx[:, :, 0] = 0
    R = int(O.layout(idx, cfg.E, cfg.N).recv_total.max()) - 9
    r = run_all(cfg, 64, R, idx=idx, w=w)
    assert r["flags"] & O.FLAG_OVERFLOW
    _full_check(r, R)


def test_fixed_regions_with_early_rows():
    """The row lookup follows the early-row layout (its overflow check uses
    the source-major row)."""
    cfg = _cfg("cp_early", N=8, T=64, H=256, E=32, k=6)
    idx, w = W.routing(cfg, 64)
    C = 20
    over = O.layout(idx, cfg.E, cfg.N, cfg.N * C + 10 ** 6, C).recv_off[:, cfg.N]
    R = int(cfg.N * C + over.max() - 3)                  # the fullest region drops its last rows
    r = run_all(cfg, 64, R, idx=idx, w=w, early_rows=C)
    assert r["flags"] & O.FLAG_OVERFLOW
    lay = O.layout(idx, cfg.E, cfg.N, R, C)
    assert ((lay.em_row < 0) & lay.slot_valid).any()
    comb, out = _partial(r)
    comb_o, lead, out_o = O.combine_partial(bf16_np(r["y"]), r["idx"], lay, r["w"])
    assert (bf16_np(out) == out_o).all()
    N, T, k = cfg.N, 64, cfg.k
    rows = [s * T * k + lay.send_pos[s, t, j] for s in range(N) for t in range(T) for j in np.flatnonzero(lead[s, t])]
    assert (bf16_np(comb).reshape(N * T * k, -1)[rows] == comb_o[rows]).all()


def _need(gib):
    free, _ = torch.cuda.mem_get_info()
    if free < gib * 2 ** 30:
        pytest.skip(f"needs {gib} GiB of free device memory, {free / 2**30:.0f} GiB free")


def _full_size(cfg, T, payload=True, ranks=None):
    r = run_all(cfg, T, payload=payload, fill=None)
    assert r["flags"] == 0
    check_partial_full_size(r, O.layout(r["idx"], cfg.E, cfg.N), ranks)


def test_combine_heavy_full_size():
    """Every token of all 16 source ranks."""
    _need(45)
    cfg = W.CONFIGS["combine_heavy"]
    _full_size(cfg, cfg.T)


def test_dsv3_decode_full_size():
    cfg = W.CONFIGS["dsv3_decode"]
    _full_size(cfg, cfg.T)


def test_kimi_combine_full_size():
    """Every token of 8 whole source ranks (of 64), the hottest-receiving
    one's senders included."""
    _need(100)
    cfg = W.CONFIGS["kimi_skewed"]
    _full_size(cfg, cfg.Tc, payload=False, ranks=[0, 9, 18, 27, 36, 45, 54, 63])

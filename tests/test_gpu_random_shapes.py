"""Seeded random problems through every entry point, against the oracle.

Each case draws a shape (N, T, H, E, k), a region mode (packed, fixed with
room, fixed and too small, fixed with early rows, sometimes too small), a
skewed routing with a few bad ids and repeated ids inside a token, token
rows with zero and extreme blocks, and expert outputs.  Then:
  - send + recv, combine send + recv and the pulling combine: every element
    against the oracle (counts, offsets, positions, row_src, fp8 bytes and
    scales, comb rows, outputs; rows nobody writes keep their fill);
  - the partial combine: every element against combine_partial and within
    its bound;
  - the direct dispatch and, where T*k <= 4096, both single launches: bit
    for bit against the two-call path's outputs and tables.
The oracle decides every expected value; the cases only widen the inputs."""
import numpy as np
import pytest
import torch

import combine_lds_atomic_amd as moe
import workloads as W
from oracle import moe_oracle as O

from gpu_harness import (check_full, check_partial_full, check_same_as_two_calls, log, run_all,  # noqa: E402
                         run_direct)

CASES = 24
EXTREME = list(range(100, 108))   # seeds of problems at the library's limits


def _draw(seed):
    rng = np.random.default_rng(0xD15C0 + seed)
    T = int(rng.choice([1, 7, 33, 100, 257, 600, 1100]))
    if seed >= 100:   # up to N = 256, E = 1024, k = 64, H = 32768, few tokens
        N = int(rng.choice([64, 128, 256]))
        L = int(rng.integers(1, 1024 // N + 1))
        k = int(rng.choice([1, 16, 33, 64]))
        k = min(k, N * L)
        T = int(rng.choice([1, 3, 9]))
    elif T < 1100:
        N = int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16, 32]))
        L = int(rng.integers(1, 9))
        k = int(rng.integers(1, min(N * L, 12) + 1))
    else:   # more than one routing chunk per rank (T*k > 4096), kept small
        N = int(rng.integers(1, 5))
        L = int(rng.integers((4 + N - 1) // N, 9))
        k = int(rng.integers(4, min(N * L, 12) + 1))
    E = N * L
    H = 128 * int(rng.integers(1, 24))
    if seed >= 100:
        H = int(rng.choice([128, 1152, 32768]))
        if seed == EXTREME[0]:          # the longest rows, one token per rank
            T, H = 1, 32768
        if N * T * k * H > 300 << 20:   # keep the oracle's arrays small
            H = 128
    # Skewed routing: Gumbel top-k over log-probabilities of a Zipf-like law.
    logp = -1.1 * np.log(1.0 + rng.permutation(E))
    keys = rng.gumbel(size=(N, T, E)) + logp
    idx = np.argsort(-keys, axis=2, kind="stable")[:, :, :k].astype(np.int32)
    if k >= 2:   # a few tokens name one expert twice
        dup = rng.random((N, T)) < 0.02
        idx[dup, 1] = idx[dup, 0]
    bad = rng.random((N, T, k)) < 0.01
    idx[bad] = rng.choice(np.array([-1, E, E + 7, 1 << 30, -(1 << 20)], np.int32), int(bad.sum()))
    w = rng.random((N, T, k)).astype(np.float32) + np.float32(0.05)
    w /= w.sum(axis=2, keepdims=True)
    # Token rows: N(0,1) with some zero blocks, tiny and huge blocks.
    x = rng.standard_normal((N, T, H)).astype(np.float32)
    nb = H // 128
    xb = x.reshape(N, T, nb, 128)
    kind = rng.random((N, T, nb))
    xb[kind < 0.03] = 0.0
    xb[(kind >= 0.03) & (kind < 0.05)] *= np.float32(1e-30)
    xb[(kind >= 0.05) & (kind < 0.07)] *= np.float32(1e30)
    mode = str(rng.choice(["packed", "fixed", "tight", "early"]))
    lay = O.layout(idx, E, N)
    R = C = 0
    if mode == "fixed":
        R = int(lay.recv_total.max()) + int(rng.integers(0, 20))
    elif mode == "tight":
        R = max(1, int(lay.recv_total.max()) - int(rng.integers(1, 20)))
    elif mode == "early":
        C = max(1, int(rng.integers(1, 2 * T * k // N + 2)))
        over = O.layout(idx, E, N, N * C + 10 ** 6, C).recv_off[:, N]
        R = max(N * C, int(N * C + over.max() + rng.integers(-15, 15)))
    return dict(N=N, T=T, H=H, E=E, k=k, idx=idx, w=w, x=O.bf16_round(x), R=R, C=C, mode=mode, seed=seed)


def test_draws_cover_the_modes():
    """The fixed seeds reach every region mode, bad ids and repeated ids."""
    draws = [_draw(i) for i in range(CASES)]
    assert {d["mode"] for d in draws} == {"packed", "fixed", "tight", "early"}
    assert any(((d["idx"] < 0) | (d["idx"] >= d["E"])).any() for d in draws)
    assert any(d["k"] >= 2 and (d["idx"][:, :, 0] == d["idx"][:, :, 1]).any() for d in draws)
    assert any(d["T"] * d["k"] > 4096 for d in draws) and any(d["T"] * d["k"] <= 4096 for d in draws)


@pytest.mark.gpu
@pytest.mark.parametrize("seed", list(range(CASES)) + EXTREME)
def test_random_problem(seed):
    d = _draw(seed)
    N, T, H, E, k, R, C = d["N"], d["T"], d["H"], d["E"], d["k"], d["R"], d["C"]
    log(f"\n[gpu] random seed={seed}: N={N} T={T} H={H} E={E} k={k} mode={d['mode']} R={R} C={C}")
    cfg = W.Config(f"rand{seed}", seed=0x5EED0000 + seed, N=N, T=T, H=H, E=E, k=k)
    x = torch.from_numpy(d["x"]).to(torch.bfloat16).cuda()
    r = run_all(cfg, T, R, idx=d["idx"], w=d["w"], x=x, early_rows=C)
    lay = O.layout(d["idx"], E, N, R, C)
    assert r["flags"] == lay.flags, (r["flags"], lay.flags)
    check_full(r, lay)
    check_partial_full(r, lay)
    calls = ["direct"] + (["direct_ll"] if T * k <= 4096 else [])
    for call in calls:
        check_same_as_two_calls(r, run_direct(r, call))
    if T * k <= 4096:   # the single-launch send half: same receive regions and positions
        B2 = moe.allocate(r["sh"], "cuda", combine=False, fill_rows=0x5A)
        idx_d = torch.from_numpy(np.ascontiguousarray(d["idx"])).cuda()
        moe.moe_dispatch_send_ll(r["sh"], x, idx_d, B2.recv_q, B2.recv_s, B2.send_pos, B2.ws)
        torch.cuda.synchronize()
        assert torch.equal(B2.send_pos, r["B"].send_pos)
        assert torch.equal(B2.recv_q, r["B"].recv_q)
        assert torch.equal(B2.recv_s.view(torch.int32), r["B"].recv_s.view(torch.int32))
        assert moe.moe_status(B2.ws) == lay.flags

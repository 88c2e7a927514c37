"""Pins for the CPU oracle (no GPU): each check is fixed by something other
than the oracle itself -- hand-worked fixtures, closed forms, a library
routine (torch's float8_e4m3fn / bfloat16 casts), invariants, or brute force."""
import json
import os
from collections import defaultdict

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- fp8 E4M3

def test_e4m3_golden_encode_decode():
    g = _load("e4m3fn_values.json")
    vals = np.array([v for v, _ in g["encode"]], np.float32)
    want = np.array([b for _, b in g["encode"]], np.uint8)
    got = O.e4m3fn_encode(vals)
    bad = [(float(v), int(a), int(b)) for v, a, b in zip(vals, got, want) if a != b]
    assert not bad, bad
    codes = np.array([c for c, _ in g["decode"]], np.uint8)
    dv = O.e4m3fn_decode(codes)
    for c, (code, v) in zip(dv, g["decode"]):
        assert c == v and np.signbit(c) == np.signbit(v), (code, c, v)
    assert np.isnan(O.e4m3fn_decode(np.array(g["nan_codes"], np.uint8))).all()
    assert O.e4m3fn_encode(np.float32(np.nan)) == 0x7F


def test_e4m3_roundtrip_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    fin = ~np.isnan(O.e4m3fn_decode(codes))
    back = O.e4m3fn_encode(O.e4m3fn_decode(codes[fin]).astype(np.float32))
    assert (back == codes[fin]).all()
    assert fin.sum() == 254


def _torch_e4m3(v):
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_matches_torch_on_reachable_domain():
    """torch's cast rounds to nearest-even like OFP8 but returns NaN above 464
    instead of saturating, so it pins |v| <= 464 (the quantiser never exceeds
    448 * (1 + 2^-23))."""
    rng = np.random.default_rng(1)
    grid = O.e4m3fn_decode(np.arange(256, dtype=np.uint8))
    grid = np.unique(np.abs(grid[~np.isnan(grid)]))
    mids = (grid[:-1] + grid[1:]) / 2                     # every rounding midpoint
    m32 = mids.astype(np.float32)
    near = np.concatenate([m32, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(1e9)),
                           grid.astype(np.float32), np.float32(464.0)[None]])
    rand = np.concatenate([
        rng.uniform(-464, 464, 2_000_000).astype(np.float32),
        (rng.standard_normal(1_000_000) * 2.0 ** rng.integers(-14, 8, 1_000_000)).astype(np.float32),
        rng.uniform(-2 ** -6, 2 ** -6, 500_000).astype(np.float32),
    ])
    v = np.concatenate([near, -near, rand])
    v = v[np.abs(v) <= 464]
    assert (O.e4m3fn_encode(v) == _torch_e4m3(v)).all()


# ---------------------------------------------------------------- bf16

def test_bf16_round_matches_torch():
    rng = np.random.default_rng(2)
    u = rng.integers(0, 2 ** 32, 2_000_000, dtype=np.uint64).astype(np.uint32)
    u = u[((u >> 23) & 0xFF) != 0xFF]                     # finite patterns only
    ties = ((rng.integers(0, 2 ** 16, 100_000).astype(np.uint32) << 16) | 0x8000).astype(np.uint32)
    ties = ties[((ties >> 23) & 0xFF) < 0xFE]
    v = np.concatenate([u, ties]).view(np.float32)
    ours = O.bf16_bits(O.bf16_round(v))
    ref = torch.from_numpy(v.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (ours == ref).all()


# ---------------------------------------------------------------- quantiser

def _bf16_rows(rng, R, H, scale=1.0):
    return O.bf16_round((rng.standard_normal((R, H)) * scale).astype(np.float32))


def test_quantize_matches_torch_division_and_cast():
    rng = np.random.default_rng(3)
    x = np.concatenate([_bf16_rows(rng, 64, 1024), _bf16_rows(rng, 8, 1024, 1e-3),
                        _bf16_rows(rng, 8, 1024, 1e3)])
    q, s = O.quantize_rows(x)
    xt = torch.from_numpy(x).view(-1, 8, 128)
    amax = xt.abs().amax(dim=2)
    st = amax / torch.tensor(448.0)
    qt = (xt / st[:, :, None]).to(torch.float8_e4m3fn).view(torch.uint8).reshape(x.shape).numpy()
    assert (s == st.numpy()).all()
    assert (q == qt).all()


def test_quantize_invariants():
    rng = np.random.default_rng(4)
    x = _bf16_rows(rng, 200, 2048)
    x[3, 128:256] = 0.0                                    # an all-zero block
    x[5, 0:128] = -0.0
    x[7, 256:384] = np.float32(2.0 ** -133)                # tiniest bfloat16 subnormal
    q, s = O.quantize_rows(x)
    assert s.dtype == np.float32 and q.dtype == np.uint8
    assert s[3, 1] == 0 and (q[3, 128:256] == 0).all()
    assert s[5, 0] == 0 and (q[5, 0:128] == 0).all()
    xb = x.reshape(200, 16, 128)
    qb = q.reshape(200, 16, 128)
    am = np.argmax(np.abs(xb), axis=2)
    top = np.take_along_axis(qb, am[:, :, None], axis=2)[:, :, 0]
    nz = s > 0
    assert ((top[nz] & 0x7F) == 0x7E).all()                # the block maximum maps to +-448
    assert (s[nz] == (np.abs(xb).max(axis=2)[nz] / np.float32(448))).all()
    # rounding error of the dequantised value
    dq = O.dequantize_rows(q, s)
    v = np.abs(x.astype(np.float64))
    sc = np.repeat(s.astype(np.float64), 128, axis=1)
    lim = np.where(v >= sc * 2.0 ** -6, v * 2.0 ** -4, sc * 2.0 ** -10) * (1 + 2.0 ** -20)
    assert (np.abs(dq - x) <= lim).all()
    # signs survive (a zero that rounds keeps its sign bit) outside all-zero blocks
    live = np.repeat(nz, 128, axis=1)
    assert ((q >> 7).astype(bool) == np.signbit(x))[live].all()


# ---------------------------------------------------------------- layout

def test_layout_golden_packed_and_fixed():
    g = _load("layout_tiny.json")
    idx = np.array(g["idx"])
    lay = O.layout(idx, g["E"], g["N"], 0)
    assert (lay.cnt == g["cnt"]).all()
    assert (lay.send_off == g["send_off"]).all()
    assert (lay.send_pos == g["send_pos"]).all()
    assert (lay.recv_off == g["recv_off"]).all()
    assert (lay.recv_total == g["recv_total"]).all()
    assert (lay.base == g["packed"]["base"]).all()
    assert (lay.exp_off == g["packed"]["exp_off"]).all()
    assert (O.row_src(lay) == g["packed"]["row_src"]).all()
    assert lay.recv_total.max() <= g["bound_rows"] and lay.flags == 0
    T = g["T"]
    rt = [None] * 12
    et = [None] * 12
    for s in range(2):
        for t in range(T):
            for j in range(2):
                rt[lay.recv_row[s, t, j]] = [s, t]
                et[lay.em_row[s, t, j]] = [s, t]
    assert rt == g["packed"]["recv_row_token"]
    assert et == g["packed"]["em_row_token"]
    fx = O.layout(idx, g["E"], g["N"], 8)
    assert (fx.base == g["fixed_R8"]["base"]).all() and fx.flags == 0
    rs = O.row_src(fx)
    assert (rs[g["fixed_R8"]["row_src_rows"]] == g["fixed_R8"]["row_src"]).all()
    assert (np.delete(rs, g["fixed_R8"]["row_src_rows"]) == -1).all()


def test_layout_golden_early_rows():
    g = _load("layout_tiny.json")
    idx = np.array(g["idx"])
    ex = g["fixed_R8_early2"]
    lay = O.layout(idx, g["E"], g["N"], 8, 2)
    assert lay.flags == 0
    assert (lay.recv_off == ex["recv_off"]).all()
    assert (lay.recv_total == g["recv_total"]).all()
    got = {}
    for s in range(2):
        for t in range(g["T"]):
            for j in range(2):
                got[str(int(lay.recv_row[s, t, j]))] = [s, t]
    assert got == ex["recv_row_token"]
    rs = O.row_src(lay)
    assert (rs[ex["row_src_rows"]] == ex["row_src"]).all()
    assert (np.delete(rs, ex["row_src_rows"]) == -1).all()
    ov = O.layout(idx, g["E"], g["N"], 5, 2)
    assert ov.flags == g["fixed_R5_early2_overflow"]["flags"]
    for s, t, j in g["fixed_R5_early2_overflow"]["dropped_slots"]:
        assert ov.recv_row[s, t, j] == -1
    assert (ov.recv_row >= 0).sum() == 10


@pytest.mark.parametrize("N,T,E,k,C,seed", [(4, 40, 16, 4, 3, 1), (3, 25, 6, 2, 1, 2), (5, 30, 20, 3, 0, 3),
                                            (2, 64, 8, 8, 40, 4)])
def test_layout_early_rows_closed_form(N, T, E, k, C, seed):
    """Region d's source-major rows are, for each sender s, its first
    min(c[s,d], C) rows at s*C.. in sender order, then its remaining rows in
    one run from N*C + (remaining rows of earlier senders); the expert-major
    rows do not depend on C."""
    rng = np.random.default_rng(seed)
    idx = _random_idx(rng, N, T, E, k)
    base = O.layout(idx, E, N)
    R = N * C + int(base.recv_total.max()) + 3
    lay = O.layout(idx, E, N, R, C)
    ref = O.layout(idx, E, N, R)
    assert lay.flags == 0
    assert (lay.em_row == ref.em_row).all() and (O.row_src(lay) == O.row_src(ref)).all()
    L = E // N
    c = np.zeros((N, N), np.int64)
    for s in range(N):
        for e in idx[s].reshape(-1):
            c[s, e // L] += 1
    for d in range(N):
        prior = 0
        for s in range(N):
            mine = [(int(lay.send_pos[s, t, j]), int(lay.recv_row[s, t, j]))
                    for t in range(T) for j in range(k) if idx[s, t, j] // L == d]
            rows = [r - d * R for _, r in sorted(mine)]          # in sender order
            m = min(c[s, d], C)
            assert rows[:m] == list(range(s * C, s * C + m))
            assert rows[m:] == list(range(N * C + prior, N * C + prior + c[s, d] - m))
            prior += c[s, d] - m


def _brute_layout(idx, E, N):
    """Independent dict-of-lists construction of the same layout."""
    _, T, k = idx.shape
    L = E // N
    groups = [defaultdict(list) for _ in range(N)]
    for s in range(N):
        for t in range(T):
            for j in range(k):
                e = int(idx[s, t, j])
                if 0 <= e < E:
                    groups[s][e].append((t, j))
    send_pos = -np.ones((N, T, k), np.int64)
    for s in range(N):
        p = 0
        for e in range(E):
            for (t, j) in groups[s][e]:
                send_pos[s, t, j] = p
                p += 1
    regions, experts = [], []
    for d in range(N):
        reg = []
        for s in range(N):
            for e in range(d * L, (d + 1) * L):
                reg += [(s, t, j) for (t, j) in groups[s][e]]
        regions.append(reg)
        em = []
        for e in range(d * L, (d + 1) * L):
            for s in range(N):
                em += [(s, t, j) for (t, j) in groups[s][e]]
        experts.append(em)
    return send_pos, regions, experts


@pytest.mark.parametrize("N,T,E,k,seed", [(1, 5, 4, 2, 0), (2, 6, 8, 3, 1), (4, 4, 8, 1, 2),
                                          (4, 6, 8, 3, 3), (2, 1, 2, 2, 4), (4, 6, 4, 3, 5)])
def test_layout_brute_force(N, T, E, k, seed):
    rng = np.random.default_rng(seed)
    idx = np.stack([[rng.choice(E, size=k, replace=False) for _ in range(T)] for _ in range(N)])
    lay = O.layout(idx, E, N, 0)
    sp, regions, experts = _brute_layout(idx, E, N)
    assert (lay.send_pos == sp).all()
    for d in range(N):
        for i, (s, t, j) in enumerate(regions[d]):
            assert lay.recv_row[s, t, j] == lay.base[d] + i
        for i, (s, t, j) in enumerate(experts[d]):
            assert lay.em_row[s, t, j] == lay.base[d] + i
        assert lay.recv_total[d] == len(regions[d])
        assert lay.exp_off[d, -1] == len(experts[d])


def _random_idx(rng, N, T, E, k, bias=None):
    logits = rng.standard_normal((N, T, E)) + (0 if bias is None else bias)
    return np.argsort(-logits, axis=2, kind="stable")[:, :, :k]


@pytest.mark.parametrize("N,T,E,k,skew", [(8, 64, 64, 4, False), (8, 64, 64, 8, True),
                                          (16, 33, 128, 8, True), (4, 100, 8, 8, False)])
def test_layout_invariants(N, T, E, k, skew):
    rng = np.random.default_rng(N * 1000 + T)
    bias = -np.log(rng.permutation(E) + 1.0) * 3 if skew else None
    idx = _random_idx(rng, N, T, E, k, bias)
    L = E // N
    lay = O.layout(idx, E, N, 0)
    assert (lay.cnt.sum(axis=1) == T * k).all()
    assert (lay.send_off[:, E] == T * k).all()
    assert (np.diff(lay.send_off, axis=1) == lay.cnt).all()
    for s in range(N):                                     # bijection onto [0, T*k)
        assert (np.sort(lay.send_pos[s].reshape(-1)) == np.arange(T * k)).all()
    for s in range(N):                                     # increasing in t inside a group
        for e in np.unique(idx[s]):
            tt, jj = np.nonzero(idx[s] == e)
            assert (np.diff(lay.send_pos[s, tt, jj]) > 0).all()
    assert lay.recv_total.sum() == N * T * k
    assert (lay.recv_total <= N * T * min(k, L)).all()       # tight bound
    assert (lay.recv_total <= N * T * max(k, L)).all()       # the pages' bound
    assert (lay.exp_off[:, L] == lay.recv_total).all()
    # every token appears exactly k times over all regions
    seen = np.zeros((N, T), np.int64)
    for s in range(N):
        np.add.at(seen[s], np.repeat(np.arange(T), k), 1)
    assert (seen == k).all()
    rows = np.concatenate([lay.recv_row.reshape(-1), lay.em_row.reshape(-1)])
    assert (np.sort(lay.recv_row.reshape(-1)) == np.arange(N * T * k)).all()
    assert (np.sort(lay.em_row.reshape(-1)) == np.arange(N * T * k)).all()
    del rows


def test_layout_bad_ids_dropped_and_flagged():
    idx = np.array([[[0, 5], [1, -1]], [[2, 3], [3, 1]]])   # 5 and -1 are outside [0, 4)
    lay = O.layout(idx, 4, 2, 0)
    assert lay.flags & O.FLAG_BADID
    assert lay.send_pos[0, 0, 1] == -1 and lay.send_pos[0, 1, 1] == -1
    assert lay.cnt.sum() == 6 and lay.recv_total.sum() == 6
    assert (lay.recv_row[lay.send_pos < 0] == -1).all()


def test_layout_fixed_region_overflow():
    rng = np.random.default_rng(9)
    idx = _random_idx(rng, 4, 16, 8, 2)
    idx[:, :, 0] = 0                                         # every token's slot 0 -> rank 0
    full = O.layout(idx, 8, 4, 0)
    R = int(full.recv_total.max()) - 3
    lay = O.layout(idx, 8, 4, R)
    assert lay.flags & O.FLAG_OVERFLOW
    ok = lay.recv_row >= 0
    assert (lay.recv_row[ok] < lay.base[lay.recv_row[ok] // R] + R).all()
    d = np.arange(4)[full.recv_total <= R]                    # regions that fit are unaffected
    for dd in d:
        m = (idx // 2 == dd)
        assert (lay.recv_row[m] - lay.base[dd] == full.recv_row[m] - full.base[dd]).all()


def test_duplicate_ids_in_a_token_get_separate_rows():
    idx = np.array([[[1, 1], [0, 1]]])
    lay = O.layout(idx, 2, 1, 0)
    assert (lay.send_pos == [[[1, 2], [0, 3]]]).all()


# ---------------------------------------------------------------- dispatch end to end

def test_dispatch_round_trip_dequantises_to_input():
    rng = np.random.default_rng(11)
    N, T, H, E, k = 4, 24, 512, 16, 4
    x = _bf16_rows(rng, N * T, H).reshape(N, T, H)
    idx = _random_idx(rng, N, T, E, k)
    lay = O.layout(idx, E, N, 0)
    rq, rs = O.dispatch_send(x, lay)
    xq, xs, rsrc = O.dispatch_recv(rq, rs, lay)
    q, s = O.quantize_rows(x.reshape(N * T, H))
    tok = rsrc // k            # s*T*k + p -> (s, p); p -> token through send_pos
    for i in range(xq.shape[0]):
        sr, p = divmod(int(rsrc[i]), T * k)
        t, j = [int(a[0]) for a in np.nonzero(lay.send_pos[sr] == p)]
        assert idx[sr, t, j] // (E // N) == np.searchsorted(lay.base, i, side="right") - 1
        assert (xq[i] == q[sr * T + t]).all() and (xs[i] == s[sr * T + t]).all()
    del tok
    dq = O.dequantize_rows(xq, xs)
    src_tok = np.array([divmod(int(r), T * k) for r in rsrc])
    back = np.array([x[sr, int(np.nonzero(lay.send_pos[sr] == p)[0][0])] for sr, p in src_tok])
    assert (np.abs(dq - back) <= np.abs(back) * 2.0 ** -4 + np.repeat(xs, 128, axis=1) * 2.0 ** -10 + 1e-30).all()


# ---------------------------------------------------------------- combine

def _combine_case(rng, N=4, T=16, H=256, E=16, k=4):
    idx = _random_idx(rng, N, T, E, k)
    lay = O.layout(idx, E, N, 0)
    logits = rng.standard_normal((N, T, k))
    w = np.exp(logits) / np.exp(logits).sum(axis=2, keepdims=True)
    return idx, lay, w.astype(np.float32)


def test_combine_one_hot_weights_return_the_chosen_row():
    rng = np.random.default_rng(12)
    N, T, H, k = 4, 16, 256, 4
    idx, lay, _ = _combine_case(rng, N, T, H, 16, k)
    rows = lay.total_rows
    y = O.bf16_bits(_bf16_rows(rng, rows, H))
    rsrc = O.row_src(lay)
    comb = O.combine_send(y, rsrc, N, T, k)
    for i in range(rows):                                   # combine_send is a pure permutation
        assert (comb[rsrc[i]] == y[i]).all()
    pick = rng.integers(0, k, (N, T))
    w = np.zeros((N, T, k), np.float32)
    np.put_along_axis(w, pick[:, :, None], 1.0, axis=2)
    out = O.combine_recv(comb, lay.send_pos, w, T, k)
    for s in range(N):
        for t in range(T):
            assert (out[s, t] == comb[s * T * k + lay.send_pos[s, t, pick[s, t]]]).all()


def test_combine_identity_returns_dequantised_input():
    """y := the dispatched rows themselves (dequantised, as bf16) and weights
    summing to one -> combine returns bf16(dequant(x)) to within 1 bf16 ulp."""
    rng = np.random.default_rng(13)
    N, T, H, E, k = 4, 16, 256, 16, 4
    x = _bf16_rows(rng, N * T, H).reshape(N, T, H)
    idx, lay, w = _combine_case(rng, N, T, H, E, k)
    rq, rs = O.dispatch_send(x, lay)
    xq, xs, rsrc = O.dispatch_recv(rq, rs, lay)
    y = O.bf16_bits(O.bf16_round(O.dequantize_rows(xq, xs).astype(np.float32)))
    out = O.bf16_from_bits(O.combine_recv(O.combine_send(y, rsrc, N, T, k), lay.send_pos, w, T, k))
    q, s = O.quantize_rows(x.reshape(N * T, H))
    ref = O.bf16_round(O.dequantize_rows(q, s).astype(np.float32)).reshape(N, T, H)
    ulp = np.ldexp(1.0, np.frexp(np.abs(ref).astype(np.float64))[1] - 8)
    assert (np.abs(out.astype(np.float64) - ref) <= ulp + 1e-38).all()
    assert (np.abs(out - x) <= np.abs(x) * 2.0 ** -3 + 1e-2).all()


def test_combine_fp64_brute_force_error_bound():
    rng = np.random.default_rng(14)
    N, T, H, E, k = 3, 10, 128, 6, 3
    idx, lay, w = _combine_case(rng, N, T, H, E, k)
    y = O.bf16_bits(_bf16_rows(rng, lay.total_rows, H))
    rsrc = O.row_src(lay)
    comb = O.combine_send(y, rsrc, N, T, k)
    out = O.bf16_from_bits(O.combine_recv(comb, lay.send_pos, w, T, k)).astype(np.float64)
    for s in range(N):
        for t in range(T):
            rows = [O.bf16_from_bits(comb[s * T * k + lay.send_pos[s, t, j]]).astype(np.float64) for j in range(k)]
            exact = sum(float(w[s, t, j]) * rows[j] for j in range(k))
            mag = sum(abs(float(w[s, t, j])) * np.abs(rows[j]) for j in range(k))
            ulp = np.ldexp(1.0, np.frexp(np.abs(exact))[1] - 8)
            lim = 0.5 * ulp + 2 * k * 2.0 ** -24 * mag + 1e-38
            assert (np.abs(out[s, t] - exact) <= lim).all()
            got1 = O.bf16_from_bits(O.combine_rows(np.stack([comb[s * T * k + lay.send_pos[s, t, j]] for j in range(k)]),
                                                   w[s, t]))
            assert (got1 == out[s, t]).all()


def test_combine_single_slot_unit_weight_is_exact():
    rng = np.random.default_rng(15)
    N, T, H, E, k = 2, 8, 128, 4, 1
    idx, lay, _ = _combine_case(rng, N, T, H, E, k)
    y = O.bf16_bits(_bf16_rows(rng, lay.total_rows, H))
    comb = O.combine_send(y, O.row_src(lay), N, T, k)
    out = O.combine_recv(comb, lay.send_pos, np.ones((N, T, 1), np.float32), T, k)
    assert (out.reshape(N * T, H) == comb[(np.arange(N)[:, None] * T + lay.send_pos[:, :, 0]).reshape(-1)]).all()


def test_combine_sums_in_slot_order():
    """The combine's float32 sum runs over slots 0..k-1 in that order.  Rows of
    2^24, 1 and -2^24 with unit weights (tests/golden/combine_slot_order.json,
    worked by hand) give sums that depend on the order of the additions: slot
    order gives the fixture's values, while the reversed order and the order
    of ascending expert id (the rows' order in the combine buffer) give others
    on some token."""
    g = _load("combine_slot_order.json")
    idx = np.array(g["idx"])
    N, T, k = idx.shape
    H, E = g["H"], g["E"]
    vals = np.array(g["y_slot_values"], np.float32)
    w = np.array(g["w"], np.float32)
    lay = O.layout(idx, E, N)
    y = np.zeros((lay.total_rows, H), np.uint16)
    for s in range(N):
        for t in range(T):
            for j in range(k):
                y[lay.em_row[s, t, j]] = O.bf16_bits(np.full(H, vals[s, t, j], np.float32))
    comb = O.combine_send(y, O.row_src(lay), N, T, k)
    out = O.bf16_from_bits(O.combine_recv(comb, lay.send_pos, w, T, k)).astype(np.float64)
    assert (out == np.array(g["out_slot_order"])[:, :, None]).all()
    for s in range(N):
        for t in range(T):
            rows = np.stack([y[lay.em_row[s, t, j]] for j in range(k)])
            assert (O.bf16_from_bits(O.combine_rows(rows, w[s, t])) == g["out_slot_order"][s][t]).all()
            # The fixture tells the orders apart: the same rows summed
            # reversed, or by expert id, give the fixture's other columns.
            rev = O.bf16_from_bits(O.combine_rows(rows[::-1], w[s, t]))
            by_e = O.bf16_from_bits(O.combine_rows(rows[np.argsort(idx[s, t])], w[s, t]))
            assert (rev == g["out_reversed_order"][s][t]).all()
            assert (by_e == g["out_expert_order"][s][t]).all()
    assert g["out_reversed_order"] != g["out_slot_order"] and g["out_expert_order"] != g["out_slot_order"]


def test_combine_skips_dropped_slots():
    rng = np.random.default_rng(16)
    N, T, H, E, k = 2, 4, 128, 4, 2
    idx = np.array([[[0, 9], [1, 2], [3, 0], [2, 1]], [[0, 1], [2, 3], [1, 0], [3, 2]]])
    lay = O.layout(idx, E, N, 0)
    y = O.bf16_bits(_bf16_rows(rng, lay.total_rows, H))
    comb = O.combine_send(y, O.row_src(lay), N, T, k)
    w = np.full((N, T, k), 0.5, np.float32)
    out = O.bf16_from_bits(O.combine_recv(comb, lay.send_pos, w, T, k))
    ref = O.bf16_round((np.float32(0.5) * O.bf16_from_bits(comb[lay.send_pos[0, 0, 0]])).astype(np.float32))
    assert (out[0, 0] == ref).all()


# ---------------------------------------------------------------- combine with send-side partial sums

def _partial_case(idx, w, y_token_values, H, E):
    """Rows of constant value per slot, placed in expert-major order."""
    idx = np.asarray(idx)
    N, T, k = idx.shape
    lay = O.layout(idx, E, N, 0)
    y = np.zeros((lay.total_rows, H), np.uint16)
    vals = np.asarray(y_token_values, np.float32)
    for s in range(N):
        for t in range(T):
            for j in range(k):
                if lay.em_row[s, t, j] >= 0:
                    y[lay.em_row[s, t, j]] = O.bf16_bits(np.full(H, vals[s, t, j], np.float32))
    return lay, y


def test_partial_golden_example():
    g = _load("combine_partial_example.json")
    lay, y = _partial_case(g["idx"], g["w"], g["y_slot_values"], g["H"], g["E"])
    w = np.asarray(g["w"], np.float32)
    comb, lead, out = O.combine_partial(y, g["idx"], lay, w)
    assert (lead == np.asarray(g["group_leaders"])).all()
    for s, rows in g["group_rows_bits"].items():
        for j, bits in rows.items():
            s_, j_ = int(s), int(j)
            assert (comb[s_ * g["T"] * g["k"] + lay.send_pos[s_, 0, j_]] == bits).all(), (s, j)
    assert (out[:, 0, :] == np.asarray(g["out_partial_bits"])).all()
    plain = O.combine_recv(O.combine_send(y, O.row_src(lay), g["N"], g["T"], g["k"]), lay.send_pos, w, g["T"], g["k"])
    assert (plain[:, 0, :] == np.asarray(g["out_plain_bits"])).all()


def test_partial_equals_plain_when_a_token_uses_one_rank():
    """All of a token's experts on one rank: one group, whose bf16 row is the
    plain combine's result, and re-rounding it changes nothing."""
    rng = np.random.default_rng(21)
    N, T, H, E, k = 4, 12, 256, 32, 4            # L = 8 experts per rank >= k
    L = E // N
    idx = np.zeros((N, T, k), np.int64)
    for s in range(N):
        for t in range(T):
            d = rng.integers(0, N)
            idx[s, t] = d * L + rng.choice(L, k, replace=False)
    lay = O.layout(idx, E, N, 0)
    w = rng.dirichlet(np.ones(k), (N, T)).astype(np.float32)
    y = O.bf16_bits(_bf16_rows(rng, lay.total_rows, H))
    comb, lead, out = O.combine_partial(y, idx, lay, w)
    assert (lead.sum(axis=2) == 1).all() and lead[:, :, 0].all()
    plain = O.combine_recv(O.combine_send(y, O.row_src(lay), N, T, k), lay.send_pos, w, T, k)
    assert (out == plain).all()


def test_partial_singleton_groups_closed_form():
    """One expert per rank (E = N), distinct experts per token: every slot is
    its own group, so out = bf16(sum_j bf16(fl32(w_j * y_j))) in slot order."""
    rng = np.random.default_rng(22)
    N, T, H, k = 6, 10, 128, 4
    idx = np.stack([np.stack([rng.choice(N, k, replace=False) for _ in range(T)]) for _ in range(N)])
    lay = O.layout(idx, N, N, 0)
    w = rng.dirichlet(np.ones(k), (N, T)).astype(np.float32)
    y = O.bf16_bits(_bf16_rows(rng, lay.total_rows, H))
    _, lead, out = O.combine_partial(y, idx, lay, w)
    assert lead.all()
    yv = O.bf16_from_bits(y[lay.em_row])                               # [N, T, k, H]
    p = O.bf16_round((w[..., None] * yv).astype(np.float32))
    acc = np.zeros((N, T, H), np.float32)
    for j in range(k):
        acc = (acc + p[:, :, j]).astype(np.float32)
    assert (out == O.bf16_bits(O.bf16_round(acc))).all()


def test_partial_unit_and_one_hot_weights_are_exact():
    rng = np.random.default_rng(23)
    N, T, H, E, k = 4, 16, 128, 16, 4
    idx = _random_idx(rng, N, T, E, k)
    lay = O.layout(idx, E, N, 0)
    y = O.bf16_bits(_bf16_rows(rng, lay.total_rows, H))
    pick = rng.integers(0, k, (N, T))
    w = np.zeros((N, T, k), np.float32)
    np.put_along_axis(w, pick[:, :, None], 1.0, axis=2)
    _, _, out = O.combine_partial(y, idx, lay, w)
    for s in range(N):
        for t in range(T):
            assert (out[s, t] == y[lay.em_row[s, t, pick[s, t]]]).all()


def test_partial_groups_are_the_distinct_ranks_of_a_token():
    rng = np.random.default_rng(24)
    N, T, H, E, k = 4, 30, 128, 16, 6
    idx = _random_idx(rng, N, T, E, k)
    idx[0, 0, 2] = 99                                                  # a dropped slot
    lay = O.layout(idx, E, N, 0)
    y = O.bf16_bits(_bf16_rows(rng, lay.total_rows, H))
    w = rng.dirichlet(np.ones(k), (N, T)).astype(np.float32)
    _, lead, _ = O.combine_partial(y, idx, lay, w)
    L = E // N
    for s in range(N):
        for t in range(T):
            ranks = [int(e) // L for e in idx[s, t] if 0 <= e < E]
            assert lead[s, t].sum() == len(set(ranks))
            for j in np.flatnonzero(lead[s, t]):                      # a leader is its rank's first slot
                assert [int(e) // L for e in idx[s, t][:j] if 0 <= e < E].count(int(idx[s, t, j]) // L) == 0


def test_partial_fp64_error_bound():
    """|out - sum_j w_j y_j| <= 2^-8 (|out| + sum_g |p_g|) + 2k 2^-24 sum_j |w_j y_j|:
    one bf16 rounding of each group row and of the result, float32 sums."""
    rng = np.random.default_rng(25)
    N, T, H, E, k = 4, 20, 128, 16, 6
    idx = _random_idx(rng, N, T, E, k)
    lay = O.layout(idx, E, N, 0)
    y = O.bf16_bits(_bf16_rows(rng, lay.total_rows, H))
    w = rng.dirichlet(np.ones(k), (N, T)).astype(np.float32)
    comb, lead, out = O.combine_partial(y, idx, lay, w)
    outf = O.bf16_from_bits(out).astype(np.float64)
    worst = 0.0
    for s in range(N):
        for t in range(T):
            rows = O.bf16_from_bits(y[lay.em_row[s, t]]).astype(np.float64)        # [k, H]
            ww = w[s, t].astype(np.float64)[:, None]
            exact = (ww * rows).sum(axis=0)
            mag = (np.abs(ww) * np.abs(rows)).sum(axis=0)
            pg = sum(np.abs(O.bf16_from_bits(comb[s * T * k + lay.send_pos[s, t, j]]).astype(np.float64))
                     for j in np.flatnonzero(lead[s, t]))
            lim = 2.0 ** -8 * (np.abs(outf[s, t]) + pg) + 2 * k * 2.0 ** -24 * mag + 2.0 ** -133
            err = np.abs(outf[s, t] - exact)
            assert (err <= lim).all()
            worst = max(worst, float((err / lim).max()))
    assert worst > 0.05          # the bound is not vacuous: some elements come near it


def test_partial_receive_sums_in_leader_order():
    """Groups are added in leader (slot) order: with rows 2^24, 1, -2^24 on three
    ranks and unit weights, float32 gives (2^24 + 1) - 2^24 = 0 in that order
    (2^24 + 1 rounds to 2^24) but 1 in the reverse order."""
    idx = np.array([[[0, 1, 2]], [[1, 2, 0]], [[2, 0, 1]]])       # N = E = 3: every slot its own group
    vals = np.array([[[2.0 ** 24, 1.0, -2.0 ** 24]]] * 3, np.float32)
    lay, y = _partial_case(idx, np.ones((3, 1, 3), np.float32), vals, 128, 3)
    _, lead, out = O.combine_partial(y, idx, lay, np.ones((3, 1, 3), np.float32))
    assert lead.all()
    assert (O.bf16_from_bits(out) == 0.0).all()


def test_partial_slots_without_a_row_take_no_part():
    """A slot whose row a full fixed region dropped behaves like a dropped id:
    the same leaders and the same output as the routing with that id removed."""
    rng = np.random.default_rng(26)
    N, T, H, E, k = 4, 24, 128, 8, 3
    idx = _random_idx(rng, N, T, E, k)
    idx[:, :, 0] = 0                                           # every token's slot 0 -> rank 0
    R = int(O.layout(idx, E, N).recv_total.max()) - 9
    lay = O.layout(idx, E, N, R)
    assert lay.flags & O.FLAG_OVERFLOW
    gone = lay.slot_valid & (lay.em_row < 0)
    assert gone.any()
    w = rng.dirichlet(np.ones(k), (N, T)).astype(np.float32)
    vals = rng.standard_normal((N, T, k)).astype(np.float32)
    lay_r, y_r = _partial_case(np.where(gone, -1, idx), w, vals, H, E)
    y = np.zeros((lay.total_rows, H), np.uint16)
    for s in range(N):
        for t in range(T):
            for j in range(k):
                if lay.em_row[s, t, j] >= 0:
                    y[lay.em_row[s, t, j]] = O.bf16_bits(np.full(H, vals[s, t, j], np.float32))
    _, lead, out = O.combine_partial(y, idx, lay, w)
    _, lead_r, out_r = O.combine_partial(y_r, np.where(gone, -1, idx), lay_r, w)
    assert (lead == lead_r).all() and (out == out_r).all()
    assert not (lead & gone).any()


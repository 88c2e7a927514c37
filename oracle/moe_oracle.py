"""CPU oracle for MoE expert-parallel dispatch / combine.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(the HIP library and its Python binding) never imports, links or calls it, and
this module imports nothing from the product path.

Everything here is the plain definition of what dispatch and combine compute,
written for a reader checking it against the sources by eye: NumPy
primitives (bincount, cumsum, stable argsort, fancy indexing) and float32 /
float64 element-wise arithmetic; no blocking, fusion or reordering.

Sources (web pages; cited by title and section):

* [EFA] "Enabling trillion-parameter models on AWS EFA" (Perplexity, 2025),
  sections "Introduction", "Send and receive buffers", "Dispatch and combine",
  "Evaluation: dispatch/combine latency".
* [OFP8] OCP 8-bit Floating Point Specification (OFP8), E4M3 encoding:
  bias 7, 3 mantissa bits, no infinities, S.1111.111 is NaN, max normal 448,
  subnormals m * 2^-9.

Readings adopted where the pages leave a step open (each is restated where it
is used):

* experts live on ranks in contiguous blocks: owner(e) = e // L, L = E // N;
* inside one (source rank, expert) group, slots keep ascending (token, slot)
  order, which makes every position unique;
* a receive region holds one contiguous block per source rank, sources in
  ascending order; inside a block the sender's order (expert, token, slot);
* the grouped-GEMM layout is expert-major, (source, token, slot) ascending
  inside an expert, no per-expert padding;
* one row per (token, slot): a token that picks two experts on one rank
  arrives there twice;
* slot ids outside [0, E) are dropped (not counted, not sent, no combine
  contribution) and raise the BADID flag;
* fp8 payload: e4m3fn, one fp32 scale per 128 consecutive elements of a row,
  scale = fl32(amax / 448), q = e4m3fn_rne_satfinite(fl32(x / scale)), and a
  block whose amax is 0 gets scale 0 and all-zero bytes;
* combine: out = bf16_rne(sum_j fl32(w_j * y_j)) accumulated in float32 in
  slot order 0..k-1 with no division by sum(w) (the router's softmax weights
  already sum to one, so the sum is the weighted average).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# Flag bits, same meaning as the library's sticky error word.
FLAG_BADID = 1      # a slot id outside [0, E) was dropped
FLAG_OVERFLOW = 2   # a fixed-size receive region could not hold its rows
FLAG_BOUND = 4      # a region count exceeded N*T*max(k, E/N)

E4M3_MAX = 448.0
SCALE_BLOCK = 128


# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------

def _round_binade(a: np.ndarray, mant_bits: int, emin: int):
    """Round non-negative float64 values to a binary format with ``mant_bits``
    explicit mantissa bits and minimum normal exponent ``emin``; ties to even.

    Returns (e, m): the rounded value is m * 2**(e - mant_bits), with
    2**mant_bits <= m < 2**(mant_bits+1) for normals and m < 2**mant_bits in
    the subnormal range (e == emin).  Pure float64 arithmetic on powers of two,
    so every step is exact except the single rint.
    """
    _, ex = np.frexp(a)                    # a = f * 2**ex, 0.5 <= f < 1 (exact)
    e = np.maximum(ex.astype(np.int64) - 1, emin)   # binade exponent, clamped at the subnormal range
    ulp = np.ldexp(1.0, e - mant_bits)     # value spacing inside that binade
    m = np.rint(a / ulp)                   # round half to even
    carry = m == float(1 << (mant_bits + 1))
    e = np.where(carry, e + 1, e)
    m = np.where(carry, float(1 << mant_bits), m)
    return e, m.astype(np.int64)


def e4m3fn_encode(v) -> np.ndarray:
    """float32 -> OCP E4M3 byte, round to nearest even, saturating to +-448.

    [OFP8] E4M3: bias 7; normals (1 + m/8) * 2**(E - 7) for E in 1..15 (E=15,
    m=7 is NaN); subnormals m * 2**-9; sign of zero kept.  Magnitudes that
    round above 448 saturate to 448 (the "satfinite" conversion); NaN maps to
    S.1111.111.
    """
    v = np.asarray(v, dtype=np.float32)
    sign = (np.signbit(v).astype(np.uint16) << 7)
    a = np.abs(v).astype(np.float64)
    nan = np.isnan(v)
    a = np.where(nan, 0.0, a)
    with np.errstate(over="ignore", invalid="ignore"):
        e, m = _round_binade(np.minimum(a, 1e30), 3, -6)
    sat = (e > 8) | ((e == 8) & (m > 14))
    e = np.where(sat, 8, e)
    m = np.where(sat, 14, m)
    normal = m >= 8
    exp_field = np.where(normal, e + 7, 0)
    mant = np.where(normal, m - 8, m)
    byte = sign | (exp_field.astype(np.uint16) << 3) | mant.astype(np.uint16)
    byte = np.where(nan, sign | 0x7F, byte)
    return byte.astype(np.uint8)


def e4m3fn_decode(b) -> np.ndarray:
    """OCP E4M3 byte -> float64 value ([OFP8] E4M3 table)."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    s = np.where(b & 0x80, -1.0, 1.0)
    ef = (b >> 3) & 0xF
    mf = b & 0x7
    val = np.where(ef == 0, mf * 2.0 ** -9, (1.0 + mf / 8.0) * np.ldexp(1.0, ef - 7))
    val = np.where((ef == 15) & (mf == 7), np.nan, val)
    return s * val


def bf16_round(v) -> np.ndarray:
    """float32 -> nearest bfloat16 (ties to even), returned as float32 values.

    bfloat16: 7 explicit mantissa bits, minimum normal exponent -126 (the same
    exponent range as float32).  Values that round past the largest finite
    bfloat16 become infinite; NaN stays NaN.
    """
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v).astype(np.float64)
    fin = np.isfinite(a)
    with np.errstate(over="ignore", invalid="ignore"):
        e, m = _round_binade(np.where(fin, a, 0.0), 7, -126)
        r = np.ldexp(m.astype(np.float64), e - 7)
        r = np.where(fin, r, a)
        out = np.where(np.signbit(v), -r, r).astype(np.float32)
    return np.where(np.isnan(v), np.float32(np.nan), out)


def bf16_bits(v32) -> np.ndarray:
    """bfloat16-representable float32 values -> their 16-bit patterns."""
    v32 = np.ascontiguousarray(v32, dtype=np.float32)
    return (v32.view(np.uint32) >> 16).astype(np.uint16)


def bf16_from_bits(u16) -> np.ndarray:
    """16-bit bfloat16 patterns -> float32 values (exact widening)."""
    u16 = np.ascontiguousarray(u16, dtype=np.uint16)
    return (u16.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------
# O4: block-scaled fp8 quantisation ([EFA] "Evaluation": block-scaled fp8
# dispatch; scale granularity and rule as stated in the module header)
# ---------------------------------------------------------------------------

def quantize_rows(x) -> tuple[np.ndarray, np.ndarray]:
    """x: float32 [R, H] holding bfloat16 values, H % 128 == 0.

    Returns q uint8 [R, H] and scales float32 [R, H // 128].
    """
    x = np.asarray(x, dtype=np.float32)
    R, H = x.shape
    assert H % SCALE_BLOCK == 0
    xb = x.reshape(R, H // SCALE_BLOCK, SCALE_BLOCK)
    amax = np.max(np.abs(xb), axis=2)                           # exact
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)    # one IEEE fp32 division
    zero = amax == 0
    with np.errstate(divide="ignore", invalid="ignore"):
        v = (xb / np.where(zero, np.float32(1), scale)[:, :, None]).astype(np.float32)
    q = e4m3fn_encode(v)
    q[zero] = 0
    scale[zero] = 0.0
    return q.reshape(R, H), scale


def dequantize_rows(q, scale) -> np.ndarray:
    """Inverse map used only by invariants: value = decode(q) * scale (float64)."""
    R, H = q.shape
    d = e4m3fn_decode(q).reshape(R, H // SCALE_BLOCK, SCALE_BLOCK)
    return (d * np.asarray(scale, np.float64)[:, :, None]).reshape(R, H)


# ---------------------------------------------------------------------------
# O1-O3, O5, O6: routing layout ([EFA] "Send and receive buffers",
# "Dispatch and combine")
# ---------------------------------------------------------------------------

@dataclass
class Layout:
    N: int
    T: int
    E: int
    k: int
    L: int
    region_rows: int            # 0 = packed regions, R > 0 = region d at rows [d*R, d*R + R)
    early_rows: int             # C: private rows per sender at the start of every fixed region (0 = none)
    cnt: np.ndarray             # [N, E]  tokens of source s routed to expert e
    send_off: np.ndarray        # [N, E+1] exclusive scan of cnt[s] over experts
    send_pos: np.ndarray        # [N, T, k] position of each slot in its sender's order; -1 = dropped
    recv_off: np.ndarray        # [N(d), N(s)+1] start of source s's block inside region d (of its rows beyond
                                #                the early rows, counted from row N*C, when C > 0)
    recv_total: np.ndarray      # [N]     rows destined to region d
    base: np.ndarray            # [N+1]   first physical row of region d (base[N] = rows in use / allocated)
    exp_off: np.ndarray         # [N(d), L+1] expert offsets inside region d (grouped-GEMM layout)
    src_in_exp: np.ndarray      # [N+1, E] rows of expert e that come from sources before s
    slot_valid: np.ndarray      # [N, T, k] bool: the slot was dispatched
    recv_row: np.ndarray        # [N, T, k] physical row in the source-major receive regions (-1 if not written)
    em_row: np.ndarray          # [N, T, k] physical row in the expert-major output (-1 if not written)
    flags: int

    @property
    def total_rows(self) -> int:
        """Rows the receive / expert-major arrays must hold."""
        return self.N * self.T * self.k if self.region_rows == 0 else self.N * self.region_rows


def layout(idx, E: int, N: int, region_rows: int = 0, early_rows: int = 0) -> Layout:
    """Everything dispatch decides from the routing alone.

    idx: int [N, T, k] expert chosen by slot j of token t on source rank s.
    early_rows: C > 0 reserves, at the start of every fixed region, C private
    rows per sender ([EFA] "Send and receive buffers": a little private
    per-sender space on every receiver lets some tokens go out with the
    routing information, before the exchange).  Reading: sender s's first C
    rows for region d (in its sender order) go to rows s*C .. s*C + C - 1 of
    the region, a place the sender knows without the exchange; its further
    rows follow from row N*C, stacked by source as without early rows.  Only
    with fixed regions (a packed region's start depends on the exchange), and
    N*C <= R.
    """
    idx = np.asarray(idx, dtype=np.int64)
    assert idx.ndim == 3 and idx.shape[0] == N
    C = early_rows
    assert C == 0 or (region_rows > 0 and N * C <= region_rows)
    _, T, k = idx.shape
    assert E % N == 0
    L = E // N
    flags = 0

    valid = (idx >= 0) & (idx < E)
    if not valid.all():
        flags |= FLAG_BADID

    # O1 per-expert counts of each source rank.
    cnt = np.zeros((N, E), np.int64)
    for s in range(N):
        cnt[s] = np.bincount(idx[s][valid[s]], minlength=E)

    # O2 exclusive scan over experts; experts of one destination rank are
    # contiguous, so the same scan gives the per-rank and per-expert offsets.
    send_off = np.zeros((N, E + 1), np.int64)
    send_off[:, 1:] = np.cumsum(cnt, axis=1)

    # O3 stable positions: ordering a sender's valid slots by expert with a
    # stable sort puts slot (t, j) at send_off[s, e] + (number of earlier slots,
    # in (token, slot) order, that chose the same expert).
    send_pos = np.full((N, T, k), -1, np.int64)
    for s in range(N):
        flat = idx[s].reshape(-1)
        ok = np.flatnonzero(valid[s].reshape(-1))
        order = ok[np.argsort(flat[ok], kind="stable")]
        sp = send_pos[s].reshape(-1)
        sp[order] = np.arange(order.size)

    # O5 receive regions: c[s, d] rows go from s to d, stacked by source (with
    # early rows: only the rows beyond each sender's first C).
    c = np.add.reduceat(cnt, np.arange(0, E, L), axis=1) if E > 0 else cnt   # [N(s), N(d)]
    over = np.maximum(c - C, 0)
    recv_off = np.zeros((N, N + 1), np.int64)
    recv_off[:, 1:] = np.cumsum(over.T, axis=1)         # scan over sources, per destination
    recv_total = c.sum(axis=0)
    bound = N * T * max(k, L)
    if (recv_total > bound).any():
        flags |= FLAG_BOUND
    base = np.zeros(N + 1, np.int64)
    if region_rows == 0:
        base[1:] = np.cumsum(recv_total)
    else:
        base[:] = np.arange(N + 1) * region_rows
        if (recv_total > region_rows).any():
            flags |= FLAG_OVERFLOW

    # O6 expert-major layout inside each destination.
    exp_cnt = cnt.sum(axis=0)                               # [E]
    exp_off = np.zeros((N, L + 1), np.int64)
    exp_off[:, 1:] = np.cumsum(exp_cnt.reshape(N, L), axis=1)
    src_in_exp = np.zeros((N + 1, E), np.int64)
    src_in_exp[1:] = np.cumsum(cnt, axis=0)

    # Per-slot destination rows.
    e = np.where(valid, idx, 0)
    s_of = np.broadcast_to(np.arange(N)[:, None, None], idx.shape)
    d = e // L
    l = e - d * L
    u = send_pos - send_off[s_of, d * L]                # index inside the (source, destination) block
    in_region = np.where(u < C, s_of * C + u, N * C + recv_off[d, s_of] + (u - C))
    in_em = exp_off[d, l] + src_in_exp[s_of, e] + (send_pos - send_off[s_of, e])
    # A fixed region keeps the rows that fit it: a source-major row exists if
    # its region row is below R; an expert-major row exists if its own index
    # and its source-major row are both below R.
    if region_rows == 0:
        recv_fits = em_fits = valid
    else:
        recv_fits = valid & (in_region < region_rows)
        em_fits = recv_fits & (in_em < region_rows)
        if (recv_fits != valid).any():
            flags |= FLAG_OVERFLOW
    recv_row = np.where(recv_fits, base[d] + in_region, -1)
    em_row = np.where(em_fits, base[d] + in_em, -1)

    return Layout(N=N, T=T, E=E, k=k, L=L, region_rows=region_rows, early_rows=C, cnt=cnt,
                  send_off=send_off, send_pos=send_pos, recv_off=recv_off,
                  recv_total=recv_total, base=base, exp_off=exp_off,
                  src_in_exp=src_in_exp, slot_valid=valid, recv_row=recv_row,
                  em_row=em_row, flags=flags)


def row_src(lay: Layout) -> np.ndarray:
    """[total_rows] for each expert-major row, the flat combine row of its slot:
    s*T*k + send_pos (the place the row returns to); -1 for rows not written."""
    out = np.full(lay.total_rows, -1, np.int64)
    s_of = np.broadcast_to(np.arange(lay.N)[:, None, None], lay.send_pos.shape)
    ok = lay.em_row >= 0
    out[lay.em_row[ok]] = (s_of * lay.T * lay.k + lay.send_pos)[ok]
    return out


def region_rows_used(lay: Layout) -> np.ndarray:
    """[N] rows actually written in each region (recv_total clipped to capacity)."""
    if lay.region_rows == 0:
        return lay.recv_total.copy()
    return np.minimum(lay.recv_total, lay.region_rows)


# ---------------------------------------------------------------------------
# Dispatch ([EFA] "Dispatch and combine": send packs per-peer blocks, receive
# shuffles into the grouped-GEMM input)
# ---------------------------------------------------------------------------

def dispatch_send(x, lay: Layout):
    """x: float32 [N, T, H] (bfloat16 values).

    Returns the receive regions (q uint8 [rows, H], scales float32 [rows, H/128]);
    rows not written by any slot are left zero here (the library leaves them
    untouched)."""
    N, T, H = x.shape
    q, sc = quantize_rows(x.reshape(N * T, H))
    rows = lay.total_rows
    recv_q = np.zeros((rows, H), np.uint8)
    recv_s = np.zeros((rows, H // SCALE_BLOCK), np.float32)
    tok = np.broadcast_to((np.arange(N)[:, None] * T + np.arange(T)[None, :])[:, :, None], lay.send_pos.shape)
    ok = lay.recv_row >= 0
    recv_q[lay.recv_row[ok]] = q[tok[ok]]
    recv_s[lay.recv_row[ok]] = sc[tok[ok]]
    return recv_q, recv_s


def dispatch_recv(recv_q, recv_s, lay: Layout):
    """Source-major receive regions -> expert-major rows + row_src."""
    x_q = np.zeros_like(recv_q)
    x_s = np.zeros_like(recv_s)
    ok = lay.em_row >= 0
    x_q[lay.em_row[ok]] = recv_q[lay.recv_row[ok]]
    x_s[lay.em_row[ok]] = recv_s[lay.recv_row[ok]]
    return x_q, x_s, row_src(lay)


# ---------------------------------------------------------------------------
# Combine ([EFA] "Introduction": combine returns each token's weighted
# average; "Dispatch and combine": one write per peer, then accumulate on the
# receive side)
# ---------------------------------------------------------------------------

def combine_send(y_em, rsrc, N: int, T: int, k: int):
    """y_em: bfloat16 bits uint16 [rows, H] in expert-major order.

    Returns comb uint16 [N*T*k, H]: comb[row_src[i]] = y_em[i]; rows no slot
    returns to stay zero here (the library writes zeros only for the rows of
    valid slots that a full fixed region dropped, and leaves positions no
    valid slot has untouched)."""
    rows, H = y_em.shape
    comb = np.zeros((N * T * k, H), np.uint16)
    ok = rsrc >= 0
    comb[rsrc[ok]] = y_em[ok]
    return comb


def combine_recv(comb, send_pos, w, T: int, k: int):
    """comb uint16 [N*T*k, H] (bfloat16 bits), send_pos [N,T,k], w float32 [N,T,k].

    out[s, t] = bf16_rne(acc), acc = 0; for j in 0..k-1 (dropped slots skipped):
    acc = fl32(acc + fl32(w[s,t,j] * y[s,t,j])).  Returns uint16 [N, T, H]."""
    N = send_pos.shape[0]
    H = comb.shape[1]
    w = np.asarray(w, np.float32)
    acc = np.zeros((N, T, H), np.float32)
    for j in range(k):
        sp = send_pos[:, :, j]
        ok = sp >= 0
        flat = (np.arange(N)[:, None] * T * k + np.where(ok, sp, 0))
        y = bf16_from_bits(comb[flat.reshape(-1)]).reshape(N, T, H)
        term = (w[:, :, j][:, :, None] * y).astype(np.float32)
        acc = np.where(ok[:, :, None], (acc + term).astype(np.float32), acc)
    return bf16_bits(bf16_round(acc))


def combine_rows(y_rows, w_rows):
    """One token at a time: y_rows uint16 [k, H] (slot order), w_rows float32 [k].
    Same arithmetic as combine_recv; used for sampled checks at full size."""
    acc = np.zeros(y_rows.shape[1], np.float32)
    for j in range(y_rows.shape[0]):
        acc = (acc + (np.float32(w_rows[j]) * bf16_from_bits(y_rows[j])).astype(np.float32)).astype(np.float32)
    return bf16_bits(bf16_round(acc))


# ---------------------------------------------------------------------------
# Combine with send-side partial accumulation
# ---------------------------------------------------------------------------
# [EFA] "Evaluation: dispatch/combine latency": accumulating a token's rows on
# the send side of combine reduces the data transferred, possibly at some cost
# in accuracy.  Readings (the page gives the idea, not the arithmetic):
#   * a group is the set of a token's slots whose rows sit on one destination
#     rank (owner(e) = e // L), counting only slots that have an expert-major
#     row; the group's first slot is its leader;
#   * the sending (expert) rank sums the group in float32 in slot order,
#     acc = fl32(acc + fl32(w_j * y_j)) with no fused multiply-add (the
#     weights travel with the token), and ships bf16_rne(acc) as one row,
#     stored where the leader's row would return (s*T*k + send_pos of the
#     leader);
#   * the receiving (source) rank adds the group rows in float32 in leader
#     order and rounds once: out = bf16_rne(sum_g float(p_g)).

def partial_token(y_rows, w_rows, dest, part):
    """One token.  y_rows uint16 [k, H] bfloat16 bits in slot order, w_rows
    float32 [k], dest int [k] the rank holding each slot's row, part bool [k]
    whether the slot has a row.

    Returns (groups, out): groups is a list of (leader slot, p uint16 [H]) in
    leader order; out uint16 [H]."""
    k, H = y_rows.shape
    groups = []
    done = set()
    for j in range(k):
        if not part[j] or dest[j] in done:
            continue
        done.add(dest[j])
        acc = np.zeros(H, np.float32)
        for m in range(j, k):
            if part[m] and dest[m] == dest[j]:
                term = (np.float32(w_rows[m]) * bf16_from_bits(y_rows[m])).astype(np.float32)
                acc = (acc + term).astype(np.float32)
        groups.append((j, bf16_bits(bf16_round(acc))))
    acc = np.zeros(H, np.float32)
    for _, p in groups:
        acc = (acc + bf16_from_bits(p)).astype(np.float32)
    return groups, bf16_bits(bf16_round(acc))


def combine_partial(y_em, idx, lay: Layout, w):
    """Send-side partial combine of every token.  y_em uint16 [rows, H]
    (expert-major bfloat16 bits), idx [N, T, k], w float32 [N, T, k].

    Returns (comb, lead, out): comb uint16 [N*T*k, H] holds each group's row
    at its leader's return position (other rows zero; the library leaves
    them untouched), lead bool [N, T, k] marks leaders, out uint16 [N, T, H]."""
    N, T, k = lay.N, lay.T, lay.k
    H = y_em.shape[1]
    idx = np.asarray(idx, np.int64)
    w = np.asarray(w, np.float32)
    part = lay.em_row >= 0
    dest = np.where(lay.slot_valid, idx, 0) // lay.L
    comb = np.zeros((N * T * k, H), np.uint16)
    lead = np.zeros((N, T, k), bool)
    out = np.zeros((N, T, H), np.uint16)
    for s in range(N):
        for t in range(T):
            rows = np.zeros((k, H), np.uint16)
            pj = part[s, t]
            rows[pj] = y_em[lay.em_row[s, t][pj]]
            groups, out[s, t] = partial_token(rows, w[s, t], dest[s, t], pj)
            for j, p in groups:
                lead[s, t, j] = True
                comb[s * T * k + lay.send_pos[s, t, j]] = p
    return comb, lead, out


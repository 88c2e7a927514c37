"""Device buffers for one dispatch / combine problem, allocated with torch
(device memory and streams are all torch is used for)."""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import moe_recv_rows, moe_shape, moe_workspace_bytes, moe_workspace_init


@dataclass
class Buffers:
    shape: moe_shape
    rows: int
    ws: torch.Tensor            # uint8 workspace
    send_pos: torch.Tensor      # int32 [N, T, k]
    exp_off: torch.Tensor       # int32 [N, L+1]
    row_src: torch.Tensor       # int32 [rows]
    recv_q: torch.Tensor | None = None   # uint8 [rows, H]   (e4m3fn bytes)
    recv_s: torch.Tensor | None = None   # float32 [rows, H/128]
    x_q: torch.Tensor | None = None      # uint8 [rows, H]
    x_s: torch.Tensor | None = None      # float32 [rows, H/128]
    comb: torch.Tensor | None = None     # bfloat16 [N, T*k, H]
    out: torch.Tensor | None = None      # bfloat16 [N, T, H]


def allocate(sh: moe_shape, device="cuda", payload: bool = True, combine: bool = True,
             fill_rows: int | None = None) -> Buffers:
    """Allocate every array the four calls need for `sh`.

    payload=False skips the fp8 receive / expert-major arrays (layout-only
    dispatch); combine=False skips comb and out.  `fill_rows`, if given, fills
    the row arrays with that byte/int so untouched rows are recognisable."""
    rows = moe_recv_rows(sh)
    N, T, H, E, k = sh.N, sh.T, sh.H, sh.E, sh.k
    L = E // N
    ws = torch.empty(moe_workspace_bytes(sh), dtype=torch.uint8, device=device)
    moe_workspace_init(sh, ws)
    b = Buffers(shape=sh, rows=rows, ws=ws,
                send_pos=torch.empty((N, T, k), dtype=torch.int32, device=device),
                exp_off=torch.empty((N, L + 1), dtype=torch.int32, device=device),
                row_src=torch.full((rows,), -7 if fill_rows is None else fill_rows, dtype=torch.int32, device=device))
    if payload:
        b.recv_q = torch.empty((rows, H), dtype=torch.uint8, device=device)
        b.recv_s = torch.empty((rows, H // 128), dtype=torch.float32, device=device)
        b.x_q = torch.empty((rows, H), dtype=torch.uint8, device=device)
        b.x_s = torch.empty((rows, H // 128), dtype=torch.float32, device=device)
        if fill_rows is not None:
            for t in (b.recv_q, b.x_q):
                t.fill_(fill_rows & 0xFF)
            for t in (b.recv_s, b.x_s):
                t.fill_(float(fill_rows))
    if combine:
        b.comb = torch.empty((N, T * k, H), dtype=torch.bfloat16, device=device)
        b.out = torch.empty((N, T, H), dtype=torch.bfloat16, device=device)
    return b

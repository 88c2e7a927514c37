"""Exhaustive quantiser-domain sweep on the GPU, through moe_dispatch_send.

Every (x, amax) pair of positive finite bfloat16 values with x <= amax -- the
whole domain the block quantiser's output depends on -- with random signs,
checked bit for bit (fp8 bytes and fp32 scales) against digests the oracle
wrote (tests/golden/make_quant_sweep.py)."""
import json
import os

import numpy as np
import pytest
import torch

import quant_sweep as S

pytestmark = pytest.mark.gpu

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "quant_sweep_digests.json")


def _first_mismatch(c, got_q, got_s):
    from oracle import moe_oracle as O
    x = S.chunk_tokens(c)
    for r0 in range(0, S.ROWS_PER_CHUNK, 256):
        q, s = O.quantize_rows(O.bf16_from_bits(x[r0:r0 + 256]))
        bad = np.argwhere(q != got_q[r0:r0 + 256])
        if bad.size:
            r, col = bad[0]
            blk = x[r0 + r, col // 128 * 128:(col // 128 + 1) * 128]
            amax = int(np.max(blk & 0x7FFF))
            return (f"chunk {c} row {r0 + r} col {col}: x=0x{int(x[r0 + r, col]):04x} amax=0x{amax:04x} "
                    f"got 0x{int(got_q[r0 + r, col]):02x} want 0x{int(q[r, col]):02x}")
        bad = np.argwhere(s.view(np.uint32) != got_s[r0:r0 + 256].view(np.uint32))
        if bad.size:
            r, b = bad[0]
            return f"chunk {c} row {r0 + r} scale block {b}: got {got_s[r0 + r, b]!r} want {s[r, b]!r}"
    return f"chunk {c}: digests differ but no element does"


def test_quantiser_exhaustive_sweep():
    import combine_lds_atomic_amd as moe
    gold = json.load(open(GOLD))
    assert gold["H"] == S.H and gold["rows_per_chunk"] == S.ROWS_PER_CHUNK and gold["chunks"] == S.n_chunks()
    sh = moe.shape(1, S.ROWS_PER_CHUNK, S.H, 1, 1)
    B = moe.allocate(sh, "cuda", combine=False)
    idx = torch.zeros((1, S.ROWS_PER_CHUNK, 1), dtype=torch.int32, device="cuda")
    for c in range(S.n_chunks()):
        x = torch.from_numpy(S.chunk_tokens(c).view(np.int16)).view(torch.bfloat16).cuda().reshape(1, -1, S.H)
        moe.moe_dispatch_send(sh, x, idx, B.recv_q, B.recv_s, B.send_pos, B.ws)
        got_q, got_s = B.recv_q.cpu().numpy(), B.recv_s.cpu().numpy()
        want = gold["digests"][c]
        if S.digest(got_q) != want["q_sha256"] or S.digest(got_s) != want["scale_sha256"]:
            pytest.fail(_first_mismatch(c, got_q, got_s))
        print(f"chunk {c + 1}/{S.n_chunks()} bit-exact", flush=True)
    assert moe.moe_status(B.ws) == 0

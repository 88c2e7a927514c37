"""moe_stream, the plain fan-out (both grid forms) and reduction streams that bench.py times as
the pack's and the receive-side sum's achievable rates: every stored byte is
the XOR its definition in include/moe_streams.h names, at sizes that leave ragged
workgroup chunks and partial unit groups."""
import numpy as np
import pytest
import torch

from combine_lds_atomic_amd import streams as moe

pytestmark = pytest.mark.gpu

from gpu_harness import log  # noqa: E402


def _units(n, seed):
    g = np.random.default_rng(seed)
    return g.integers(0, 2**32, size=(n, 4), dtype=np.uint32)


@pytest.mark.parametrize("pattern", [moe.STREAM_FANOUT, moe.STREAM_FANOUT_ONESHOT])
@pytest.mark.parametrize("k", [1, 3, 4, 8])
@pytest.mark.parametrize("n16", [1, 4095, 1_000_003])
def test_fanout(pattern, k, n16):
    log(f"moe_stream fan-out pattern={pattern} k={k} n16={n16}")
    src = _units(2 * n16, n16 + k)
    sentinel = np.uint32(0xA5A5A5A5)
    d_src = torch.from_numpy(src.view(np.int32)).cuda()
    d_dst = torch.full((k * n16 + 64, 4), int(sentinel.view(np.int32)), dtype=torch.int32, device="cuda")
    moe.moe_stream(pattern, k, d_dst, d_src, n16)
    got = d_dst.cpu().numpy().view(np.uint32)
    want = src[0::2] ^ src[1::2]
    for j in range(k):
        assert np.array_equal(got[j * n16:(j + 1) * n16], want), j
    assert (got[k * n16:] == sentinel).all()      # nothing stored past the k arrays


@pytest.mark.parametrize("k", [1, 2, 4, 5, 8])
@pytest.mark.parametrize("n16", [1, 4097, 1_000_003])
def test_reduce(k, n16):
    log(f"moe_stream reduce k={k} n16={n16}")
    src = _units(k * n16, 7 * n16 + k)
    sentinel = np.uint32(0x5A5A5A5A)
    d_src = torch.from_numpy(src.view(np.int32)).cuda()
    d_dst = torch.full((n16 + 64, 4), int(sentinel.view(np.int32)), dtype=torch.int32, device="cuda")
    moe.moe_stream(moe.STREAM_REDUCE, k, d_dst, d_src, n16)
    got = d_dst.cpu().numpy().view(np.uint32)
    want = np.bitwise_xor.reduce(src.reshape(k, n16, 4), axis=0)
    assert np.array_equal(got[:n16], want)
    assert (got[n16:] == sentinel).all()


def test_zero_units_store_nothing():
    d = torch.full((8, 4), 7, dtype=torch.int32, device="cuda")
    moe.moe_stream(moe.STREAM_REDUCE, 8, d, d, 0)
    moe.moe_stream(moe.STREAM_FANOUT, 8, d, d, 0)
    moe.moe_stream(moe.STREAM_FANOUT_ONESHOT, 8, d, d, 0)
    torch.cuda.synchronize()
    assert (d.cpu() == 7).all()

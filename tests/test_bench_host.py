"""bench.py's host-side arithmetic, without a GPU: the per-phase byte counts
behind every GB/s figure (each phase's inputs read once and outputs written
once, counted here from the arrays the calls take), the (token, destination
rank) group count of the send-side partial combine (brute force), and the
one-GPU guard of --gpus, the latency fit and the --shape check."""
import subprocess
import sys

import numpy as np
import pytest

import bench


@pytest.mark.parametrize("N,T,H,E,k,Tc", [(16, 4096, 7168, 256, 8, None), (64, 128, 7168, 384, 8, 4096),
                                          (16, 128, 2048, 128, 8, None), (4, 7, 256, 8, 3, 5)])
def test_phase_bytes_are_the_arrays_each_call_touches(N, T, H, E, k, Tc):
    Tcc = T if Tc is None else Tc
    P, Pc = N * T * k, N * Tcc * k
    tokens, fp8_row, scale_row, bf16_row = N * T * H * 2, H, 4 * (H // 128), 2 * H
    ids, pos, w = 4 * N * T * k, 4 * N * T * k, 4 * N * Tcc * k
    counts = 4 * N * E
    G = Pc - N * Tcc   # any group count in [N*Tc, Pc]
    nb = bench.algorithmic_bytes(N, T, H, E, k, Tc, G)
    # dispatch send: tokens and ids in; every slot's fp8 row + scales, send_pos and the count table out
    assert nb["dispatch_send"] == tokens + ids + P * (fp8_row + scale_row) + pos + counts
    # direct dispatch: the same plus one row_src entry per row
    assert nb["dispatch_direct"] == nb["dispatch_send"] + 4 * P
    # dispatch recv: every received row read once and written once
    assert nb["dispatch_recv"] == 2 * P * (fp8_row + scale_row)
    # combine send: every expert output row read once, written once
    assert nb["combine_send"] == 2 * Pc * bf16_row
    # combine recv: k rows, k weights and k positions per token in, one bf16 row out
    out = N * Tcc * H * 2
    assert nb["combine_recv"] == Pc * bf16_row + out + w + 4 * N * Tcc * k
    # pull: the same rows read in place, plus the ids that locate them
    assert nb["combine_pull"] == nb["combine_recv"] + 4 * N * Tcc * k
    # partial: send reads every row and writes one row per group; recv reads the groups
    assert nb["combine_send_partial"] == Pc * bf16_row + G * bf16_row + 3 * 4 * N * Tcc * k
    assert nb["combine_recv_partial"] == G * bf16_row + out + 2 * 4 * N * Tcc * k


def test_combine_heavy_phase_bytes():
    nb = bench.algorithmic_bytes(16, 4096, 7168, 256, 8)
    assert [round(nb[p] / 1e9, 3) for p in bench.PHASES] == [4.819, 7.751, 15.032, 8.46]


def test_group_count_matches_brute_force():
    rng = np.random.default_rng(5)
    for N, T, E, k in [(4, 9, 16, 3), (8, 5, 64, 8), (2, 11, 4, 4), (1, 3, 8, 2)]:
        L = E // N
        idx = np.stack([np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]) for _ in range(N)])
        want = sum(len({int(e) // L for e in idx[s, t]}) for s in range(N) for t in range(T))
        assert bench.combine_groups(idx.astype(np.int32), L) == want
        assert N * T <= want <= N * T * k


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True, text=True,
                       cwd=bench.ROOT, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


@pytest.mark.parametrize("N,T,H,E,k,Tc", [(16, 4096, 7168, 256, 8, None), (64, 128, 7168, 384, 8, 4096),
                                          (4, 7, 256, 8, 3, 5)])
def test_read_and_written_bytes_add_up_to_the_phase_bytes(N, T, H, E, k, Tc):
    nb = bench.algorithmic_bytes(N, T, H, E, k, Tc)
    rw = bench.phase_read_write(N, T, H, E, k, Tc)
    for p in bench.PHASES:
        assert sum(rw[p]) == nb[p], p
    Tcc = T if Tc is None else Tc
    assert rw["dispatch_recv"][0] == rw["dispatch_recv"][1]          # a permutation: read once, written once
    assert rw["combine_send"][0] == rw["combine_send"][1]
    assert rw["combine_recv"][1] == N * Tcc * H * 2                  # one bf16 row per token out
    assert rw["dispatch_send"][1] > (k / 2) * rw["dispatch_send"][0] * 0.97   # the pack writes about k/2 times what it reads


def test_latency_model_recovers_alpha_and_beta():
    """Points on an exact line t = alpha + bytes / beta give back alpha and
    beta; a phase timed on fewer than three workloads gets no fit."""
    alpha, beta = 12.5, 6300.0   # us, GB/s
    sizes = [0.04e9, 0.3e9, 4.8e9, 15.0e9, 30.1e9]
    pts = {"combine_send": [(b, alpha + b / 1e9 / beta * 1e6) for b in sizes],
           "dispatch_send": [(1e9, 200.0), (2e9, 360.0)]}
    fit = bench.latency_model(pts)
    assert set(fit) == {"combine_send"}
    f = fit["combine_send"]
    assert abs(f["alpha_us"] - alpha) < 0.01 and abs(f["beta_GB/s"] - beta) < 0.1
    assert f["workloads"] == len(sizes) and f["max_rel_residual"] < 1e-9


def test_latency_model_weights_relative_error():
    """A fixed cost that only the small points show is kept: the fit on
    relative residuals does not let the large points swamp alpha."""
    pts = {"p": [(0.05e9, 20.0), (0.1e9, 28.0), (5e9, 808.0), (10e9, 1600.0)]}
    f = bench.latency_model(pts)["p"]
    assert 10.0 < f["alpha_us"] < 15.0
    assert 6000.0 < f["beta_GB/s"] < 6400.0


def test_malformed_shape_is_rejected_before_any_gpu_work():
    """--shape takes five integers; anything else ends the run with a
    message before a device is touched."""
    r = subprocess.run([sys.executable, "bench.py", "--shape", "16,128,7168", "--no-cpu-baseline"],
                       capture_output=True, text=True, cwd=bench.ROOT, timeout=300)
    assert r.returncode != 0
    assert "N,T,H,E,k" in (r.stdout + r.stderr)

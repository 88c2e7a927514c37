"""Worker processes for oracle checks whose per-token arithmetic runs on
small arrays (the partial combine's per-token group sums): there NumPy's
calls are short and threads serialise on the interpreter lock, so the work
goes to fresh ("spawn") processes that import only NumPy and the oracle,
never the GPU.  Inputs and results travel through the pool's pipes."""
from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np

from oracle import moe_oracle as O


def _init():
    os.environ["OMP_NUM_THREADS"] = "1"


def partial_tokens(args):
    """The oracle's partial_token for a run of tokens: rows uint16 [n, k, H]
    (slot order), w float32 [n, k], dest [n, k], part bool [n, k].  Returns,
    per token, ([(leader slot, group row)], out)."""
    rows, w, dest, part = args
    return [O.partial_token(rows[t], w[t], dest[t], part[t]) for t in range(rows.shape[0])]


def pool(procs: int):
    return mp.get_context("spawn").Pool(procs, initializer=_init)


def processes() -> int:
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, cores))

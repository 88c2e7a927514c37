"""Seeded synthetic workloads for MoE expert-parallel dispatch / combine.

This module only *generates inputs*: routing choices, router weights, token
rows and expert-output rows.  It holds none of the arithmetic that dispatch or
combine perform (no counting, offsets, quantisation or weighted sums), so the
oracle and the HIP path can both consume it without sharing method code.

Shapes follow the evaluation setup of "Enabling trillion-parameter models on
AWS EFA" (Perplexity, 2025), section "Evaluation: dispatch/combine latency":
hidden size 7168, DeepSeek-V3 / Kimi-K2 expert counts, dispatch batch 128 and
combine batch 4096 tokens per rank.  Real router activations and expert
weights are not available; the recipe below stands in for them.

Recipe (per config, one 64-bit seed; every tensor kind and rank gets its own
child stream, so a rank's data does not depend on how many ranks exist):

* tokens ``x[s]``: float32 N(0,1) rounded to bfloat16 (round to nearest even);
* router logits ``[T, E]``: float32 N(0,1), plus for the skewed config a
  per-expert bias ``-ln(rank_of_e + 1)`` where ``rank_of_e`` is the 0-based
  position of ``e`` in a seeded random permutation (Zipf-like load);
* ``topk_idx[s, t, :]``: the k largest logits in descending order, ties to the
  lower expert index; the forced-worst-case variant keeps only rank 0's experts;
* ``topk_w``: softmax over the k chosen logits in float64, rounded to float32;
* expert outputs ``y``: float32 N(0,1) rounded to bfloat16, one row per
  (token, slot), generated directly in expert-major row order.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

# Child-stream tags (tensor kinds).
_K_LOGITS, _K_TOKENS, _K_Y, _K_PERM = 1, 2, 3, 4


@dataclass(frozen=True)
class Config:
    name: str
    N: int              # logical EP ranks
    T: int              # dispatch tokens per rank
    H: int              # hidden size
    E: int              # experts
    k: int              # experts per token
    T_comb: int = 0     # combine tokens per rank (0 = same as T)
    skew: bool = False  # Zipf-like expert bias
    forced_rank0: bool = False  # every token's experts on rank 0
    seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def L(self) -> int:
        return self.E // self.N

    @property
    def Tc(self) -> int:
        return self.T_comb or self.T

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


CONFIGS: dict[str, Config] = {
    "tiny": Config("tiny", N=16, T=128, H=2048, E=128, k=8, seed=0x7A11_0001,
                   note="T=128, H=2048, E=128, k=8, N=16 (8 experts/rank)"),
    "dsv3_decode": Config("dsv3_decode", N=32, T=128, H=7168, E=256, k=8, seed=0x7A11_0002,
                          note="DeepSeek-V3-shaped decode: T=128, H=7168, E=256, k=8, N=32"),
    "combine_heavy": Config("combine_heavy", N=16, T=4096, H=7168, E=256, k=8, seed=0x7A11_0003,
                            note="T=4096, H=7168, E=256, k=8, N=16 (16 experts/rank)"),
    "kimi_skewed": Config("kimi_skewed", N=64, T=128, T_comb=4096, H=7168, E=384, k=8, skew=True,
                          seed=0x7A11_0004,
                          note="Kimi-K2-shaped, Zipf-like skew: E=384, k=8, N=64; dispatch T=128, combine T=4096"),
    "prefill": Config("prefill", N=8, T=16384, H=7168, E=256, k=8, seed=0x7A11_0005,
                      note="prefill chunk: T=16384, H=7168, E=256, k=8, N=8 (32 experts/rank)"),
}
CONFIGS["prefill_forced"] = CONFIGS["prefill"].with_(name="prefill_forced", forced_rank0=True,
                                                      note="prefill, every token's 8 experts on rank 0")


def _rng(seed: int, kind: int, rank: int, chunk: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed & (2**63 - 1), kind, rank, chunk]))


def _torch_seed(seed: int, kind: int, rank: int, chunk: int = 0) -> int:
    ss = np.random.SeedSequence([seed & (2**63 - 1), kind, rank, chunk])
    return int(ss.generate_state(1, np.uint64)[0] >> np.uint64(1))


def topk_desc(logits: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest entries of each row, largest first; equal
    values keep ascending index order (the first k of a stable sort of
    -logits)."""
    R, E = logits.shape
    if k >= E:
        return np.argsort(-logits, axis=1, kind="stable")[:, :k]
    part = np.argpartition(-logits, k - 1, axis=1)[:, :k]
    kth = np.min(np.take_along_axis(logits, part, axis=1), axis=1)
    tied = (logits >= kth[:, None]).sum(axis=1) > k        # rows with a tie at the cut
    part = np.sort(part, axis=1)                            # ascending index ...
    vals = np.take_along_axis(logits, part, axis=1)
    order = np.argsort(-vals, axis=1, kind="stable")        # ... then descending value
    out = np.take_along_axis(part, order, axis=1)
    if tied.any():
        rows = np.flatnonzero(tied)
        out[rows] = np.argsort(-logits[rows], axis=1, kind="stable")[:, :k]
    return out


def expert_bias(cfg: Config) -> np.ndarray:
    """Per-expert logit bias of the skewed config (zeros otherwise)."""
    if not cfg.skew:
        return np.zeros(cfg.E, np.float32)
    perm = _rng(cfg.seed, _K_PERM, 0).permutation(cfg.E)
    rank_of = np.empty(cfg.E, np.int64)
    rank_of[perm] = np.arange(cfg.E)
    return (-np.log(rank_of + 1.0)).astype(np.float32)


def routing(cfg: Config, T: int | None = None):
    """Returns (topk_idx int32 [N, T, k], topk_w float32 [N, T, k])."""
    T = cfg.T if T is None else T
    bias = expert_bias(cfg)
    idx = np.empty((cfg.N, T, cfg.k), np.int32)
    w = np.empty((cfg.N, T, cfg.k), np.float32)
    for s in range(cfg.N):
        logits = _rng(cfg.seed, _K_LOGITS, s, T).standard_normal((T, cfg.E), dtype=np.float32) + bias
        if cfg.forced_rank0:
            logits[:, cfg.L:] = -np.inf
        top = topk_desc(logits, cfg.k)
        lv = np.take_along_axis(logits, top, axis=1).astype(np.float64)
        ex = np.exp(lv - lv[:, :1])
        w[s] = (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)
        idx[s] = top
    return idx, w


def _randn_bf16_into(out, seed: int, kind: int, rank: int, chunk_rows: int):
    """Fill a 2-D bfloat16 torch tensor with N(0,1) values, chunk by chunk
    (each chunk its own seeded generator on the tensor's device)."""
    import torch
    rows = out.shape[0]
    for c0 in range(0, rows, chunk_rows):
        c1 = min(rows, c0 + chunk_rows)
        g = torch.Generator(device=out.device)
        g.manual_seed(_torch_seed(seed, kind, rank, c0 // chunk_rows))
        out[c0:c1] = torch.randn((c1 - c0, out.shape[1]), generator=g, device=out.device,
                                 dtype=torch.float32).to(torch.bfloat16)
    return out


def tokens(cfg: Config, device="cpu", T: int | None = None):
    """bfloat16 torch tensor [N, T, H] of N(0,1) token rows."""
    import torch
    T = cfg.T if T is None else T
    x = torch.empty((cfg.N, T, cfg.H), dtype=torch.bfloat16, device=device)
    for s in range(cfg.N):
        _randn_bf16_into(x[s], cfg.seed, _K_TOKENS, s, max(1, (1 << 26) // cfg.H))
    return x


def expert_outputs(cfg: Config, rows: int, device="cpu"):
    """bfloat16 torch tensor [rows, H] of N(0,1) expert-output rows (the
    grouped GEMM's output, already in expert-major row order)."""
    import torch
    y = torch.empty((rows, cfg.H), dtype=torch.bfloat16, device=device)
    return _randn_bf16_into(y, cfg.seed, _K_Y, 0, max(1, (1 << 26) // cfg.H))

"""Input generator checks (no GPU) and the oracle / product independence rule."""
import ast
import os

import numpy as np
import pytest

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_topk_matches_stable_argsort_with_ties():
    rng = np.random.default_rng(0)
    lg = rng.integers(-3, 4, size=(500, 16)).astype(np.float32)      # many ties
    for k in (1, 3, 8, 16):
        ref = np.argsort(-lg, axis=1, kind="stable")[:, :k]
        assert (W.topk_desc(lg, k) == ref).all()
    lg = rng.standard_normal((2000, 256)).astype(np.float32)
    assert (W.topk_desc(lg, 8) == np.argsort(-lg, axis=1, kind="stable")[:, :8]).all()


@pytest.mark.parametrize("name", ["tiny", "kimi_skewed", "prefill_forced"])
def test_routing_recipe(name):
    cfg = W.CONFIGS[name]
    T = 32
    idx, w = W.routing(cfg, T)
    assert idx.shape == (cfg.N, T, cfg.k) and idx.dtype == np.int32
    assert ((idx >= 0) & (idx < cfg.E)).all()
    assert all(len(set(r)) == cfg.k for r in idx.reshape(-1, cfg.k).tolist())
    assert np.allclose(w.sum(axis=2), 1.0, atol=1e-6) and (np.diff(w, axis=2) <= 0).all()
    if cfg.forced_rank0:
        assert (idx < cfg.L).all()
    idx2, w2 = W.routing(cfg, T)
    assert (idx == idx2).all() and (w == w2).all()               # seeded


def test_skew_bias_shape():
    cfg = W.CONFIGS["kimi_skewed"]
    b = W.expert_bias(cfg)
    assert b.max() == 0.0 and np.isclose(np.sort(-b)[1], np.log(2.0))
    idx, _ = W.routing(cfg, 128)
    load = np.bincount(idx.reshape(-1), minlength=cfg.E)
    assert np.sort(load)[::-1][:10].sum() > 0.4 * load.sum()      # heavily skewed
    assert (load == 0).any()


def test_tokens_are_seeded_bf16():
    import torch
    cfg = W.CONFIGS["tiny"].with_(N=2, H=256)
    a = W.tokens(cfg, "cpu", T=4)
    b = W.tokens(cfg, "cpu", T=4)
    assert a.dtype == torch.bfloat16 and a.shape == (2, 4, 256) and torch.equal(a, b)
    assert 0.8 < a.float().std().item() < 1.2


def _imports(path):
    tree = ast.parse(open(path).read())
    out = set()
    for n in ast.walk(tree):
        if isinstance(n, ast.Import):
            out |= {a.name.split(".")[0] for a in n.names}
        elif isinstance(n, ast.ImportFrom) and n.module:
            out.add(n.module.split(".")[0])
    return out


def test_oracle_and_product_do_not_import_each_other():
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith(".py"):
            assert "combine_lds_atomic_amd" not in _imports(os.path.join(ROOT, "oracle", f))
    pkg = os.path.join(ROOT, "combine_lds_atomic_amd")
    for dp, _, fs in os.walk(pkg):
        for f in fs:
            if f.endswith(".py"):
                im = _imports(os.path.join(dp, f))
                assert "oracle" not in im and "workloads" not in im, f

"""The seeded input recipe: shapes, dtypes, distributions, determinism (CPU)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W


def test_configs_match_the_benchmark_layers():
    shapes = [(c.T, c.d, c.E, c.h, c.top_k) for c in W.CONFIGS]
    assert shapes == [(64, 256, 4, 512, 1), (16, 5120, 16, 8192, 1), (8192, 5120, 16, 8192, 1),
                      (4096, 5120, 128, 8192, 1), (16384, 5120, 128, 8192, 8)]
    assert [c.bias for c in W.CONFIGS] == ["none", "none", "normal", "zipf", "none"]
    assert W.CONFIGS[4].router == "uniform"
    assert W.CONFIGS[4].pairs == 131072


def test_draws_are_deterministic_and_distinct():
    cfg = W.config(0)
    assert torch.equal(W.gen_x(cfg), W.gen_x(cfg))
    a = W.gen_expert_weight(cfg, "w1", 0)
    assert torch.equal(a, W.gen_expert_weight(cfg, "w1", 0))
    assert not torch.equal(a, W.gen_expert_weight(cfg, "w1", 1))
    assert not torch.equal(a, W.gen_expert_weight(cfg, "w3", 0))
    assert W.stream_seed(0, W.W1, 3) != W.stream_seed(1, W.W1, 3)


def test_distributions():
    cfg = W.config(0).with_(T=4096, d=512)
    x = W.gen_x(cfg)
    assert x.dtype == torch.bfloat16 and x.shape == (4096, 512)
    assert abs(x.float().std().item() - 1.0) < 0.01
    wr, b = W.gen_router(cfg)
    assert wr.dtype == torch.float32 and b is None
    assert abs(wr.std().item() - 0.02) < 0.001
    w2 = W.gen_expert_weight(cfg, "w2", 1)
    assert w2.shape == (cfg.d, cfg.h) and abs(w2.std().item() - 0.02) < 0.0005
    s1, s3, s2 = W.gen_shared(cfg)
    assert s1.dtype == torch.bfloat16 and s2.shape == (cfg.d, cfg.h)
    wu, _ = W.gen_router(W.config(4).with_(d=512))
    assert wu.min() >= -0.02 and wu.max() <= 0.02 and abs(wu.std().item() - 0.04 / 12 ** 0.5) < 5e-4
    _, bn = W.gen_router(W.config(2))
    assert bn.shape == (16,)
    _, bz = W.gen_router(W.config(3))
    np.testing.assert_allclose(bz.numpy(), -W.ZIPF_C * np.log(np.arange(128) + 1.0), rtol=1e-6)


def _loads(i):
    cfg = W.config(i)
    wr, b = W.gen_router(cfg)
    logits = oracle.router_logits(W.gen_x(cfg), wr, b)
    ids, margin = oracle.select_topk(logits, cfg.top_k)
    return np.bincount(ids.ravel(), minlength=cfg.E), margin


@pytest.mark.slow
def test_realized_expert_loads():
    # Maverick-shaped prefill: Zipf(1.1)-like head, ~T / H(128, 1.1) tokens on expert 0
    cnt, _ = _loads(3)
    target = 4096 * W.zipf_head_share(128)
    assert abs(cnt[0] - target) < 0.03 * target
    assert cnt[0] > cnt[1] > cnt[2] > cnt[3] and (cnt > 0).sum() > 100
    # Scout-shaped prefill: uneven loads from the N(0, 0.5) bias
    cnt, _ = _loads(2)
    assert cnt.sum() == 8192 and cnt.max() > 4 * cnt.min() > 0
    # wide routing: 131072 pairs, every expert busy
    cnt, margin = _loads(4)
    assert cnt.sum() == 131072 and cnt.min() > 800
    # Scout-shaped decode: 16 tokens over most of the 16 experts
    cnt, _ = _loads(1)
    assert cnt.sum() == 16 and (cnt > 0).sum() >= 8

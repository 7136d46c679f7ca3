"""The layer with bf16 routed experts (the pure-bf16 baseline path) on the GPU
against the oracle's bf16 expert path, same bar as the int4 layer: every row
within 2e-2 relative error (infinity norm of the oracle's fp64 row), ids equal
wherever the top-k margin exceeds 1e-4."""
import numpy as np
import pytest
import torch

import moe_ffn_int4_amd as moe
import workloads as W
from gpu_util import (TOL, build_layer, check_ids, covering_rows, oracle_forward_rows,
                      resolved_path, row_errors, sample_rows, say)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

SMALL = {
    "tiny": W.config(0),
    "several tiles, ragged tail": W.config(0).with_(T=300, d=384, E=5, h=640, top_k=2),
    "single token": W.config(0).with_(T=1, E=5, top_k=2),
    "empty experts": W.config(0).with_(T=200, E=8, top_k=1, bias="zipf", bias_param=3.0),
    "tile edge 257": W.config(0).with_(T=257, E=2, d=384, top_k=1),
    "mixed expert sizes": W.config(0).with_(T=300, E=12, top_k=2, bias="zipf", bias_param=0.6),
}


def _run(layer, path="auto"):
    cfg = layer.cfg
    ids = torch.empty(cfg.T, cfg.top_k, dtype=torch.int32, device=DEV)
    y = moe.forward(layer.x_d, layer.wr_d, layer.b_d, layer.experts_d, layer.shared_d,
                    cfg.top_k, path=path, topk_ids=ids)
    torch.cuda.synchronize()
    return y.cpu(), ids.cpu().numpy()


def _check(layer, y, ids, rows):
    ref, margin = oracle_forward_rows(layer, rows, gpu_ids=ids)
    ties = check_ids(ids[rows], ref.ids, margin)
    err = row_errors(y[torch.as_tensor(rows)], ref.y)
    say(f"  rows={len(rows)} ties={ties} max row rel err={err.max():.3e}")
    assert err.max() <= TOL


@pytest.mark.parametrize("path", ["prefill", "decode", "hybrid", "prefill_wide"])
@pytest.mark.parametrize("name", list(SMALL))
def test_small_layers_every_token(name, path):
    cfg = SMALL[name]
    say(f"forward bf16 experts[{path}]: {name} T={cfg.T} d={cfg.d} E={cfg.E} h={cfg.h} k={cfg.top_k}")
    layer = build_layer(cfg, routed="bf16")
    y, ids = _run(layer, path)
    _check(layer, y, ids, np.arange(cfg.T))


@pytest.mark.parametrize("i", [1, 2, 3, 4])
def test_benchmark_layers_covered(i):
    cfg = W.config(i)
    say(f"forward bf16 experts: config {i} ({cfg.name})")
    layer = build_layer(cfg, routed="bf16")
    y, ids = _run(layer)
    assert torch.isfinite(y.float()).all()
    cov = covering_rows(ids, cfg.E, resolved_path(cfg.T, cfg.E, cfg.top_k),
                        extra=sample_rows(cfg.T, 4, seed=i))
    say("  " + cov.report)
    _check(layer, y, ids, cov.rows)


def test_rejects_mismatched_experts():
    cfg = W.config(0)
    layer = build_layer(cfg, routed="bf16")
    bad = moe.Bf16Experts.empty(cfg.E + 1, cfg.d, cfg.h, DEV)
    with pytest.raises(ValueError):
        moe.forward(layer.x_d, layer.wr_d, layer.b_d, bad, layer.shared_d, cfg.top_k)

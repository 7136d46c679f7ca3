"""The layer with fp8 routed experts (the fp8_mixed path: row-wise fp8
activations and weights, bf16 products) on the GPU against the oracle's fp8
expert path (the C per-token loop, pinned to the numpy form), same bar as the
int4 layer: every row within 2e-2 relative error (infinity norm of the
oracle's fp64 row), ids equal wherever the top-k margin exceeds 1e-4. The
oracle quantizes the same fp32 weight draws itself."""
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
    "k=E": W.config(0).with_(T=70, E=3, top_k=3),
    "empty experts": W.config(0).with_(T=200, E=8, top_k=1, bias="zipf", bias_param=3.0),
    "tile edge 128": W.config(0).with_(T=128, E=2, top_k=1),
    "tile edge 257": W.config(0).with_(T=257, E=2, d=384, top_k=1),
    "k=16 of 40": W.config(0).with_(T=40, d=512, E=40, h=256, top_k=16),
    "mixed expert sizes": W.config(0).with_(T=300, E=12, top_k=2, bias="zipf", bias_param=0.6),
}


def _run(layer, path="auto", workspace=None):
    cfg = layer.cfg
    ids = torch.empty(cfg.T, cfg.top_k, dtype=torch.int32, device=DEV)
    y = moe.forward(layer.x_d, layer.wr_d, layer.b_d, layer.experts_d, layer.shared_d,
                    cfg.top_k, path=path, topk_ids=ids, workspace=workspace)
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
    say(f"forward fp8 experts[{path}]: {name} T={cfg.T} d={cfg.d} E={cfg.E} h={cfg.h} k={cfg.top_k}")
    layer = build_layer(cfg, routed="fp8")
    y, ids = _run(layer, path)
    _check(layer, y, ids, np.arange(cfg.T))


@pytest.mark.parametrize("path", ["prefill", "decode", "prefill_wide"])
@pytest.mark.parametrize("ub", [0.5, 0.0])
def test_activation_bound(ub, path):
    """ub 0.5 binds on x rows (their elements past 0.5 saturate at +-448) and on
    every H row; ub 0 means no bound."""
    cfg = W.config(0).with_(T=100, E=5, top_k=2)
    say(f"forward fp8 experts[{path}]: ub={ub}")
    layer = build_layer(cfg, routed="fp8", act_ub=ub)
    y, ids = _run(layer, path)
    _check(layer, y, ids, np.arange(cfg.T))


def test_paths_agree_and_workspace_reuse():
    cfg = W.config(0).with_(T=300, E=6, top_k=2)
    layer = build_layer(cfg, routed="fp8")
    ws = moe.alloc_workspace(cfg.T, cfg.d, cfg.E, cfg.h, cfg.top_k, DEV, fp8=True)
    ws.fill_(0xFF)
    y1, i1 = _run(layer, "prefill", ws)
    y1b, _ = _run(layer, "prefill", ws)
    assert torch.equal(y1, y1b)
    for other in ("decode", "hybrid", "prefill_wide"):
        y2, i2 = _run(layer, other, ws)
        np.testing.assert_array_equal(i1, i2)
        assert row_errors(y1, y2.float().numpy().astype(np.float64)).max() <= 1e-2, other


@pytest.mark.parametrize("i", [1, 2, 3, 4])
def test_benchmark_layers_covered(i):
    cfg = W.config(i)
    say(f"forward fp8 experts: config {i} ({cfg.name})")
    layer = build_layer(cfg, routed="fp8")
    y, ids = _run(layer)
    assert torch.isfinite(y.float()).all()
    cov = covering_rows(ids, cfg.E, resolved_path(cfg.T, cfg.E, cfg.top_k),
                        extra=sample_rows(cfg.T, 4, seed=i))
    say("  " + cov.report)
    _check(layer, y, ids, cov.rows)


def test_rejects_small_workspace_and_bad_bound():
    cfg = W.config(0)
    layer = build_layer(cfg, routed="fp8")
    small = moe.alloc_workspace(cfg.T, cfg.d, cfg.E, cfg.h, cfg.top_k, DEV)  # int4 size
    with pytest.raises(moe.MoEError, match="workspace"):
        _run(layer, workspace=small)
    bad = moe.Fp8Experts(*(getattr(layer.experts_d, n) for n in
                           ("w1q", "w3q", "w2q", "w1s", "w3s", "w2s")), float("nan"))
    with pytest.raises(moe.MoEError, match="act_ub"):
        moe.forward(layer.x_d, layer.wr_d, layer.b_d, bad, layer.shared_d, cfg.top_k)

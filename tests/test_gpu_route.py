"""K2 router/top-k and K3 dispatch on the GPU vs the oracle.

Logits within fp32 accumulation error of the oracle's; expert ids equal (as
sets) wherever the oracle's top-k margin exceeds 1e-4; gates the sigmoid of the
chosen logits; dispatch bit-exact against its definition (counting sort of the
GPU's own ids, pairs ascending inside each expert).
"""
import numpy as np
import pytest
import torch

import moe_ffn_int4_amd as moe
import workloads as W
from gpu_util import check_ids, say
from oracle import router_logits, select_topk, sigmoid

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _route(cfg):
    x = W.gen_x(cfg)
    wr, b = W.gen_router(cfg)
    r = moe.route(x.to(DEV), wr.to(DEV), None if b is None else b.to(DEV), cfg.top_k)
    torch.cuda.synchronize()
    r = {k: v.cpu().numpy() for k, v in r.items()}
    logits = router_logits(x, wr.numpy(), None if b is None else b.numpy())
    return r, logits


def _check_dispatch(r, E, k):
    ids = r["ids"].reshape(-1)
    P = ids.size
    counts = np.bincount(ids, minlength=E)
    np.testing.assert_array_equal(r["counts"], counts)
    np.testing.assert_array_equal(r["offsets"], np.concatenate([[0], np.cumsum(counts)]))
    # counting sort, stable: pairs grouped by expert, ascending inside each group
    want = np.argsort(ids, kind="stable").astype(np.int32)
    np.testing.assert_array_equal(r["perm"], want)
    np.testing.assert_array_equal(r["inv"][r["perm"]], np.arange(P))
    assert P == r["offsets"][-1]


CASES = {
    "tiny": W.config(0),
    "decode": W.config(1),
    "scout_prefill": W.config(2),
    "maverick_prefill": W.config(3),
    "wide_routing": W.config(4),
    "k=E": W.config(0).with_(T=100, E=6, top_k=6),
    "ragged": W.config(0).with_(T=333, E=7, top_k=3, bias="normal", bias_param=2.0),
    "single token": W.config(0).with_(T=1, E=5, top_k=2),
    "256 experts": W.config(0).with_(T=500, d=512, E=256, top_k=16),
}


@pytest.mark.parametrize("name", list(CASES))
def test_routing_matches_oracle(name):
    cfg = CASES[name]
    say(f"route: {name} T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.top_k}")
    r, logits = _route(cfg)
    scale = np.abs(logits).max() + 1.0
    np.testing.assert_allclose(r["logits"], logits, rtol=0, atol=2e-5 * scale)
    ref_ids, margin = select_topk(logits, cfg.top_k)
    ties = check_ids(r["ids"], ref_ids, margin)
    say(f"  tokens within the 1e-4 margin: {ties}")
    # the GPU's ids are a valid top-k of its own logits, by descending logit
    chosen = np.take_along_axis(r["logits"], r["ids"].astype(np.int64), axis=1)
    assert np.all(np.diff(chosen, axis=1) <= 0)
    kth = chosen[:, -1]
    mask = np.ones_like(r["logits"], dtype=bool)
    np.put_along_axis(mask, r["ids"].astype(np.int64), False, axis=1)
    others = np.where(mask, r["logits"], -np.inf).max(axis=1)
    assert np.all(kth >= others)
    assert all(len(set(row)) == cfg.top_k for row in r["ids"].tolist())
    np.testing.assert_allclose(r["gates"], sigmoid(chosen), rtol=2e-6, atol=1e-7)
    _check_dispatch(r, cfg.E, cfg.top_k)


def test_routing_is_deterministic():
    cfg = W.config(4).with_(T=4096)
    a, _ = _route(cfg)
    b, _ = _route(cfg)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])

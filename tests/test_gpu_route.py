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


def test_prefill_router_keeps_fp32_weights():
    """Batches of 256+ tokens compute the logits on bf16 matrix cores from the
    router weights split into three bf16 parts. With x = 1, d = 128 and weights
    such as 2^-8 + 2^-16 + 2^-24 (one bit in each part), every partial sum is a
    short binary fraction, so fp32 accumulation in any order gives the exact
    logit; dropping any part of a weight moves a logit by at least 2^-17."""
    T, d, E = 256, 128, 4
    x = torch.ones(T, d, dtype=torch.bfloat16)
    w = np.empty((E, d), dtype=np.float32)
    w[0] = 2.0 ** -8 + 2.0 ** -16 + 2.0 ** -24        # hi, mid and lo all non-zero
    w[1] = -(2.0 ** -8 + 2.0 ** -16)                  # hi and mid, negative
    w[2] = 2.0 ** -9 + 2.0 ** -20                     # mid far below hi
    w[3, ::2] = 2.0 ** -8 + 2.0 ** -24                # cancels to zero in pairs
    w[3, 1::2] = -(2.0 ** -8 + 2.0 ** -24)
    assert not np.all(w == torch.from_numpy(w).to(torch.bfloat16).float().numpy())
    r = moe.route(x.to(DEV), torch.from_numpy(w).to(DEV), None, 1)
    torch.cuda.synchronize()
    got = r["logits"].cpu().numpy().astype(np.float64)
    want = w.astype(np.float64).sum(axis=1)
    np.testing.assert_array_equal(got, np.broadcast_to(want, got.shape))

"""The allocation-free forward (moe_forward_noalloc) against moe_forward_path.

moe_forward_noalloc runs the same kernels on the library's static device
scratch instead of a caller's workspace. Called through the C ABI, its outputs
(y, expert ids, gates) must equal those of moe_forward_path with a workspace of
its own, bit for bit, on two calls in a row, the second with fewer tokens than
the first (the scratch then holds the first call's data). Layers past the
scratch's size are refused with MOE_ERR_WORKSPACE.
"""
import numpy as np
import pytest
import torch

import moe_ffn_int4_amd as moe
import workloads as W
from gpu_util import build_layer, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _compare(layer, T, path):
    cfg = layer.cfg
    x = layer.x_d[:T].contiguous()
    outs = []
    for fn in (moe.forward, moe.forward_noalloc):
        ids = torch.full((T, cfg.top_k), -1, dtype=torch.int32, device=DEV)
        gates = torch.full((T, cfg.top_k), -1.0, dtype=torch.float32, device=DEV)
        y = fn(x, layer.wr_d, layer.b_d, layer.experts_d, layer.shared_d, cfg.top_k, path=path,
               topk_ids=ids, topk_gates=gates)
        outs.append((y, ids, gates))
    torch.cuda.synchronize()
    (ya, ia, ga), (yb, ib, gb) = outs
    assert torch.equal(ia, ib)
    assert torch.equal(ga.view(torch.int32), gb.view(torch.int32))
    assert torch.equal(ya.view(torch.int16), yb.view(torch.int16))
    assert torch.isfinite(yb.float()).all()


# (layer, path, tokens of the first call, tokens of the second)
CASES = {
    "Scout decode": (W.config(1), "auto", 16, 5),
    "hybrid, mixed expert sizes": (W.config(0).with_(T=300, E=12, top_k=2, bias="zipf",
                                                     bias_param=0.6), "hybrid", 300, 90),
    "256-row tiles, ragged": (W.config(0).with_(T=257, d=384, E=2, top_k=1), "prefill_wide", 257, 130),
    "decode, top-2": (W.config(0).with_(T=32, E=5, top_k=2), "decode", 32, 1),
}


@pytest.mark.parametrize("name", list(CASES))
def test_noalloc_equals_forward_path(name):
    cfg, path, t1, t2 = CASES[name]
    say(f"no-alloc forward: {name} T={t1} then T={t2} [{path}]")
    layer = build_layer(cfg)
    _compare(layer, t1, path)
    _compare(layer, t2, path)


def test_noalloc_rejects_layers_past_the_scratch():
    layer = build_layer(W.config(0))
    cfg = layer.cfg
    T = 200000  # about 0.8 GB of workspace at d = 256, h = 512
    assert moe.workspace_bytes(T, cfg.d, cfg.E, cfg.h, 1) > moe.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(T, cfg.d, dtype=torch.bfloat16, device=DEV)
    y = torch.full((T, cfg.d), 7, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    with pytest.raises(moe.MoEError, match="workspace"):
        moe.forward_noalloc(x, layer.wr_d, layer.b_d, layer.experts_d, layer.shared_d, 1, y=y)
    torch.cuda.synchronize()
    assert bool((y.view(torch.int16) == 7).all())  # refused before any launch

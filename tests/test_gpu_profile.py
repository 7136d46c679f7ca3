"""Per-stage timing (moe_profile_*): the stages a path runs report their calls
and a positive duration, the durations fit inside the forward's own time, and
timing leaves the output unchanged bit for bit (with timing on, the kernels
launch through hipExtLaunchKernel with events; with it off, plainly)."""
import pytest
import torch

import moe_ffn_int4_amd as moe
import workloads as W
from gpu_util import build_layer, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# pairs per expert from a few hundred down to one and zero (600 pairs: the
# top-k and dispatch kernels)
MIXED = W.config(0).with_(T=300, E=12, top_k=2, bias="zipf", bias_param=0.6)
# 32 pairs: the one-block routing kernel, which also dispatches
SMALL = W.config(0).with_(T=16, E=12, top_k=2)
LARGE = W.config(0).with_(T=1100, E=8, top_k=1)
ROUTE = {"router", "topk", "dispatch"}
CASES = {
    "decode, one-block routing": (SMALL, "decode",
                                  {"router", "topk", "decode_up", "decode_down", "combine"}),
    "decode": (MIXED, "decode", ROUTE | {"decode_up", "decode_down", "combine"}),
    "prefill": (MIXED, "prefill", ROUTE | {"grouped_up", "grouped_down", "combine"}),
    "hybrid": (MIXED, "hybrid", ROUTE | {"grouped_up", "grouped_down", "decode_up",
                                         "decode_down", "combine"}),
    "prefill_wide": (LARGE, "prefill_wide", ROUTE | {"grouped_up", "grouped_down", "combine"}),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_profile_times_each_stage(case):
    cfg, path, expected = CASES[case]
    layer = build_layer(cfg)
    ws = moe.alloc_workspace(cfg.T, cfg.d, cfg.E, cfg.h, cfg.top_k, layer.dev)

    def fwd():
        return moe.forward(layer.x_d, layer.wr_d, layer.b_d, layer.experts_d, layer.shared_d,
                           cfg.top_k, path=path, workspace=ws)

    y_plain = fwd()
    torch.cuda.synchronize()
    moe.profile_enable(True)
    try:
        moe.profile_read()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        y_timed = fwd()
        end.record()
        torch.cuda.synchronize()
        stages = moe.profile_read()
    finally:
        moe.profile_enable(False)
    total_ms = start.elapsed_time(end)
    ran = {k for k, (ms, n) in stages.items() if n > 0}
    say(f"  {path}: {', '.join(f'{k} {ms * 1e3:.1f} us' for k, (ms, n) in stages.items() if n)}"
        f"; forward {total_ms * 1e3:.1f} us")
    assert ran == expected, f"timed stages {sorted(ran)}"
    for k in ran:
        assert stages[k][0] > 0.0, f"stage {k}: no time"
    # stages run one after another on the caller's stream, except that the
    # hybrid path's streaming stages overlap the GEMMs on the library's stream
    serial = sum(ms for k, (ms, n) in stages.items()
                 if n and not (path == "hybrid" and k.startswith("decode")))
    assert serial <= total_ms * 1.05 + 0.01, f"stage sum {serial} ms > forward {total_ms} ms"
    assert torch.equal(y_plain, y_timed), "timing changed the output"

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

# pairs per expert from a few hundred down to one and zero; T*E and T*k small
# enough for the one-block routing kernel, which also dispatches
MIXED = W.config(0).with_(T=300, E=12, top_k=2, bias="zipf", bias_param=0.6)
# T*E past the one-block routing: separate top-k and dispatch kernels
LARGE = W.config(0).with_(T=1100, E=8, top_k=1)
CASES = {
    "decode": (MIXED, {"router", "topk", "decode_up", "decode_down", "combine"}),
    "prefill": (MIXED, {"router", "topk", "grouped_up", "grouped_down", "combine"}),
    "hybrid": (MIXED, {"router", "topk", "grouped_up", "grouped_down", "decode_up",
                       "decode_down", "combine"}),
    "prefill_wide": (LARGE, {"router", "topk", "dispatch", "grouped_up", "grouped_down",
                             "combine"}),
}


@pytest.mark.parametrize("path", sorted(CASES))
def test_profile_times_each_stage(path):
    cfg, expected = CASES[path]
    assert cfg.T * cfg.E > 8192 or "dispatch" not in expected
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

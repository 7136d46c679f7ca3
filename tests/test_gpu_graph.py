"""The forward captured in a HIP graph (torch.cuda.CUDAGraph) on every path.

A caller that captures moe_forward replays the recorded kernels on new data in
the same buffers. Each replay here follows eager work (new input rows copied
into the captured buffer, the output cleared) and a synchronization, and its
output and expert ids must equal the eager forward's on the same input bit for
bit (the kernels are deterministic: fixed reduction orders, no atomics). The
hybrid path forks the small experts' streaming kernels onto the library's own
stream and joins them back, which the capture must follow through its events.
"""
import pytest
import torch

import moe_ffn_int4_amd as moe
import workloads as W
from gpu_util import build_layer, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# pairs per expert from a few hundred down to one and zero: GEMM tiles and
# streamed experts on the hybrid path, several chunk sizes on the decode path
CFG = W.config(0).with_(T=300, E=12, top_k=2, bias="zipf", bias_param=0.6)


@pytest.mark.parametrize("path", ["decode", "prefill", "prefill_wide", "hybrid"])
def test_graph_replays_equal_eager(path):
    cfg = CFG
    layer = build_layer(cfg)
    ws = moe.alloc_workspace(cfg.T, cfg.d, cfg.E, cfg.h, cfg.top_k, layer.dev)
    x_buf = torch.empty_like(layer.x_d)
    y = torch.empty(cfg.T, cfg.d, dtype=torch.bfloat16, device=DEV)
    ids = torch.empty(cfg.T, cfg.top_k, dtype=torch.int32, device=DEV)

    def fwd():
        moe.forward(x_buf, layer.wr_d, layer.b_d, layer.experts_d, layer.shared_d, cfg.top_k,
                    path=path, y=y, topk_ids=ids, workspace=ws)

    # three inputs: the layer's, its rows reversed, and a second seeded draw
    inputs = [layer.x_d, layer.x_d.flip(0).contiguous(), W.gen_x(cfg.with_(seed=7)).to(DEV)]
    eager = []
    for xi in inputs:
        x_buf.copy_(xi)
        fwd()
        torch.cuda.synchronize()
        eager.append((y.clone(), ids.clone()))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        fwd()  # a forward on the capture stream before capturing it
        side.synchronize()
        with torch.cuda.graph(graph, stream=side):
            fwd()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for rep in range(3):
        for i, (xi, (y_ref, ids_ref)) in enumerate(zip(inputs, eager)):
            x_buf.copy_(xi)
            y.zero_()
            ids.fill_(-1)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            say(f"  {path}: replay {rep} input {i}")
            assert torch.equal(ids, ids_ref), f"replay {rep}, input {i}: expert ids differ"
            assert torch.equal(y, y_ref), f"replay {rep}, input {i}: output differs from eager"

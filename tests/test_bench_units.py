"""The benchmark's algorithmic units, held to closed forms worked out by hand.

`roofline.achieved` divides a launch's algorithmic bytes (decode) or FLOPs
(prefill) by its duration, so these counts decide the reported fraction of
peak. They are checked here against independent arithmetic: the layer's FLOPs
(router 2TdE, routed SwiGLU 6Tkdh, shared SwiGLU 6Tdh) against the values for
the five benchmark layers, and the bytes a decode step must stream (every
touched expert's int4 codes and scales once, the shared expert's bf16 weights,
the router weights, x and y) against per-expert and shared totals.
"""
import numpy as np
import pytest

import bench
import workloads as W

# FLOPs of the five benchmark layers, worked out from T, d, E, h and top_k
FLOPS = {0: 0.1008e9, 1: 8.06e9, 2: 4.125e12, 3: 2.067e12, 4: 37.13e12}


@pytest.mark.parametrize("c", sorted(FLOPS))
def test_layer_flops(c):
    assert W.config(c).flops() == pytest.approx(FLOPS[c], rel=2e-3)


def test_decode_step_bytes_per_expert():
    cfg = W.config(1)  # d = 5120, h = 8192, E = 16, T = 16, top-1
    d, h = cfg.d, cfg.h
    per_expert = 3 * d * h // 2 + 3 * (d * h // 128) * 4  # W1, W3, W2 codes + fp32 scales
    assert per_expert == 66_846_720
    shared = 3 * d * h * 2
    assert shared == 251_658_240
    for touched in (1, 11, 16):
        counts = np.zeros(cfg.E, dtype=np.int64)
        counts[:touched] = 1
        counts[0] += cfg.T * cfg.top_k - touched
        u = bench.stage_units(cfg, counts)
        assert u["touched"] == touched
        assert u["step_bytes"] == touched * per_expert + shared + cfg.E * d * 4 + 2 * cfg.T * d * 2


def test_stage_flops_cover_the_layer():
    # the up and down launches (routed rows plus the shared expert's) and the
    # router add up to the layer's FLOPs; the decode stages count the same work
    for c in (1, 2):
        cfg = W.config(c)
        counts = np.bincount(np.arange(cfg.T * cfg.top_k) % cfg.E, minlength=cfg.E).astype(np.int64)
        u = bench.stage_units(cfg, counts)
        total = u["router"][1] + u["grouped_up"][1] + u["grouped_down"][1]
        assert total == pytest.approx(cfg.flops(), rel=1e-12)
        assert u["decode_up"][1] + u["decode_down"][1] == u["grouped_up"][1] + u["grouped_down"][1]


def test_group_and_format_bytes():
    cfg = W.config(1)
    d, h = cfg.d, cfg.h
    counts = np.zeros(cfg.E, dtype=np.int64)
    counts[0] = cfg.T
    base = cfg.E * d * 4 + 2 * cfg.T * d * 2 + 3 * d * h * 2
    # groups of 32: four times the scales of groups of 128
    u32 = bench.stage_units(cfg, counts, g=32)
    assert u32["step_bytes"] == 3 * d * h // 2 + 3 * (d * h // 32) * 4 + base
    # bf16 routed experts: two bytes per weight
    ub = bench.stage_units(cfg, counts, experts="bf16")
    assert ub["step_bytes"] == 3 * d * h * 2 + base
    # fp8 row-wise: one byte per weight and one fp32 scale per row
    u8 = bench.stage_units(cfg, counts, experts="fp8")
    assert u8["step_bytes"] == 3 * d * h + (2 * h + d) * 4 + base


def test_traffic_record_tracks_its_sources(tmp_path, monkeypatch):
    """A counter record is reported only for its own stage and workload and
    only while every source file it names is byte-identical to the one
    measured; any edit of a source turns the field to null."""
    import hashlib
    import json
    src = tmp_path / "moe_ffn_int4_amd" / "csrc" / "k.hip"
    src.parent.mkdir(parents=True)
    src.write_text("kernel as profiled\n")
    (tmp_path / "profiles").mkdir()
    rec = {"stage": "grouped_up", "workload": "scout_prefill", "hbm_bytes_per_launch": 123.0,
           "sources_sha256": {"moe_ffn_int4_amd/csrc/k.hip":
                              hashlib.sha256(src.read_bytes()).hexdigest()}}
    (tmp_path / "profiles" / "traffic.json").write_text(
        json.dumps({"grouped_up@scout_prefill": rec}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("grouped_up", "scout_prefill") == 123.0
    assert bench.measured_traffic("grouped_up", "wide_routing") is None
    assert bench.measured_traffic("decode_up", "scout_prefill") is None
    assert bench.measured_traffic("grouped_up", None) is None
    src.write_text("kernel as profiled, then edited\n")
    assert bench.measured_traffic("grouped_up", "scout_prefill") is None
    src.unlink()
    assert bench.measured_traffic("grouped_up", "scout_prefill") is None

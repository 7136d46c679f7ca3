#!/usr/bin/env python3
"""Benchmark of the int4 Mixture-of-Experts feed-forward layer on one MI355X.

A step is one full pass of the layer (router, top-k, dispatch, routed + shared
SwiGLU experts, gate-weighted combine) over one batch of synthetic tokens,
through the C ABI, with weights already quantized and resident in HBM. The
default workload is the Scout-shaped decode layer (T=16, d=5120, 16 routed
experts + 1 shared, h=8192, top-1, int4 g128); ``--config`` picks another of
the five benchmark layers.

Steps cycle through ``--layers`` independently seeded copies of the layer (as
consecutive layers of a model would), so a step streams weights that are not
in the 256 MB last-level cache from the step before.

Prints ONE JSON line: metric, value, unit, n_gpus, steps, warmup, ms_per_step,
higher_is_better, scaling, vs_baseline, dtype, data and config, plus
  roofline      the dominant kernel: algorithmic bytes (or FLOPs) per launch
                divided by its mean launch time, from HIP events the kernels
                record at their own start and end (a second, eager pass over
                the same steps), with the rocprofv3 counter traffic when the
                recorded measurement matches the kernel's sources;
  cpu_baseline  the CPU oracle (per-token C loop, fp64) timed on the host's
                cores over a bounded sample of the same workload, in tokens/s
                and GFLOP/s;
  detail        per-stage times, whole-step rates (HBM GB/s of every stage's
                algorithmic bytes, layer TFLOP/s, the grouped GEMMs' TFLOP/s),
                the practical HBM ceiling and the quantizer leg;
  prefill       with the default decode layer, the three prefill layers timed
                in the same run, each with its own roofline and CPU sample.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + TFLOP/s (prefill) and HBM GB/s (decode) on 1 MI355X"
HBM_PEAK_GBPS = 8000.0         # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
FP8_MFMA_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 MFMA
DEFAULT_STEPS = {0: 500, 1: 500, 2: 40, 3: 40, 4: 10}
DEFAULT_WARMUP = {0: 20, 1: 20, 2: 5, 3: 5, 4: 3}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--config", type=int, default=1, help="benchmark layer 0..4 (default 1)")
    ap.add_argument("--layers", type=int, default=None, help="independent layer copies to cycle")
    ap.add_argument("--path", default="auto", choices=["auto", "prefill", "decode", "hybrid", "prefill_wide"])
    ap.add_argument("--experts", default="int4", choices=["int4", "bf16", "fp8"],
                    help="routed expert weights: int4 g128 (default), bf16 (the baseline "
                         "path) or fp8 row-wise (the fp8_mixed path)")
    ap.add_argument("--group", type=int, default=128, choices=[128, 64, 32],
                    help="int4 experts: weights per scale (default 128)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=None, help="tokens in the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for HBM counter scaling)")
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--prefill", default=None,
                    help="comma-separated prefill layers also timed in the same run and "
                         "reported under `prefill` (default with the decode layer: 2,3,4; "
                         "'' for none)")
    ap.add_argument("--no-quantizer", action="store_true", help="skip the K1 quantizer leg")
    ap.add_argument("--stage-timing", default="separate", choices=["separate", "inline"],
                    help="per-kernel HIP events in a second pass (separate) or in the timed "
                         "loop itself (inline)")
    ap.add_argument("--graph", action="store_true",
                    help="replay each layer copy's forward as a captured HIP graph")
    a = ap.parse_args()
    if a.prefill is None:
        a.prefill = "2,3,4" if a.config == 1 else ""
    return a


def measured_traffic(stage: str, workload: str):
    """HBM bytes per launch of a stage on a workload from the committed
    rocprofv3 counter summary (profiles/traffic.json, records keyed
    "<stage>@<workload>"; a stage whose launch runs several kernels sums them),
    or None if there is no record or a source file of its kernels or their
    launch changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if workload is None or not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(f"{stage}@{workload}")
    if not rec or rec.get("workload") != workload:
        return None
    # every file that defines the kernel or its launch must be as profiled
    sources = rec.get("sources_sha256")
    if not sources:
        return None
    for rel, digest in sources.items():
        src = os.path.join(ROOT, rel)
        if not os.path.isfile(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != digest:
            return None
    return rec["hbm_bytes_per_launch"]


def layer_weight_bytes(cfg, experts: str = "int4", g: int = 128) -> int:
    if experts == "bf16":
        routed = cfg.E * 3 * cfg.h * cfg.d * 2
    elif experts == "fp8":
        routed = cfg.E * (3 * cfg.h * cfg.d + (2 * cfg.h + cfg.d) * 4)
    else:
        routed = cfg.E * 3 * (cfg.h * cfg.d // 2 + cfg.h * (cfg.d // g) * 4)
    shared = 3 * cfg.h * cfg.d * 2
    return routed + shared


def build_layer(cfg, dev, experts: str = "int4", group: int = 128):
    import torch
    import moe_ffn_int4_amd as moe
    import workloads as W
    x = W.gen_x(cfg)
    wr, b = W.gen_router(cfg)
    if experts == "bf16":
        ex = moe.Bf16Experts.empty(cfg.E, cfg.d, cfg.h, dev)
    elif experts == "fp8":
        ex = moe.Fp8Experts.empty(cfg.E, cfg.d, cfg.h, dev, W.FP8_ACT_UB)
    else:
        ex = moe.Int4Experts.empty(cfg.E, cfg.d, cfg.h, dev, group)
    for e in range(cfg.E):
        ws = [W.gen_expert_weight(cfg, w, e, dev) for w in ("w1", "w3", "w2")]
        if experts == "bf16":
            ex.set_expert(e, *(w.to(torch.bfloat16) for w in ws))
        else:
            ex.quantize_expert(e, *ws)
        del ws
    shared_raw = W.gen_shared(cfg, dev)
    shared = moe.pack_shared(*shared_raw)
    torch.cuda.synchronize()
    return dict(cfg=cfg, x=x.to(dev), wr=wr.to(dev), b=None if b is None else b.to(dev),
                experts=ex, shared=shared, shared_raw=shared_raw, x_cpu=x, wr_cpu=wr, b_cpu=b,
                routed=experts, group=group)


# the library's AUTO path choice (moe_int4.h): the streaming decode path up to
# 64 pairs; the hybrid path while the pairs average under 256 per routed
# expert, whose routed experts with at most 32 pairs stream beside the GEMMs
DECODE_MAX_PAIRS, HYBRID_AVG_PAIRS, HYBRID_ROWS = 64, 256, 32


def resolved_path(cfg, path: str) -> str:
    P = cfg.T * cfg.top_k
    if path != "auto":
        return path
    if P <= DECODE_MAX_PAIRS:
        return "decode"
    return "hybrid" if P < HYBRID_AVG_PAIRS * cfg.E else "prefill_wide"


def stage_units(cfg, counts, experts: str = "int4", g: int = 128, path: str = "auto"):
    """Algorithmic bytes and FLOPs of each stage for one launch, given the
    realized per-expert pair counts of the step (int4: g weights per scale).
    On the hybrid path the GEMM stages count the shared expert and the routed
    experts with more than HYBRID_ROWS pairs, the streaming stages the rest."""
    T, d, h, E, k = cfg.T, cfg.d, cfg.h, cfg.E, cfg.top_k
    P = T * k
    touched = int((counts > 0).sum())
    if experts == "bf16":
        w13, w2 = 2 * h * d * 2, d * h * 2          # one routed expert's W1 + W3, its W2
    elif experts == "fp8":
        w13, w2 = 2 * (h * d + h * 4), d * h + d * 4  # fp8 codes + row scales
    else:
        w13 = 2 * (h * d // 2 + h * (d // g) * 4)   # one routed expert's W1 + W3 (int4 + scales)
        w2 = d * h // 2 + d * (h // g) * 4          # its W2

    def units(n_exp, pairs, shared):
        """bytes, FLOPs of the up and down launches over n_exp routed experts
        holding `pairs` pairs, plus the shared expert's T rows if `shared`"""
        rows = pairs + (T if shared else 0)
        sw = 2 * h * d * 2 if shared else 0
        up_b = n_exp * w13 + sw + T * d * 2 + rows * h * 2
        dn_b = n_exp * w2 + sw // 2 + rows * h * 2 + rows * d * 4
        return (up_b, 4.0 * rows * d * h), (dn_b, 2.0 * rows * d * h)

    hybrid = resolved_path(cfg, path) == "hybrid"
    if hybrid:
        big = counts > HYBRID_ROWS
        small = (counts > 0) & ~big
        g_up, g_dn = units(int(big.sum()), int(counts[big].sum()), True)
        s_up, s_dn = units(int(small.sum()), int(counts[small].sum()), False)
        gemm_pairs = int(counts[big].sum())
    else:
        g_up, g_dn = units(touched, P, True)
        s_up, s_dn = g_up, g_dn
        gemm_pairs = P
    return {
        "router": (E * d * 4 + T * d * 2 + T * E * 4, 2.0 * T * d * E),
        "grouped_up": g_up,
        "grouped_down": g_dn,
        "decode_up": s_up,
        "decode_down": (s_dn[0] + T * d * 2, s_dn[1]),
        "combine": ((P + T) * d * 4 + T * d * 2, 2.0 * P * d),
        # fp8 experts: x rows, then H's routed rows, read (bf16) and written (fp8 + scale)
        "act_quant": (T * (d * 3 + 4) + P * (h * 3 + 4), 0.0),
        # FLOPs of the up / down launches on fp8 matrix cores (routed rows), the rest bf16
        "fp8_flops": {"grouped_up": 4.0 * gemm_pairs * d * h, "grouped_down": 2.0 * gemm_pairs * d * h}
        if experts == "fp8" else {},
        "touched": touched,
        "step_bytes": touched * (w13 + w2) + 3 * h * d * 2 + E * d * 4 + 2 * T * d * 2,
    }


def hbm_ceiling(dev, nbytes: int = 2 << 30, reps: int = 10):
    """Practical HBM rates on this device, from the library's measurement
    kernels (a streaming read with the decode kernels' non-temporal loads, and
    a plain copy) over buffers eight times the 256 MB last-level cache, timed
    with events on the current stream. The nominal peak stays the roofline's
    peak; these say how much of it plain streaming reaches."""
    import torch
    import moe_ffn_int4_amd as moe

    src = torch.empty(nbytes // 4, dtype=torch.int32, device=dev).fill_(0x5A5A5A5A)
    dst = torch.empty_like(src)
    sink = torch.empty(moe.hbm_read_sink_words(), dtype=torch.int32, device=dev)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        start.record()
        for _ in range(reps):
            fn()
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) * 1e-3 / reps

    t_read = timed(lambda: moe.hbm_read(src, sink))
    t_copy = timed(lambda: moe.hbm_copy(dst, src))
    del src, dst, sink
    torch.cuda.empty_cache()
    return {"read_GBps": nbytes / t_read / 1e9, "copy_GBps": 2 * nbytes / t_copy / 1e9,
            "buffer_bytes": nbytes}


def cpu_baseline(layer, n_sample, dev, min_seconds=10.0):
    """The CPU oracle on a bounded sample of the workload's tokens, repeated
    until at least min_seconds of CPU time are measured."""
    import numpy as np
    import torch
    import workloads as W
    from oracle import native, router_logits, select_topk
    from oracle.moe import Bf16Expert, Int4Expert

    cfg = layer["cfg"]
    n = min(n_sample, cfg.T)
    rows = np.linspace(0, cfg.T - 1, n).round().astype(np.int64)
    xs = layer["x_cpu"][torch.as_tensor(rows)]
    b = None if layer["b_cpu"] is None else layer["b_cpu"].numpy()
    ids, _ = select_topk(router_logits(xs, layer["wr_cpu"].numpy(), b), cfg.top_k)
    experts = [None] * cfg.E
    for e in sorted(set(ids.ravel().tolist())):
        if layer["routed"] == "bf16":  # the same bf16 rounding of the draws the GPU was given
            experts[e] = Bf16Expert(*(
                W.gen_expert_weight(cfg, w, e, dev).to(torch.bfloat16).cpu()
                .view(torch.int16).numpy().view(np.uint16).copy() for w in ("w1", "w3", "w2")))
            continue
        if layer["routed"] == "fp8":  # the oracle's own fp8 quantization of the same draws
            experts[e] = native.fp8_expert(
                *(W.gen_expert_weight(cfg, w, e, dev).cpu().numpy() for w in ("w1", "w3", "w2")),
                W.FP8_ACT_UB)
            continue
        parts = []  # oracle's own quantization of the same draws
        for w in ("w1", "w3", "w2"):
            parts.extend(native.quantize_int4(W.gen_expert_weight(cfg, w, e, dev).cpu().numpy(),
                                              layer["group"]))
        experts[e] = Int4Expert(*parts)
    shared = tuple(s.cpu() for s in layer["shared_raw"])
    native.lib()
    # the sample is run again until about min_seconds of CPU work are timed
    reps = 0
    t0 = time.perf_counter()
    while True:
        ref = native.moe_forward_per_token(xs, layer["wr_cpu"].numpy(), b, cfg.top_k, experts, shared,
                                           group_size=layer["group"])
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or reps >= 1000:
            break
    cores = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit():
        cores = min(cores, int(omp))
    return ref, rows, {
        "value": n * reps / dt, "unit": "tokens/s",
        # the layer's algorithmic FLOPs per token times the tokens run
        "GFLOP_per_s": n * reps * (cfg.flops() / cfg.T) / dt / 1e9,
        "cores": cores, "kind": "oracle",
        "cpu_model": cpu_model(), "omp_num_threads": omp or None,
        "sample": f"{n} of the {cfg.T} tokens of the first layer copy (fp64 per-token C loop, "
                  f"{len(set(ids.ravel().tolist()))} experts), run {reps} times; {dt:.2f} s wall",
    }


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def quantizer_leg(dev, reps: int = 20):
    """K1 alone: one 8192 x 5120 fp32 expert matrix (a W1 of the benchmark
    layers) quantized to int4 g128, row-major and tiled. Algorithmic bytes per
    call: 4 B read + 0.5 B codes + 4/128 B of scale written per weight."""
    import torch
    import moe_ffn_int4_amd as moe
    rows, K = 8192, 5120
    ws = [torch.randn(rows, K, device=dev) * 0.02 for _ in range(4)]  # 671 MB: past the LLC
    q = torch.empty(rows, K // 2, dtype=torch.uint8, device=dev)
    sc = torch.empty(rows, K // 128, dtype=torch.float32, device=dev)
    nbytes = rows * K * (4 + 0.5 + 4 / 128)
    out = {"matrix": f"{rows} x {K} fp32 -> int4 g128", "algorithmic_bytes": nbytes}
    for tiled in (False, True):
        for i in range(4):
            moe.quantize_int4(ws[i], q, sc, tiled=tiled)
        torch.cuda.synchronize()
        # the kernel's own duration (events it records at its start and end),
        # and the call rate of back-to-back calls (events around the calls)
        moe.profile_enable(True)
        moe.profile_read()
        for i in range(reps):
            moe.quantize_int4(ws[i % 4], q, sc, tiled=tiled)
        torch.cuda.synchronize()
        ms, n = moe.profile_read()["quantize"]
        moe.profile_enable(False)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(reps):
            moe.quantize_int4(ws[i % 4], q, sc, tiled=tiled)
        end.record()
        torch.cuda.synchronize()
        us = ms * 1e3 / n
        us_calls = start.elapsed_time(end) * 1e3 / reps
        out["tiled" if tiled else "row_major"] = {
            "us_per_launch": us, "GBps": nbytes / us / 1e3, "frac_of_peak": nbytes / us / 1e3 / HBM_PEAK_GBPS,
            "us_per_call_back_to_back": us_calls}
    del ws, q, sc
    torch.cuda.empty_cache()
    return out


def measure(ci: int, args, steps: int, warmup: int, cpu_sample: int, cpu_seconds: float,
            with_ceiling: bool):
    """Time `steps` forwards of benchmark layer `ci` (after `warmup`), per-stage
    kernel times, the dominant kernel's roofline and (optionally) the oracle
    baseline on a sample of the first layer copy; frees the layers after."""
    import numpy as np
    import torch
    import moe_ffn_int4_amd as moe
    import workloads as W

    dev = torch.device("cuda:0")
    cfg0 = W.config(ci)
    nlayers = args.layers or max(2, min(8, math.ceil(
        4e9 / layer_weight_bytes(cfg0, args.experts, args.group))))
    print(f"[bench] config {ci} {cfg0.name}: T={cfg0.T} d={cfg0.d} E={cfg0.E} h={cfg0.h} "
          f"k={cfg0.top_k}; {nlayers} layer copies, {warmup} warmup + {steps} timed steps",
          file=sys.stderr, flush=True)

    layers = [build_layer(cfg0.with_(seed=s), dev, args.experts, args.group) for s in range(nlayers)]
    ws = moe.alloc_workspace(cfg0.T, cfg0.d, cfg0.E, cfg0.h, cfg0.top_k, dev,
                             fp8=args.experts == "fp8")
    y = torch.empty(cfg0.T, cfg0.d, dtype=torch.bfloat16, device=dev)
    ids = [torch.empty(cfg0.T, cfg0.top_k, dtype=torch.int32, device=dev) for _ in layers]

    def step(i):
        L = layers[i % nlayers]
        moe.forward(L["x"], L["wr"], L["b"], L["experts"], L["shared"], cfg0.top_k,
                    path=args.path, y=y, topk_ids=ids[i % nlayers], workspace=ws)

    # each layer copy's per-expert pair counts (for the algorithmic bytes and
    # FLOPs of its launches), from the library's routing call, so they do not
    # depend on which copies the warmup steps reached
    counts = [moe.route(L["x"], L["wr"], L["b"], cfg0.top_k)["counts"].cpu().numpy().astype(np.int64)
              for L in layers]
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    print(f"[bench] warmup done; experts touched per layer copy: "
          f"{[int((c > 0).sum()) for c in counts]}", file=sys.stderr, flush=True)

    graphs = None
    if args.graph:
        graphs = []
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(nlayers):  # capture one forward per layer copy
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=side):
                    step(i)
                graphs.append(g)
        torch.cuda.current_stream().wait_stream(side)
        for i in range(warmup):
            graphs[i % nlayers].replay()
        torch.cuda.synchronize()

    def run(i):
        if graphs is not None:
            graphs[i % nlayers].replay()
        else:
            step(i)

    inline = args.stage_timing == "inline"
    moe.profile_enable(inline)
    moe.profile_read()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        run(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if inline:
        stages = moe.profile_read()
        moe.profile_enable(False)
    else:
        # the same steps again, eagerly, with the kernels recording HIP events
        # at their own start and end: per-kernel durations
        moe.profile_enable(True)
        moe.profile_read()
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        stages = moe.profile_read()
        moe.profile_enable(False)
    wall = t1 - t0
    ms_per_step = wall * 1e3 / steps

    units = [stage_units(L["cfg"], c, args.experts, args.group, args.path) for L, c in zip(layers, counts)]
    launched = {k: v for k, v in stages.items() if v[1] > 0}
    decode_like = cfg0.T * cfg0.top_k < 1024

    def roofline(stage):
        """algorithmic bytes (decode) or FLOPs (prefill) of one launch of
        `stage`, averaged over its launches in the timed steps (the decode
        projections launch twice a step: the shared expert's chunks and the
        routed ones), over its mean launch time"""
        st_ms, st_n = launched[stage]
        per_step = [u.get(stage, (0, 0.0)) for u in units]
        byts = sum(per_step[i % nlayers][0] for i in range(steps)) / st_n
        flops = sum(per_step[i % nlayers][1] for i in range(steps)) / st_n
        mean_s = st_ms / st_n / 1e3
        if decode_like:
            achieved = byts / mean_s / 1e9
            roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": achieved / HBM_PEAK_GBPS, "traffic": None}
        else:
            achieved = flops / mean_s / 1e12
            # the launch's FLOPs at their own dtype's peak: fp8 routed rows, bf16 the rest
            f8 = sum(units[i % nlayers]["fp8_flops"].get(stage, 0.0) for i in range(steps)) / st_n
            peak = flops / ((flops - f8) / BF16_MFMA_PEAK_TFLOPS + f8 / FP8_MFMA_PEAK_TFLOPS)
            roof = {"bound": "mfma", "achieved": achieved, "peak": peak,
                    "unit": "TFLOP/s", "frac": achieved / peak, "traffic": None}
        roof["traffic"] = measured_traffic(
            stage, cfg0.name if (args.experts == "int4" and args.group == 128) else None)
        if roof["traffic"] is not None:
            roof["traffic_unit"] = "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-scaled)"
        roof["kernel"] = stage
        roof["mean_launch_us"] = mean_s * 1e6
        roof["launches_per_step"] = st_n / steps
        roof["algorithmic_per_launch"] = byts if decode_like else flops
        return roof

    # the dominant kernel: the longest stage; on prefill layers the up projection's GEMM
    dom = max(launched, key=lambda k: launched[k][0])
    if not decode_like and "grouped_up" in launched:
        dom = "grouped_up"
    roof = roofline(dom)
    ceiling = hbm_ceiling(dev) if with_ceiling else None
    if decode_like and ceiling:
        # how much of plain streaming the kernel reaches (the nominal peak stays `peak`)
        roof["practical_hbm"] = dict(ceiling, frac_of_read=roof["achieved"] / ceiling["read_GBps"])

    step_bytes = sum(units[i % nlayers]["step_bytes"] for i in range(steps)) / steps
    # the grouped GEMM kernels alone (routed and shared up and down projections
    # on MFMA tiles): their FLOPs over their summed kernel time
    gemm_stages = [k for k in ("grouped_up", "grouped_down") if k in launched]
    gemm_tflops = None
    if gemm_stages:
        gf = sum(units[i % nlayers].get(k, (0, 0.0))[1] for k in gemm_stages for i in range(steps))
        gt = sum(launched[k][0] for k in gemm_stages) / 1e3
        gemm_tflops = gf / gt / 1e12
    detail = {
        "stages_us_per_step": {k: round(v[0] * 1e3 / steps, 2) for k, v in launched.items()},
        # the whole layer: algorithmic bytes of every stage's weights and
        # activations over the wall-clock step
        "step_hbm_GBps": step_bytes / (wall / steps) / 1e9,
        "step_hbm_frac": step_bytes / (wall / steps) / 1e9 / HBM_PEAK_GBPS,
        "step_TFLOPs": cfg0.flops() / (wall / steps) / 1e12,
        "gemm_TFLOPs": gemm_tflops,
        "touched_experts": [u["touched"] for u in units],
        "layer_copies": nlayers,
        "path": args.path,
        "graph": bool(args.graph),
        "stage_timing": args.stage_timing,
    }
    if ceiling:
        detail["practical_hbm"] = ceiling
    if "grouped_down" in launched and not decode_like:
        detail["grouped_down_roofline"] = {k: v for k, v in roofline("grouped_down").items()
                                           if k in ("achieved", "peak", "frac", "mean_launch_us")}

    base = None
    if cpu_sample > 0:
        ref, rows, base = cpu_baseline(layers[0], cpu_sample, dev, min_seconds=cpu_seconds)
        # spot parity of the same tokens on the GPU (layer copy 0)
        step(0)
        torch.cuda.synchronize()
        yg = y[torch.as_tensor(rows, device=dev)].float().cpu().numpy().astype(np.float64)
        err = np.abs(yg - ref.y).max(axis=1) / np.maximum(np.abs(ref.y).max(axis=1), 1e-6)
        base["gpu_vs_oracle_max_row_rel_err"] = float(err.max())

    res = {"cfg": cfg0, "steps": steps, "warmup": warmup, "ms_per_step": ms_per_step,
           "value": cfg0.T * steps / wall, "roofline": roof, "detail": detail, "cpu_baseline": base}
    del layers, ws, y, ids, graphs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def workload_name(cfg0, args) -> str:
    import workloads as W
    return (f"{cfg0.name}: T={cfg0.T} d={cfg0.d} E={cfg0.E}+1 shared h={cfg0.h} top_k={cfg0.top_k}, "
            + {"int4": f"int4 g{args.group}", "bf16": "bf16",
               "fp8": f"fp8 row-wise (act ub {W.FP8_ACT_UB:g})"}[args.experts]
            + " routed / bf16 shared")


def main() -> int:
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one MI355X: the library runs on a single GPU; "
              "--gpus must be 1 (expert parallelism across GPUs is a design, not implemented).",
              file=sys.stderr)
        return 2

    import torch
    import moe_ffn_int4_amd as moe

    if not os.path.exists(moe.LIB_PATH):
        from moe_ffn_int4_amd import build as _b
        _b.build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if moe.lib().moe_device_check() != 0:
        raise SystemExit(f"not a gfx950 device: {moe.lib().moe_last_error().decode()}")

    ci = args.config
    steps = args.steps if args.steps is not None else DEFAULT_STEPS[ci]
    warmup = args.warmup if args.warmup is not None else DEFAULT_WARMUP[ci]
    n_sample = 0 if args.no_cpu_baseline else (args.cpu_sample or None)
    import workloads as W
    cfg0 = W.config(ci)
    decode_like = cfg0.T * cfg0.top_k < 1024
    if n_sample is None:
        n_sample = 16 if decode_like else 8
    head = measure(ci, args, steps, warmup, n_sample, 10.0, with_ceiling=True)

    detail = head["detail"]
    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        detail["copy_calibration_bytes"] = n
        del src, dst

    out = {
        "metric": METRIC, "value": head["value"], "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8+bf16" if args.experts == "fp8" else "bf16", "data": "synthetic",
        "config": {"workload": workload_name(cfg0, args),
                   "T": cfg0.T, "d": cfg0.d, "E": cfg0.E, "h": cfg0.h, "top_k": cfg0.top_k,
                   "parallelism": "single GPU"},
        "roofline": head["roofline"],
    }
    if head["cpu_baseline"] is not None:
        out["cpu_baseline"] = head["cpu_baseline"]

    # the prefill half of the metric: the other benchmark layers in the same run
    prefill = [int(c) for c in args.prefill.split(",") if c.strip()] if args.prefill else []
    if prefill:
        out["prefill"] = {}
        for pc in prefill:
            if pc == ci:
                continue
            pcfg = W.config(pc)
            r = measure(pc, args, DEFAULT_STEPS[pc], DEFAULT_WARMUP[pc],
                        0 if args.no_cpu_baseline else (2 if pcfg.top_k > 1 else 4), 3.0,
                        with_ceiling=False)
            entry = {
                "workload": workload_name(pcfg, args),
                "steps": r["steps"], "warmup": r["warmup"],
                "ms_per_step": r["ms_per_step"], "tokens_per_s": r["value"],
                "layer_TFLOPs": r["detail"]["step_TFLOPs"],
                "gemm_TFLOPs": r["detail"]["gemm_TFLOPs"],
                "roofline": r["roofline"],
                "stages_us_per_step": r["detail"]["stages_us_per_step"],
                "touched_experts": r["detail"]["touched_experts"],
                "step_hbm_GBps": r["detail"]["step_hbm_GBps"],
            }
            if "grouped_down_roofline" in r["detail"]:
                entry["grouped_down_roofline"] = r["detail"]["grouped_down_roofline"]
            if r["cpu_baseline"] is not None:
                entry["cpu_baseline"] = r["cpu_baseline"]
            out["prefill"][pcfg.name] = entry
            print(f"[bench] {pcfg.name}: {r['ms_per_step']:.3f} ms/step, "
                  f"{r['roofline']['kernel']} {r['roofline']['frac']:.3f} of peak",
                  file=sys.stderr, flush=True)
    if not args.no_quantizer:
        detail["quantizer"] = quantizer_leg(dev)
    out["detail"] = detail
    line = json.dumps(out)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())

"""Helpers for the GPU parity tests: build a layer on the GPU from the seeded
workloads, and build the oracle's view of the same layer on the host.

Inputs come only from ``workloads``; the oracle's int4 codes come from the
oracle's own quantizer applied to the same fp32 draws, never from the GPU.
"""
from __future__ import annotations

import sys
from dataclasses import dataclass
from typing import Dict, Iterable, List, Optional

import numpy as np
import torch

import moe_ffn_int4_amd as moe
import workloads as W
from oracle import native
from oracle.moe import Bf16Expert, Int4Expert, MoEResult

TOL = 2e-2  # max relative error of an output row (infinity norm)
MARGIN = 1e-4  # top-k margin above which expert ids must match exactly


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


@dataclass
class Layer:
    cfg: W.MoEConfig
    x: torch.Tensor          # bf16 [T, d], CPU
    wr: torch.Tensor         # fp32 [E, d], CPU
    b: Optional[torch.Tensor]
    shared: tuple            # bf16, CPU
    gen_dev: str             # where routed weights are drawn
    dev: torch.device
    x_d: torch.Tensor
    wr_d: torch.Tensor
    b_d: Optional[torch.Tensor]
    shared_d: tuple
    experts_d: object        # moe.Int4Experts, moe.Bf16Experts or moe.Fp8Experts
    routed: str = "int4"     # routed expert weights: "int4", "bf16" or "fp8"
    act_ub: float = 0.0      # fp8 experts: activation scale bound
    group: int = 128         # int4 experts: weights per scale


def build_layer(cfg: W.MoEConfig, dev="cuda:0", routed_draw: Optional[str] = None,
                routed: str = "int4", act_ub: float = W.FP8_ACT_UB, group: int = 128) -> Layer:
    """The layer on the GPU. Routed weights are drawn on the CPU for small
    layers and on the GPU (then quantized there) for the 5120 x 8192 ones.
    ``routed="bf16"`` keeps the routed experts in bf16 (RNE of the same draws);
    ``routed="fp8"`` quantizes them to fp8 row-wise on the GPU (bound ``act_ub``);
    int4 experts use groups of ``group`` weights per scale."""
    dev = torch.device(dev)
    if routed_draw is None:
        routed_draw = "cpu" if cfg.d * cfg.h <= 1 << 22 else str(dev)
    x = W.gen_x(cfg)
    wr, b = W.gen_router(cfg)
    shared = W.gen_shared(cfg)
    if routed == "bf16":
        ex = moe.Bf16Experts.empty(cfg.E, cfg.d, cfg.h, dev)
    elif routed == "fp8":
        ex = moe.Fp8Experts.empty(cfg.E, cfg.d, cfg.h, dev, act_ub)
    else:
        ex = moe.Int4Experts.empty(cfg.E, cfg.d, cfg.h, dev, group)
    for e in range(cfg.E):
        ws = [W.gen_expert_weight(cfg, w, e, routed_draw).to(dev) for w in ("w1", "w3", "w2")]
        if routed == "bf16":
            ex.set_expert(e, *(w.to(torch.bfloat16) for w in ws))
        else:
            ex.quantize_expert(e, *ws)
        del ws
    torch.cuda.synchronize(dev)
    shared_d = moe.pack_shared(*(s.to(dev) for s in shared))
    torch.cuda.synchronize(dev)
    return Layer(cfg, x, wr, b, shared, routed_draw, dev, x.to(dev), wr.to(dev),
                 None if b is None else b.to(dev), shared_d, ex, routed, float(act_ub), int(group))


def oracle_expert(layer: Layer, e: int):
    """Expert e for the oracle from the same fp32 draw: quantized by the oracle
    (int4 and fp8 layers), or the same bf16 rounding the GPU was given (bf16 layers)."""
    if layer.routed == "bf16":
        bits = []
        for w in ("w1", "w3", "w2"):
            wb = W.gen_expert_weight(layer.cfg, w, e, layer.gen_dev).to(torch.bfloat16).cpu()
            bits.append(wb.view(torch.int16).numpy().view(np.uint16).copy())
            del wb
        return Bf16Expert(*bits)
    if layer.routed == "fp8":
        ws = [W.gen_expert_weight(layer.cfg, w, e, layer.gen_dev).cpu().numpy()
              for w in ("w1", "w3", "w2")]
        return native.fp8_expert(*ws, layer.act_ub)
    parts = []
    for w in ("w1", "w3", "w2"):
        wf = W.gen_expert_weight(layer.cfg, w, e, layer.gen_dev).cpu().numpy()
        parts.extend(native.quantize_int4(wf, layer.group))
        del wf
    return Int4Expert(*parts)


def oracle_forward_rows(layer: Layer, rows: np.ndarray, gpu_ids: Optional[np.ndarray] = None):
    """Oracle output for the tokens ``rows`` (per-token C loop).

    Where a token's top-k margin is <= MARGIN, several choices are correct;
    there the oracle evaluates the layer on the GPU's choice (``gpu_ids``).
    """
    from oracle import router_logits, select_topk
    cfg = layer.cfg
    xs = layer.x[torch.as_tensor(rows)]
    b = None if layer.b is None else layer.b.numpy()
    logits = router_logits(xs, layer.wr.numpy(), b)
    ids, margin = select_topk(logits, cfg.top_k)
    forced = None
    if gpu_ids is not None:
        tie = margin <= MARGIN
        if tie.any():
            forced = ids.copy()
            forced[tie] = gpu_ids[rows][tie]
            ids = forced
    need = sorted(set(int(e) for e in np.unique(ids)))
    experts: List = [None] * cfg.E
    for i, e in enumerate(need):
        experts[e] = oracle_expert(layer, e)
        if len(need) > 16 and (i + 1) % 32 == 0:
            say(f"  oracle: {i + 1}/{len(need)} experts quantized")
    # the per-token loop in batches of tokens, reporting progress between them
    batch = 32
    parts = []
    for i in range(0, len(rows), batch):
        parts.append(native.moe_forward_per_token(
            xs[i:i + batch], layer.wr.numpy(), b, cfg.top_k, experts, layer.shared,
            forced_ids=None if forced is None else forced[i:i + batch], group_size=layer.group))
        if len(rows) > batch:
            say(f"  oracle: {min(i + batch, len(rows))}/{len(rows)} tokens")
    r = MoEResult(*(np.concatenate([getattr(p, f) for p in parts])
                    for f in ("y", "ids", "gates", "logits", "margin")))
    return r, margin


def row_errors(y_gpu: torch.Tensor, y_ref: np.ndarray) -> np.ndarray:
    """Per-row ||y_gpu - y_ref||_inf / max(||y_ref||_inf, 1e-6)."""
    yg = y_gpu.float().cpu().numpy().astype(np.float64)
    num = np.abs(yg - y_ref).max(axis=1)
    den = np.maximum(np.abs(y_ref).max(axis=1), 1e-6)
    return num / den


def check_ids(gpu_ids: np.ndarray, ref_ids: np.ndarray, margin: np.ndarray) -> int:
    """Ids must match as sets wherever the margin exceeds MARGIN; returns #ties."""
    sure = margin > MARGIN
    a = np.sort(gpu_ids[sure], axis=1)
    b = np.sort(ref_ids[sure], axis=1)
    bad = np.nonzero(np.any(a != b, axis=1))[0]
    assert bad.size == 0, f"{bad.size} tokens with a clear margin chose different experts"
    return int((~sure).sum())


# The library's AUTO path choice, as include/moe_int4.h documents it: the
# streaming decode path up to 64 token-expert pairs; the hybrid path while the
# pairs average under 256 per routed expert, whose routed experts with at most
# 32 pairs are streamed in 16-row chunks beside the GEMMs; 256-row GEMM tiles
# otherwise. GEMM row tiles are 128 rows (hybrid, prefill) or 256 (prefill_wide,
# whose partial tiles of at most 128 rows run a half-tile body), so a row from
# every 128-row piece of an expert's slots reaches every tile and both halves.
DECODE_MAX_PAIRS, HYBRID_AVG_PAIRS, HYBRID_ROWS = 64, 256, 32
ROW_PIECE, CHUNK_ROWS = 128, 16


def resolved_path(T: int, E: int, top_k: int, path: str = "auto") -> str:
    if path != "auto":
        return path
    P = T * top_k
    if P <= DECODE_MAX_PAIRS:
        return "decode"
    return "hybrid" if P < HYBRID_AVG_PAIRS * E else "prefill_wide"


@dataclass
class Coverage:
    rows: np.ndarray   # tokens to check, ascending
    units: int         # work units (row pieces of GEMM tiles, streamed chunks)
    report: str


def covering_rows(ids: np.ndarray, E: int, path: str,
                  extra: Optional[np.ndarray] = None) -> Coverage:
    """Tokens whose rows reach every unit of work the GPU ran for this routing.

    From the GPU's expert ids [T, k], the slots of each expert are its pairs
    p = t * k + j in ascending order (the dispatch order). Units: every
    ROW_PIECE-slot piece of each expert run on GEMM tiles (its ragged tail
    included) and every CHUNK_ROWS-slot chunk of each streamed expert; the
    shared expert's ROW_PIECE-token pieces (CHUNK_ROWS on the decode path).
    Greedy: for each unit not yet reached, take the token of that unit that
    reaches the most units not yet reached (the unit's last row on ties).
    Every touched expert and every tile (so every XCD's range) then has a
    checked row; the result is asserted here, independently of the greedy.
    """
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    P = T * k
    pair_e = ids.reshape(-1)
    if pair_e.min() < 0 or pair_e.max() >= E:
        raise ValueError("expert id out of range")
    order = np.argsort(pair_e, kind="stable")          # slot -> pair
    counts = np.bincount(pair_e, minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    slot_of = np.empty(P, dtype=np.int64)
    slot_of[order] = np.arange(P)
    rank = slot_of - offsets[pair_e]                    # position inside its expert
    if path == "decode":
        usize = np.full(E, CHUNK_ROWS)
        shared_size = CHUNK_ROWS
    elif path == "hybrid":
        usize = np.where(counts <= HYBRID_ROWS, CHUNK_ROWS, ROW_PIECE)
        shared_size = ROW_PIECE
    else:
        usize = np.full(E, ROW_PIECE)
        shared_size = ROW_PIECE
    nunits = (counts + usize - 1) // usize
    ubase = np.concatenate([[0], np.cumsum(nunits)])
    n_routed = int(ubase[E])
    n_shared = (T + shared_size - 1) // shared_size
    pair_unit = ubase[pair_e] + rank // usize[pair_e]
    token_units = np.concatenate(
        [pair_unit.reshape(T, k), (n_routed + np.arange(T) // shared_size)[:, None]], axis=1)
    covered = np.zeros(n_routed + n_shared, dtype=bool)
    chosen = [] if extra is None else [int(t) for t in extra]
    for t in chosen:
        covered[token_units[t]] = True
    for u in range(n_routed + n_shared):
        if covered[u]:
            continue
        if u < n_routed:
            e = int(np.searchsorted(ubase, u, side="right") - 1)
            i = u - int(ubase[e])
            lo = int(offsets[e]) + i * int(usize[e])
            hi = min(lo + int(usize[e]), int(offsets[e + 1]))
            cands = order[lo:hi][::-1] // k
        else:
            i = u - n_routed
            cands = np.arange(i * shared_size, min((i + 1) * shared_size, T))[::-1]
        gain = (~covered[token_units[cands]]).sum(axis=1)
        t = int(cands[int(np.argmax(gain))])
        chosen.append(t)
        covered[token_units[t]] = True
    rows = np.unique(np.asarray(chosen, dtype=np.int64))
    # independent check: the chosen tokens' pairs reach every unit
    reach = np.zeros_like(covered)
    reach[token_units[rows].ravel()] = True
    assert reach.all(), "coverage selection missed a unit"
    touched = int((counts > 0).sum())
    seen = len(set(ids[rows].ravel().tolist()))
    streamed = int(((usize == CHUNK_ROWS) & (counts > 0)).sum()) if path != "decode" else touched
    report = (f"coverage[{path}]: experts {seen}/{touched} touched, routed units {n_routed}/{n_routed} "
              f"({streamed} experts in {CHUNK_ROWS}-row chunks, the rest in {ROW_PIECE}-row pieces), "
              f"shared units {n_shared}/{n_shared}, {len(rows)} of {T} tokens")
    return Coverage(rows, n_routed + n_shared, report)


def sample_rows(T: int, n: int, seed: int = 0) -> np.ndarray:
    if n >= T:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(T, size=n, replace=False))
    rows[0], rows[-1] = 0, T - 1  # the first and the last token always
    return np.unique(rows)

"""Seeded synthetic inputs for the int4 Mixture-of-Experts feed-forward layer.

This module only draws random tensors with the shapes and value distributions
of the five benchmark layers. It contains none of the layer's arithmetic: no
quantization, routing, activation or matrix products. The CPU oracle, the
tests, ``smoke()`` and ``bench.py`` all take their inputs from here, so both
sides of every parity check see the same bits.

Distributions (all seeded, seed 0 unless a caller overrides it):

* ``x``: fp32 N(0, 1) rounded to bf16 (round to nearest even).
* router weight ``Wr`` [E, d]: fp32 N(0, 0.02); the wide-routing layer uses
  U(-0.02, 0.02) instead.
* router bias ``b`` [E]: absent, N(0, 0.5) (Scout-shaped prefill), or the
  Zipf-shaped ``b_e = -c * ln(e + 1)`` (Maverick-shaped prefill).
* routed expert weights: fp32 N(0, 0.02), W1/W3 [h, d] and W2 [d, h] ("nt"
  layout: output rows, reduction dim contiguous). They are drawn one expert at
  a time so that the 128-expert layers (64 GB of fp32) never exist at once.
* shared expert weights S1/S3 [h, d], S2 [d, h]: fp32 N(0, 0.02) rounded to
  bf16.

Random streams: every tensor (and every expert of a routed tensor) has its own
``torch.Generator`` seeded from ``(seed, tensor id, expert)`` through a
splitmix64 mix. Values depend on the generator's device: torch's CPU and GPU
generators are different algorithms. x and the router are always drawn on the
CPU; expert weights (routed and shared) are drawn on whichever device the caller
names, and a parity check that needs them on the host copies the device draw
back.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import torch

# tensor ids for the per-tensor random streams
X, ROUTER_W, ROUTER_B, W1, W3, W2, S1, S3, S2 = range(1, 10)
ROUTED = {"w1": W1, "w3": W3, "w2": W2}

_MASK64 = (1 << 64) - 1


def _splitmix64(z: int) -> int:
    z = (z + 0x9E3779B97F4A7C15) & _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def stream_seed(seed: int, tensor_id: int, expert: int = 0) -> int:
    """63-bit seed of the random stream for one tensor (and one expert)."""
    z = _splitmix64(seed & _MASK64)
    z = _splitmix64(z ^ (tensor_id * 0x100000001B3))
    z = _splitmix64(z ^ (expert * 0xC2B2AE3D27D4EB4F))
    return z & ((1 << 63) - 1)


def _gen(seed: int, tensor_id: int, expert: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(stream_seed(seed, tensor_id, expert))
    return g


@dataclass(frozen=True)
class MoEConfig:
    """Shape and input distribution of one MoE feed-forward layer."""

    name: str
    T: int          # tokens in the batch
    d: int          # model dimension
    E: int          # routed experts
    h: int          # expert hidden dimension (routed and shared)
    top_k: int      # experts chosen per token
    router: str = "normal"      # "normal" N(0, 0.02) or "uniform" U(-0.02, 0.02)
    bias: str = "none"          # "none" | "normal" | "zipf"
    bias_param: float = 0.0     # std of the normal bias, or c of the Zipf bias
    seed: int = 0

    @property
    def pairs(self) -> int:
        return self.T * self.top_k

    def with_(self, **kw) -> "MoEConfig":
        return replace(self, **kw)

    def flops(self) -> float:
        """Algorithmic FLOPs: router + routed SwiGLU + shared SwiGLU."""
        return (2.0 * self.T * self.d * self.E
                + 6.0 * self.T * self.top_k * self.d * self.h
                + 6.0 * self.T * self.d * self.h)


# c of the Zipf-shaped bias, chosen once with the oracle's routing at seed 0 so
# that expert 0 receives about T * p1 tokens, p1 = 1 / H(128, 1.1) = 0.2257
# (the share of the head of a Zipf(1.1) law over 128 experts).
ZIPF_C = 0.79

CONFIGS = [
    MoEConfig("tiny", T=64, d=256, E=4, h=512, top_k=1),
    MoEConfig("scout_decode", T=16, d=5120, E=16, h=8192, top_k=1),
    MoEConfig("scout_prefill", T=8192, d=5120, E=16, h=8192, top_k=1,
              bias="normal", bias_param=0.5),
    MoEConfig("maverick_prefill", T=4096, d=5120, E=128, h=8192, top_k=1,
              bias="zipf", bias_param=ZIPF_C),
    MoEConfig("wide_routing", T=16384, d=5120, E=128, h=8192, top_k=8,
              router="uniform"),
]


# Activation scale upper bound of the layers built with fp8 routed experts: a
# parameter of the layer (like its weights), far above the row maxima of the
# N(0, 1) activations, so it binds only where a test lowers it.
FP8_ACT_UB = 1200.0


def config(i: int) -> MoEConfig:
    return CONFIGS[i]


# ----------------------------------------------------------------------------
# draws
# ----------------------------------------------------------------------------

def gen_x(cfg: MoEConfig) -> torch.Tensor:
    """Activations [T, d] bf16 (CPU)."""
    g = _gen(cfg.seed, X, 0, "cpu")
    return torch.randn(cfg.T, cfg.d, generator=g, dtype=torch.float32).to(torch.bfloat16)


def gen_router(cfg: MoEConfig):
    """Router weight [E, d] fp32 and bias [E] fp32 or None (CPU)."""
    g = _gen(cfg.seed, ROUTER_W, 0, "cpu")
    if cfg.router == "uniform":
        wr = torch.rand(cfg.E, cfg.d, generator=g, dtype=torch.float32) * 0.04 - 0.02
    else:
        wr = torch.randn(cfg.E, cfg.d, generator=g, dtype=torch.float32) * 0.02
    if cfg.bias == "none":
        b = None
    elif cfg.bias == "normal":
        gb = _gen(cfg.seed, ROUTER_B, 0, "cpu")
        b = torch.randn(cfg.E, generator=gb, dtype=torch.float32) * cfg.bias_param
    elif cfg.bias == "zipf":
        e = torch.arange(cfg.E, dtype=torch.float64)
        b = (-cfg.bias_param * torch.log(e + 1.0)).to(torch.float32)
    else:
        raise ValueError(f"unknown bias kind {cfg.bias!r}")
    return wr, b


def expert_shape(cfg: MoEConfig, which: str):
    return (cfg.d, cfg.h) if which == "w2" else (cfg.h, cfg.d)


def gen_expert_weight(cfg: MoEConfig, which: str, expert: int, device="cpu") -> torch.Tensor:
    """One routed expert's fp32 weight: W1/W3 [h, d], W2 [d, h], on ``device``."""
    g = _gen(cfg.seed, ROUTED[which], expert, device)
    return torch.randn(*expert_shape(cfg, which), generator=g, dtype=torch.float32,
                       device=device) * 0.02


def gen_shared(cfg: MoEConfig, device="cpu"):
    """Shared expert weights S1 [h, d], S3 [h, d], S2 [d, h] in bf16 on ``device``
    (drawn by that device's generator, like the routed weights)."""
    out = []
    for tid, shape in ((S1, (cfg.h, cfg.d)), (S3, (cfg.h, cfg.d)), (S2, (cfg.d, cfg.h))):
        g = _gen(cfg.seed, tid, 0, device)
        out.append((torch.randn(*shape, generator=g, dtype=torch.float32, device=device) * 0.02)
                   .to(torch.bfloat16))
    return tuple(out)


def zipf_head_share(E: int, s: float = 1.1) -> float:
    """Share of the most popular of E items under a Zipf(s) law."""
    return 1.0 / sum((i + 1) ** -s for i in range(E))


__all__ = [
    "MoEConfig", "CONFIGS", "config", "gen_x", "gen_router", "gen_expert_weight",
    "gen_shared", "expert_shape", "stream_seed", "zipf_head_share", "ZIPF_C",
]


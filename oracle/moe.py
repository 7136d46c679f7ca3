"""MoE feed-forward forward pass of the oracle, fp64 (test infrastructure only).

Follows the MoE forward described on the discosf.com page "1 卡跑通 Llama 4",
section "混合专家路由": the router scores every expert for each token, the top-k
experts are chosen, each chosen expert runs on its tokens, its output is added
back onto the token weighted by the token's score for it (``scatter_add_``),
and finally the shared expert's output, which every token goes through, is
added as well. This module computes it in that order: per expert, on the batch
of tokens routed to it, then a scatter-add.

Each expert is a SwiGLU FFN, ``(Swish(x W) * (x V)) W2`` with
``Swish(z) = z * sigmoid(z)`` (docs.ifdog.com page "Llama 开源模型系列", section
"SwiGLU：门控激活的数学"). Weights are stored "nt" (output rows, reduction dim
contiguous, as ``bmm_nt`` on the lshu.cn page): W1 = W and W3 = V are [h, d],
W2 is [d, h], so ``x W`` is ``x @ W1.T``.

Precision: everything in fp64. bf16 activations and bf16 shared weights widen
exactly; routed weights are ``code * scale`` (exact in fp64). Router logits are
accumulated in fp64 and then rounded to fp32: the top-k choice is an integer
decided by floating point, and it is taken in fp32, the precision the GPU
kernel decides it in.

Readings (where the pages are silent or disagree):

* score function: a sigmoid gate of the logit (the docs.ifdog.com page says a
  linear layer "usually" followed by softmax; the benchmark layer fixes a
  sigmoid gate). Experts are selected on the logits, which order them exactly
  as the sigmoid does.
* ties in top-k go to the lower expert id.
* the gate multiplies the expert's output (not its input); the k gates are not
  renormalised.
* an optional per-expert router bias is added to the logits before selection
  and before the sigmoid.
* the shared expert has gate 1 and the same hidden size as a routed expert.
* no residual connection: the result is the layer's output only.
* ``margin[t]`` = k-th minus (k+1)-th largest fp32 logit of token t (+inf when
  k = E). Where it is tiny, several id sets are correct; ``forced_ids`` lets a
  caller evaluate the layer on a given choice.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Optional, Sequence, Union

import numpy as np

from .quantize import GROUP, dequantize, int4_group_quantize


def _f64(a) -> np.ndarray:
    """Widen an array (numpy, or a torch CPU tensor of any float dtype) to fp64."""
    if hasattr(a, "detach"):  # torch tensor
        a = a.detach().to("cpu").float().numpy()
    return np.asarray(a, dtype=np.float64)


@dataclass
class Int4Expert:
    """One routed expert's quantized weights (codes int8 in [-8, 7], fp32 scales)."""

    c1: np.ndarray  # [h, d]
    s1: np.ndarray  # [h, d / 128]
    c3: np.ndarray  # [h, d]
    s3: np.ndarray  # [h, d / 128]
    c2: np.ndarray  # [d, h]
    s2: np.ndarray  # [d, h / 128]

    @staticmethod
    def from_fp32(w1, w3, w2, group_size: int = GROUP) -> "Int4Expert":
        c1, s1 = int4_group_quantize(w1, group_size)
        c3, s3 = int4_group_quantize(w3, group_size)
        c2, s2 = int4_group_quantize(w2, group_size)
        return Int4Expert(c1, s1, c3, s3, c2, s2)

    def dequantized(self, group_size: int = GROUP):
        return (dequantize(self.c1, self.s1, group_size),
                dequantize(self.c3, self.s3, group_size),
                dequantize(self.c2, self.s2, group_size))


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) to fp64, exactly: a bf16 is the top half of an fp32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@dataclass
class Bf16Expert:
    """One routed expert held in bf16: the pure-bf16 inference path, which the
    lshu.cn page (section "三条推理路径差异") lists as the accuracy baseline of the
    int4 and fp8 paths. W1, W3 [h, d] and W2 [d, h] as bf16 bit patterns."""

    w1: np.ndarray  # uint16 [h, d]
    w3: np.ndarray  # uint16 [h, d]
    w2: np.ndarray  # uint16 [d, h]

    def dequantized(self, group_size: int = GROUP):
        """The weights widened exactly to fp64 (group_size is unused)."""
        return bf16_bits_to_f64(self.w1), bf16_bits_to_f64(self.w3), bf16_bits_to_f64(self.w2)


@dataclass
class MoEResult:
    y: np.ndarray        # [T, d] fp64 layer output
    ids: np.ndarray      # [T, k] int32 chosen experts, by descending logit
    gates: np.ndarray    # [T, k] fp64 sigmoid of the chosen logits
    logits: np.ndarray   # [T, E] fp32 router logits (bias included)
    margin: np.ndarray   # [T] fp32 k-th minus (k+1)-th largest logit


def sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def silu(z):
    """Swish / SiLU: ``z * sigmoid(z)``."""
    z = np.asarray(z, dtype=np.float64)
    return z * sigmoid(z)


def router_logits(x, wr, b=None) -> np.ndarray:
    """``x @ Wr.T (+ b)`` accumulated in fp64, rounded to fp32: [T, E]."""
    acc = _f64(x) @ _f64(wr).T
    if b is not None:
        acc = acc + _f64(b)[None, :]
    return acc.astype(np.float32)


def select_topk(logits32, k: int):
    """Top-k experts per token by descending fp32 logit, ties to the lower id.

    Returns ``(ids [T, k] int32, margin [T] fp32)``.
    """
    logits32 = np.asarray(logits32, dtype=np.float32)
    T, E = logits32.shape
    if not 1 <= k <= E:
        raise ValueError("top_k must be in [1, E]")
    expert_ids = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((expert_ids, -logits32), axis=-1)  # primary: -logit, then id
    ids = order[:, :k].astype(np.int32)
    if k < E:
        kth = np.take_along_axis(logits32, order[:, k - 1:k], axis=1)[:, 0]
        nxt = np.take_along_axis(logits32, order[:, k:k + 1], axis=1)[:, 0]
        margin = (kth.astype(np.float64) - nxt.astype(np.float64)).astype(np.float32)
    else:
        margin = np.full(T, np.inf, dtype=np.float32)
    return ids, margin


def gate_scores(chosen_logits) -> np.ndarray:
    """Gate of each chosen expert: the sigmoid of its fp32 logit."""
    return sigmoid(chosen_logits)


def scatter_add(y, t_idx, weights, out) -> None:
    """``y[t_idx[i]] += weights[i] * out[i]`` (the pages' ``scatter_add_``)."""
    np.add.at(y, t_idx, weights[:, None] * out)


def swiglu(xrows, w1, w3, w2) -> np.ndarray:
    """``(silu(x W1^T) * (x W3^T)) W2^T`` in fp64 for rows of x."""
    x = _f64(xrows)
    a = x @ _f64(w1).T
    b = x @ _f64(w3).T
    return (silu(a) * b) @ _f64(w2).T


def shared_forward(x, s1, s3, s2) -> np.ndarray:
    """The shared expert on every token (bf16 weights widened exactly)."""
    return swiglu(x, s1, s3, s2)


ExpertSource = Union[Sequence[Union[Int4Expert, Bf16Expert]],
                     Callable[[int], Union[Int4Expert, Bf16Expert]]]


def moe_forward(x, wr, b, top_k: int, experts: ExpertSource, shared,
                forced_ids: Optional[np.ndarray] = None,
                group_size: int = GROUP) -> MoEResult:
    """The MoE feed-forward layer on every row of ``x``.

    ``experts`` is a sequence of ``Int4Expert`` (or ``Bf16Expert``) or a callable
    ``e -> expert``
    (so that large layers can be supplied one expert at a time; only experts
    that receive tokens are requested). ``shared`` is ``(S1, S3, S2)``.
    ``forced_ids`` [T, k], if given, replaces the top-k choice (the gates are
    still the sigmoids of those experts' logits).
    """
    xf = _f64(x)
    T = xf.shape[0]
    logits = router_logits(xf, wr, b)
    ids, margin = select_topk(logits, top_k)
    if forced_ids is not None:
        ids = np.asarray(forced_ids, dtype=np.int32).reshape(T, top_k)
    gates = gate_scores(np.take_along_axis(logits, ids.astype(np.int64), axis=1))

    get = experts if callable(experts) else (lambda e: experts[e])
    y = np.zeros((T, xf.shape[1]), dtype=np.float64)
    E = logits.shape[1]
    for e in range(E):
        t_idx, j_idx = np.nonzero(ids == e)  # pairs routed to e, in (t, j) order
        if t_idx.size == 0:
            continue
        ex = get(e)
        if hasattr(ex, "ffn"):  # experts with their own arithmetic (fp8 row-wise)
            out = ex.ffn(xf[t_idx])
        else:
            w1, w3, w2 = ex.dequantized(group_size)
            out = swiglu(xf[t_idx], w1, w3, w2)
        scatter_add(y, t_idx, gates[t_idx, j_idx], out)
    y += shared_forward(xf, *shared)
    return MoEResult(y=y, ids=ids, gates=gates, logits=logits, margin=margin)

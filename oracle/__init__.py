"""CPU oracle for the int4 Mixture-of-Experts feed-forward layer.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call, link or run anything in
this package. The product (``moe_ffn_int4_amd``) never touches it, and the two
share no code: no kernels, headers, helpers, tables or pre/post-processing.
Both sides take their inputs from the seeded generators in ``workloads``.

What it computes, and the passage each step follows (pages as titled in the
source set; no line numbers):

* ``quantize.int4_group_quantize`` -- the int4 group quantizer printed as
  ``int4_row_quantize`` on the discosf.com page "1 卡跑通 Llama 4", section
  "FP8 / Int4 混合量化": groups of 128 consecutive weights,
  ``scale = clamp(max|w|, min=1e-6) / 8``, ``code = clamp(round(w / scale), -8, 7)``.
  fp32 arithmetic, as the printed code does on a fp32 tensor.
* ``moe.moe_forward`` -- the MoE feed-forward of the same page, section
  "混合专家路由": router scores, top-k selection, each chosen expert's output
  added back to its token weighted by its score (``scatter_add_``), plus the
  shared expert that every token passes through. Experts are SwiGLU FFNs,
  ``(Swish(xW) * xV) W2`` with ``Swish(x) = x * sigmoid(x)``, from the
  docs.ifdog.com page "Llama 开源模型系列", section "SwiGLU：门控激活的数学".
  fp64 throughout (weights widened exactly).
* ``moe.Bf16Expert`` -- routed experts held in bf16 instead of int4: the
  pure-bf16 inference path, which the lshu.cn page lists (section
  "三条推理路径差异") as the accuracy baseline of the quantized paths. The
  forward is the same; the weights widen exactly.
* ``native`` -- the same forward written as a plain C per-token loop
  (``csrc/oracle.c``), plus the quantizer as a plain C loop. It pins the
  grouped numpy form: both must agree.

Readings where the pages are silent or ambiguous (router score function,
tie-breaking, bias, gate placement, int4 storage order) are listed in the
module docstrings of ``moe`` and ``quantize``.

Parity status: every function here is pinned by CPU tests (``tests/test_oracle_*``)
against hand-worked groups, closed forms, invariants and brute force.
"""
from .quantize import int4_group_quantize, dequantize  # noqa: F401
from .moe import (  # noqa: F401
    Bf16Expert, MoEResult, bf16_bits_to_f64, moe_forward, router_logits, select_topk, sigmoid,
    silu, swiglu, shared_forward,
)

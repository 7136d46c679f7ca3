"""FP8 row-wise path of the oracle (test infrastructure only).

The lshu.cn page "Llama 4 单卡量化推理与选型指南" (section "量化环节") shows
the fp8 branch of ``bmm_nt``: the activations are quantized per row to fp8
(``quantize_fp8_per_row(x, num_tokens, activation_scale_ub)``), the weights are
fp8 with one scale per row ("FP8 行级" in the section "三条推理路径差异"), and
the batched fp8 x fp8 product is scaled by both row scales and returned in
bf16 (``f8f8bf16_rowwise_batched``). This module computes that path.

Readings (the page shows the calls, not their arithmetic):

* fp8 is OCP E4M3 ("e4m3fn": 4 exponent bits, bias 7, 3 mantissa bits, no
  infinities, largest finite 448, subnormals down to 2^-9), the fp8 format
  gfx950's matrix cores take. Conversion rounds to nearest, ties to even.
* A weight row's scale is ``max(max|w|, 1e-12) / 448`` and its codes are
  ``fp8(w / scale)``; an activation row's scale is
  ``min(max(max|x|, 1e-12), ub) / 448`` with ``ub`` the activation scale upper
  bound, and its codes are ``fp8(clamp(x / scale, -448, 448))``. Scales and
  quotients are fp32 (the division correctly rounded).
* Where the page's calls return bf16 the value is rounded to bf16 (RNE): the
  two up-projections, the SwiGLU product (computed from those bf16 values)
  and the expert output. The sums of exact fp8 products are taken in fp64.
* The shared expert and the router are unchanged (bf16 weights, fp32 logits).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .moe import silu

FP8_MAX = 448.0
_TINY = np.float32(1e-12)
_FP8_MAX32 = np.float32(FP8_MAX)


def fp8_round(v) -> np.ndarray:
    """The fp8 (E4M3) value nearest to each element (ties to even), as fp64.

    |v| must be at most 448 (the quantizers clamp before converting). In each
    binade [2^e, 2^(e+1)) the spacing is 2^(e-3); below 2^-6 (subnormals) it is
    2^-9.
    """
    a = np.abs(np.asarray(v, dtype=np.float64))
    if np.any(a > FP8_MAX):
        raise ValueError("fp8_round expects |v| <= 448")
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    # log2 can be off by one at exact powers of two: fix the binade exactly
    e = np.where(np.exp2(e) > a, e - 1, e)
    e = np.where(np.exp2(e + 1) <= a, e + 1, e)
    spacing = np.exp2(np.maximum(e, -6.0) - 3.0)
    q = np.rint(a / spacing) * spacing  # exact: a / spacing is a short binary fraction
    return np.copysign(q, np.asarray(v, dtype=np.float64))


def fp8_encode(v) -> np.ndarray:
    """E4M3 bit patterns (uint8) of values that are already fp8 values."""
    v = np.asarray(v, dtype=np.float64)
    sign = (np.signbit(v)).astype(np.uint8) << 7
    a = np.abs(v)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.where(np.exp2(e) > a, e - 1, e)
    e = np.where(np.exp2(e + 1) <= a, e + 1, e)
    normal = a >= 2.0 ** -6
    exp_field = np.where(normal, e + 7, 0)
    mant = np.where(normal, (a / np.exp2(e) - 1.0) * 8.0, a / 2.0 ** -9)
    if not np.all(mant == np.rint(mant)):
        raise ValueError("fp8_encode expects fp8 values (use fp8_round first)")
    code = (exp_field.astype(np.int64) << 3) | mant.astype(np.int64)
    return (sign | code.astype(np.uint8)).astype(np.uint8)


def fp8_decode(codes) -> np.ndarray:
    """fp64 values of E4M3 bit patterns (0x7F / 0xFF are NaN)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    val = np.where(ef == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(ef - 7.0))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return sign * val


def bf16_round(v) -> np.ndarray:
    """Nearest bf16 value (ties to even), as fp64, for finite fp32-range values."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)  # fp64 -> fp32 rounds (RNE) first
    bits = f.view(np.uint32).astype(np.uint64)
    # ties to even on the dropped 16 bits
    rounded = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return rounded.astype(np.uint32).view(np.float32).astype(np.float64)


def quantize_rows(w, ub=None):
    """Row-wise fp8 quantization of fp32 values [R, K].

    Returns ``(codes uint8 [R, K], scales fp32 [R])``. ``ub`` (activation rows)
    caps the row maximum before the scale is formed; then the quotients are
    clamped to +-448 (values above the capped maximum saturate).
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    m = np.abs(w).max(axis=1)
    m = np.maximum(m, _TINY)
    if ub is not None:
        m = np.minimum(m, np.float32(ub))
    scales = (m / _FP8_MAX32).astype(np.float32)
    q = (w / scales[:, None]).astype(np.float32)
    q = np.clip(q, -_FP8_MAX32, _FP8_MAX32)
    return fp8_encode(fp8_round(q)), scales


def _rowwise_product(xq, sx, wq, sw):
    """bf16( (xq @ wq^T) * sx[:, None] * sw[None, :] ) with the sum of exact fp8
    products in fp64."""
    acc = fp8_decode(xq) @ fp8_decode(wq).T
    return bf16_round(acc * sx.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :])


@dataclass
class Fp8Expert:
    """One routed expert in fp8: codes (E4M3 bytes) and per-row fp32 scales.
    W1, W3 [h, d]; W2 [d, h]."""

    q1: np.ndarray
    s1: np.ndarray
    q3: np.ndarray
    s3: np.ndarray
    q2: np.ndarray
    s2: np.ndarray
    ub: float

    @staticmethod
    def from_fp32(w1, w3, w2, ub: float) -> "Fp8Expert":
        q1, s1 = quantize_rows(w1)
        q3, s3 = quantize_rows(w3)
        q2, s2 = quantize_rows(w2)
        return Fp8Expert(q1, s1, q3, s3, q2, s2, float(ub))

    def ffn(self, x) -> np.ndarray:
        """The expert on rows ``x`` (values of bf16 activations), fp64 result
        holding the bf16 expert output."""
        ub = self.ub if self.ub > 0 else None  # a bound <= 0 means none
        x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
        xq, sx = quantize_rows(x32, ub)
        a1 = _rowwise_product(xq, sx, self.q1, self.s1)
        a3 = _rowwise_product(xq, sx, self.q3, self.s3)
        h = bf16_round(silu(a1) * a3)
        hq, sh = quantize_rows(h.astype(np.float32), ub)
        return _rowwise_product(hq, sh, self.q2, self.s2)

"""Int4 group quantizer of the oracle (test infrastructure only).

Follows ``int4_row_quantize`` as printed on the discosf.com page
"1 卡跑通 Llama 4", section "FP8 / Int4 混合量化":

1. view the weights as consecutive groups of ``group_size`` (=128) values in
   memory order;
2. per group, the largest absolute value;
3. clamp it from below at 1e-6, then divide by 8: that is the group's scale;
4. divide every weight by its group's scale, round, clamp to [-8, 7], store as
   an 8-bit integer.

Precision: the printed code runs on a float32 tensor, so every step here is
float32 IEEE arithmetic: a correctly rounded fp32 division (never a multiply
by a reciprocal) and round-half-to-even (torch's ``round``). ``1e-6`` is the
float32 nearest to 1e-6 (0x358637BD), which is what a float32 ``clamp`` uses.

Readings (the pages leave these open):

* The comment next to the scale says "[-8, 8]" while the code clamps to
  [-8, 7]; the code is followed, so ``w / s >= 7.5`` maps to 7.
* The clamp at 1e-6 is applied to ``max|w|`` before the division by 8, as in
  the code (the smallest scale is therefore 1.25e-7).
* Groups run along the last (contiguous) axis, which is the reduction axis of
  the "nt" weight layout used by ``bmm_nt`` on the lshu.cn page.

Dequantization is symmetric: ``w_hat = code * scale`` (the lshu.cn page,
section "量化环节", passes all-zero zero-points to the int4 matmul).
"""
from __future__ import annotations

import numpy as np

GROUP = 128
_CLAMP_MIN = np.float32(1e-6)
_EIGHT = np.float32(8.0)


def int4_group_quantize(w, group_size: int = GROUP):
    """Quantize fp32 weights [..., K] to int4 codes (int8 storage) and fp32 scales.

    Returns ``(codes, scales)``: codes int8 with the shape of ``w``; scales fp32
    with shape ``w.shape[:-1] + (K // group_size,)``.
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.shape[-1] % group_size:
        raise ValueError("last dimension must be a multiple of the group size")
    groups = w.reshape(-1, group_size)
    max_val = np.abs(groups).max(axis=1, keepdims=True)
    scales = np.maximum(max_val, _CLAMP_MIN) / _EIGHT
    codes = np.clip(np.rint(groups / scales), -8, 7).astype(np.int8)
    return (codes.reshape(w.shape),
            scales.reshape(w.shape[:-1] + (w.shape[-1] // group_size,)))


def dequantize(codes, scales, group_size: int = GROUP):
    """``code * scale`` in fp64 (exact: a 4-bit integer times an fp32 value)."""
    codes = np.asarray(codes)
    scales = np.asarray(scales)
    c = codes.astype(np.float64).reshape(-1, group_size)
    s = scales.astype(np.float64).reshape(-1, 1)
    return (c * s).reshape(codes.shape)

"""Pins of the oracle's bf16 routed-expert path (CPU).

* E = 1, k = 1: the layer is sigmoid(logit) * SwiGLU_0(x) + SwiGLU_s(x), written
  out here with numpy float64 matmuls (the textbook SwiGLU FFN);
* int4 experts whose dequantized weights are exactly representable in bf16
  (power-of-two scales) give bit-identical results through the int4 and the
  bf16 expert types (the int4 path is pinned on its own);
* the C per-token loop equals the grouped numpy form.
"""
import numpy as np
import pytest
import torch

from oracle import Bf16Expert, bf16_bits_to_f64, moe_forward
from oracle import native
from oracle.moe import Int4Expert


def _bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (round to nearest even, via torch)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _layer(rng, T, d, h, E):
    x = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).to(torch.bfloat16)
    wr = (rng.standard_normal((E, d)) * 0.02).astype(np.float32)
    sh = tuple(torch.from_numpy((rng.standard_normal(s) * 0.02).astype(np.float32))
               .to(torch.bfloat16) for s in ((h, d), (h, d), (d, h)))
    return x, wr, sh


def _np_swiglu(x, w1, w3, w2):
    a = x @ w1.T
    b = x @ w3.T
    return (a / (1.0 + np.exp(-a)) * b) @ w2.T


def test_bits_widen_exactly():
    # values with at most 8 significant bits are bf16 values: they round-trip
    v = np.array([1.0, -2.5, 3.140625, 2.0 ** -100, -0.0, 65280.0], dtype=np.float32)
    np.testing.assert_array_equal(bf16_bits_to_f64(_bits(v)), v.astype(np.float64))
    # and any finite bit pattern widens as torch widens bf16 to fp32
    bits = np.random.default_rng(0).integers(0, 1 << 16, size=4096, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # drop inf / nan patterns
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(bf16_bits_to_f64(bits), want.astype(np.float64))


def test_single_expert_closed_form():
    rng = np.random.default_rng(3)
    T, d, h = 6, 128, 256
    x, wr, sh = _layer(rng, T, d, h, 1)
    ex = Bf16Expert(*(_bits(rng.standard_normal(s) * 0.05) for s in ((h, d), (h, d), (d, h))))
    w1, w3, w2 = ex.dequantized()
    xf = x.float().numpy().astype(np.float64)
    logit = xf @ wr.astype(np.float64).T
    gate = 1.0 / (1.0 + np.exp(-logit.astype(np.float32).astype(np.float64)))
    s1, s3, s2 = (t.float().numpy().astype(np.float64) for t in sh)
    want = gate * _np_swiglu(xf, w1, w3, w2) + _np_swiglu(xf, s1, s3, s2)
    got = moe_forward(x, wr, None, 1, [ex], sh)
    np.testing.assert_allclose(got.y, want, rtol=1e-12, atol=1e-12)
    got_c = native.moe_forward_per_token(x, wr, None, 1, [ex], sh)
    np.testing.assert_allclose(got_c.y, want, rtol=1e-10, atol=1e-12)


def test_matches_int4_experts_with_exact_bf16_values():
    rng = np.random.default_rng(5)
    T, d, h, E, k = 12, 256, 128, 3, 2
    x, wr, sh = _layer(rng, T, d, h, E)
    int4, bf16 = [], []
    for _ in range(E):
        mats = []
        for shape in ((h, d), (h, d), (d, h)):
            codes = rng.integers(-8, 8, size=shape).astype(np.int8)
            # one power-of-two scale per group of 128: code * scale is exact in bf16
            scales = np.exp2(-rng.integers(4, 12, size=(shape[0], shape[1] // 128))).astype(np.float32)
            mats.append((codes, scales))
        ie = Int4Expert(mats[0][0], mats[0][1], mats[1][0], mats[1][1], mats[2][0], mats[2][1])
        int4.append(ie)
        bf16.append(Bf16Expert(*(_bits(w) for w in ie.dequantized())))
    for a, b in zip(int4, bf16):
        for wa, wb in zip(a.dequantized(), b.dequantized()):
            np.testing.assert_array_equal(wa, wb)
    ya = moe_forward(x, wr, None, k, int4, sh)
    yb = moe_forward(x, wr, None, k, bf16, sh)
    np.testing.assert_array_equal(ya.y, yb.y)
    np.testing.assert_array_equal(ya.ids, yb.ids)


def test_per_token_loop_equals_grouped_form():
    rng = np.random.default_rng(9)
    T, d, h, E, k = 10, 128, 256, 4, 2
    x, wr, sh = _layer(rng, T, d, h, E)
    b = (rng.standard_normal(E) * 0.1).astype(np.float32)
    ex = [Bf16Expert(*(_bits(rng.standard_normal(s) * 0.05) for s in ((h, d), (h, d), (d, h))))
          for _ in range(E)]
    g = moe_forward(x, wr, b, k, ex, sh)
    c = native.moe_forward_per_token(x, wr, b, k, ex, sh)
    np.testing.assert_array_equal(g.ids, c.ids)
    np.testing.assert_allclose(c.y, g.y, rtol=1e-11, atol=1e-13)


def test_mixed_expert_types_are_rejected():
    rng = np.random.default_rng(1)
    x, wr, sh = _layer(rng, 2, 128, 128, 2)
    ie = Int4Expert.from_fp32(*(rng.standard_normal(s).astype(np.float32) * 0.02
                                for s in ((128, 128), (128, 128), (128, 128))))
    be = Bf16Expert(*(_bits(rng.standard_normal((128, 128))) for _ in range(3)))
    with pytest.raises(TypeError):
        native.moe_forward_per_token(x, wr, None, 1, [ie, be], sh)

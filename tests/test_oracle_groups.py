"""Pins of the oracle's int4 quantizer and layer at the smaller groups (64 and
32 weights per scale; the lshu.cn page, section "维护状态", expects smaller
group sizes next).

* the hand-worked groups (values worked by hand from the printed steps) give
  the same scale and codes when their group holds 64 or 32 weights, and the
  zero groups beside them take the clamp's scale and code 0;
* every group of random, tiny and near-tie rows equals exact rational
  arithmetic on its own 64 or 32 inputs, for the numpy and the C quantizer;
* a matrix with a different scale in every 32-wide piece round-trips exactly
  at groups of 32 and does not at 128 (so the group size reaches the scales);
* the layer at groups of 32 equals the plain SwiGLU on the dequantized weights
  computed here from codes and scales with library routines.
"""
import numpy as np
import pytest
import torch

from oracle import dequantize, int4_group_quantize, moe_forward, native
from oracle.moe import Int4Expert
from test_oracle_quantize import _exact_group, _golden_groups, _near_tie_groups
from fractions import Fraction

QUANTIZERS = {"numpy": int4_group_quantize, "c": native.quantize_int4}
CLAMP_SCALE_BITS = 0x340637BD  # fp32(1e-6) / 8


@pytest.mark.parametrize("impl", sorted(QUANTIZERS))
@pytest.mark.parametrize("g", [64, 32])
def test_hand_worked_groups_at_smaller_sizes(impl, g):
    for name, w128, scale_bits, codes128 in _golden_groups():
        if not np.all(w128[g:] == 0) and not np.all(w128 == w128[0]):
            continue
        w = w128.reshape(1, 128).copy()
        if np.all(w128 == w128[0]):           # a constant group stays constant
            want_codes = codes128
            want_bits = [scale_bits] * (128 // g)
        else:                                  # values in the first group, zeros after
            want_codes = codes128.copy()
            want_bits = [scale_bits] + [CLAMP_SCALE_BITS] * (128 // g - 1)
        c, s = QUANTIZERS[impl](w, g)
        assert s.shape == (1, 128 // g)
        assert [int(b) for b in s.view(np.uint32)[0]] == [int(b) for b in want_bits], name
        np.testing.assert_array_equal(c[0], want_codes, err_msg=name)


@pytest.mark.parametrize("impl", sorted(QUANTIZERS))
@pytest.mark.parametrize("g", [64, 32])
def test_exact_rational_reference_small_groups(impl, g):
    rng = np.random.default_rng(10 + g)
    rand = (rng.standard_normal((4, 128)) * 0.02).astype(np.float32)
    rand[0, :g] *= np.float32(40.0)            # groups of one row at very different scales
    tiny = (rng.standard_normal((2, 128)) * 1e-7).astype(np.float32)
    w = np.concatenate([rand, tiny, _near_tie_groups(rng)])
    c, s = QUANTIZERS[impl](w, g)
    assert s.shape == (w.shape[0], 128 // g)
    for r in range(w.shape[0]):
        for j in range(128 // g):
            s_ref, c_ref = _exact_group(w[r, j * g:(j + 1) * g])
            assert Fraction(float(s[r, j])) == s_ref, f"row {r} group {j} scale"
            np.testing.assert_array_equal(c[r, j * g:(j + 1) * g], c_ref, err_msg=f"row {r} group {j}")


def test_group_size_reaches_the_scales():
    rng = np.random.default_rng(5)
    codes = rng.integers(-8, 8, size=(16, 256)).astype(np.int8)
    codes[:, ::32] = -8
    scales = (2.0 ** rng.integers(-10, -3, size=(16, 8))).astype(np.float32)
    w = dequantize(codes, scales, 32).astype(np.float32)
    for impl in QUANTIZERS.values():
        c, s = impl(w, 32)
        np.testing.assert_array_equal(c, codes)
        np.testing.assert_array_equal(s, scales)
        c128, s128 = impl(w, 128)
        assert not np.array_equal(dequantize(c128, s128, 128), w.astype(np.float64))


def test_layer_at_groups_of_32_against_library_swiglu():
    rng = np.random.default_rng(6)
    T, d, h, E, k = 5, 128, 256, 3, 2
    x = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).to(torch.bfloat16)
    xf = x.float().numpy().astype(np.float64)
    wr = (rng.standard_normal((E, d)) * 0.1).astype(np.float32)
    experts, dense = [], []
    for _ in range(E):
        ws = [(rng.standard_normal(sh) * 0.05).astype(np.float32) for sh in ((h, d), (h, d), (d, h))]
        parts = []
        for w in ws:
            parts.extend(int4_group_quantize(w, 32))
        ex = Int4Expert(*parts)
        experts.append(ex)
        # dequantized by broadcasting each scale over its 32 codes (library ops only)
        dense.append([np.asarray(cc, np.float64) * np.repeat(np.asarray(sc, np.float64), 32, axis=1)
                      for cc, sc in ((ex.c1, ex.s1), (ex.c3, ex.s3), (ex.c2, ex.s2))])
    shared = tuple(torch.from_numpy((rng.standard_normal(sh) * 0.05).astype(np.float32))
                   .to(torch.bfloat16) for sh in ((h, d), (h, d), (d, h)))
    r = moe_forward(x, wr, None, k, experts, shared, group_size=32)
    sh = [s.float().numpy().astype(np.float64) for s in shared]

    def ffn(v, w1, w3, w2):
        a = torch.from_numpy(v @ w1.T)
        return ((torch.nn.functional.silu(a).numpy()) * (v @ w3.T)) @ w2.T

    want = ffn(xf, *sh)
    logits = xf @ wr.astype(np.float64).T
    for t in range(T):
        for j in range(k):
            e = int(r.ids[t, j])
            want[t] += 1.0 / (1.0 + np.exp(-np.float64(np.float32(logits[t, e])))) * \
                ffn(xf[t:t + 1], *dense[e])[0]
    np.testing.assert_allclose(r.y, want, rtol=1e-9, atol=1e-12)
    rc = native.moe_forward_per_token(x, wr, None, k, experts, shared, group_size=32)
    np.testing.assert_allclose(rc.y, want, rtol=1e-9, atol=1e-12)

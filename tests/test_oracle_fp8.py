"""Pins of the oracle's fp8 row-wise path (CPU).

* E4M3 rounding and encoding equal torch's float8_e4m3fn conversion (random
  values over the whole range, subnormals, and every exact tie); decoding
  equals torch's for all 256 bit patterns;
* bf16 rounding equals torch's;
* the row quantizers: a row's largest element maps to +-448, codes times the
  scale stay within half an fp8 step of the input, the activation bound caps
  the scale and saturates larger elements, all-zero rows give zero codes;
* the fp8 expert on inputs that are exact fp8 values with unit scales equals
  the plain SwiGLU FFN up to the bf16 / fp8 roundings of its intermediates.
"""
import numpy as np
import pytest
import torch

from oracle import moe_forward, swiglu
from oracle.fp8 import (FP8_MAX, Fp8Expert, bf16_round, fp8_decode, fp8_encode, fp8_round,
                        quantize_rows)


def _torch_fp8_bits(v):
    return torch.from_numpy(np.asarray(v, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def _all_fp8_values():
    codes = np.arange(256, dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    return codes, vals


def test_encoding_matches_torch_random():
    rng = np.random.default_rng(0)
    mag = np.exp2(rng.uniform(-12, np.log2(FP8_MAX), 200_000))
    v = (mag * rng.choice([-1.0, 1.0], mag.size)).astype(np.float32)
    np.testing.assert_array_equal(fp8_encode(fp8_round(v)), _torch_fp8_bits(v))


def test_encoding_matches_torch_on_ties():
    codes, vals = _all_fp8_values()
    finite = np.sort(np.unique(vals[np.isfinite(vals) & (vals >= 0)]))
    mids = (finite[:-1] + finite[1:]) / 2  # exact midpoints: ties
    v = np.concatenate([mids, -mids]).astype(np.float32)
    assert np.all(v.astype(np.float64) == np.concatenate([mids, -mids]))
    np.testing.assert_array_equal(fp8_encode(fp8_round(v)), _torch_fp8_bits(v))


def test_decoding_matches_torch():
    codes, vals = _all_fp8_values()
    np.testing.assert_array_equal(np.isnan(fp8_decode(codes)), np.isnan(vals))
    ok = ~np.isnan(vals)
    np.testing.assert_array_equal(fp8_decode(codes)[ok], vals[ok])
    assert fp8_decode(np.array([126], np.uint8))[0] == 448.0


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    v = (rng.standard_normal(100_000) * np.exp2(rng.integers(-20, 20, 100_000))).astype(np.float32)
    want = torch.from_numpy(v).to(torch.bfloat16).float().numpy().astype(np.float64)
    np.testing.assert_array_equal(bf16_round(v), want)


def test_row_quantizer_invariants():
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((64, 512)) * 0.02).astype(np.float32)
    w[3] = 0.0
    codes, scales = quantize_rows(w)
    assert codes.dtype == np.uint8 and scales.dtype == np.float32
    deq = fp8_decode(codes) * scales.astype(np.float64)[:, None]
    assert np.all(fp8_decode(codes[3]) == 0)
    for r in (0, 7, 63):
        i = np.argmax(np.abs(w[r]))
        assert abs(fp8_decode(codes[r, i])) == FP8_MAX
    # within half an fp8 step of the quotient (step = 2^(e-3), relative <= 1/16)
    q = w.astype(np.float64) / scales.astype(np.float64)[:, None]
    err = np.abs(fp8_decode(codes) - q)
    step = np.exp2(np.maximum(np.floor(np.log2(np.maximum(np.abs(q), 2.0 ** -9))), -6) - 3)
    assert np.all(err <= step / 2 * (1 + 1e-6))
    assert np.all(np.abs(deq - w) <= np.abs(w) / 16 + scales[:, None] * 2.0 ** -10)


def test_activation_bound_caps_the_scale():
    x = np.array([[1.0, -2.0, 500.0, 3.0], [0.5, 0.25, -0.125, 0.0]], dtype=np.float32)
    codes, scales = quantize_rows(x, ub=100.0)
    assert scales[0] == np.float32(np.float32(100.0) / np.float32(448.0))
    assert fp8_decode(codes[0, 2]) == FP8_MAX  # 500 saturates
    free, s_free = quantize_rows(x)  # no bound: the row max sets the scale
    assert s_free[0] == np.float32(np.float32(500.0) / np.float32(448.0))
    assert scales[1] == s_free[1]  # under the bound nothing changes
    np.testing.assert_array_equal(codes[1], free[1])


def test_fp8_expert_against_swiglu_on_exact_inputs():
    """With fp8-exact weights whose rows reach 448 (unit scales) and fp8-exact
    activations reaching 448, only the bf16 roundings of the products and the
    fp8 quantization of the hidden row differ from the plain FFN."""
    rng = np.random.default_rng(3)
    codes, vals = _all_fp8_values()
    pool = vals[np.isfinite(vals) & (np.abs(vals) <= 64) & (np.abs(vals) >= 1)]
    d, h, T = 128, 256, 5

    def mat(r, c, div):
        m = rng.choice(pool, size=(r, c)) * rng.choice([-1.0, 1.0], size=(r, c))
        # each row reaches |448| once, at its own column: row scale = 448 / div / 448
        m[np.arange(r), rng.integers(0, c, r)] = 448.0 * rng.choice([-1.0, 1.0], r)
        return m / div

    w1, w3, w2 = mat(h, d, 4096.0), mat(h, d, 4096.0), mat(d, h, 4096.0)
    x = mat(T, d, 64.0)
    ex = Fp8Expert.from_fp32(w1.astype(np.float32), w3.astype(np.float32), w2.astype(np.float32),
                             ub=1e6)
    np.testing.assert_array_equal(ex.s1, np.float32(2.0 ** -12))
    np.testing.assert_array_equal(fp8_decode(ex.q1) * 2.0 ** -12, w1)
    got = ex.ffn(x)
    want = swiglu(x, w1, w3, w2)
    # the hidden row's fp8 quantization moves each element by at most half a
    # step, 1/16 of it relative; the bf16 roundings add ~2^-9
    rel = np.abs(got - want).max(axis=1) / np.abs(want).max(axis=1)
    assert rel.max() < 1 / 16, rel
    # and a plausible slip (the gate and linear branches swapped) lands far outside
    bad = swiglu(x, w3, w1, w2)
    assert (np.abs(bad - want).max(axis=1) / np.abs(want).max(axis=1)).min() > 2 / 16


def test_fp8_layer_closed_form_all_ties():
    """Router weights and bias zero: every logit ties, ids 0..k-1, gates 0.5."""
    rng = np.random.default_rng(4)
    T, d, h, E, k = 4, 128, 128, 3, 2
    x = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).to(torch.bfloat16)
    ex = [Fp8Expert.from_fp32(*(rng.standard_normal(s).astype(np.float32) * 0.05
                                for s in ((h, d), (h, d), (d, h))), ub=1200.0) for _ in range(E)]
    sh = tuple(torch.zeros(s, dtype=torch.bfloat16) for s in ((h, d), (h, d), (d, h)))
    r = moe_forward(x, np.zeros((E, d), np.float32), None, k, ex, sh)
    np.testing.assert_array_equal(r.ids, np.tile(np.arange(k), (T, 1)))
    xf = x.float().numpy().astype(np.float64)
    want = 0.5 * (ex[0].ffn(xf) + ex[1].ffn(xf))
    np.testing.assert_allclose(r.y, want, rtol=0, atol=0)


# ---- the C loop form (oracle/csrc/oracle.c) against the pinned numpy form

def test_c_fp8_values_match_torch():
    # all 256 codes, the two NaN patterns included (NaN compares equal here)
    from oracle import native
    codes, vals = _all_fp8_values()
    assert np.isnan(vals).sum() == 2
    got = np.array([native.lib().oracle_fp8_value(int(c)) for c in codes])
    np.testing.assert_array_equal(got, vals)


@pytest.mark.parametrize("ub", [None, 0.75])
def test_c_row_quantizer_matches_numpy(ub):
    from oracle import native
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((24, 384)) * np.exp2(rng.integers(-12, 8, (24, 1)))).astype(np.float32)
    w[3] = 0.0                                     # all-zero row
    w[5, :] = np.float32(2.0 ** -30)               # tiny row: scale floor 1e-12
    codes, vals = _all_fp8_values()
    finite = np.sort(np.unique(vals[np.isfinite(vals) & (vals >= 0)]))
    mids = (finite[:-1] + finite[1:]) / 2            # every tie (scale 1: row maximum 448)
    w[6, :mids.size] = mids
    w[6, mids.size] = 448.0
    w[7, :mids.size] = -mids
    w[7, mids.size] = -448.0
    qn, sn = quantize_rows(w, ub)
    qc, sc = native.quantize_fp8_rows(w, ub)
    np.testing.assert_array_equal(sc, sn)
    np.testing.assert_array_equal(qc, qn)


def test_c_fp8_layer_matches_numpy():
    """The per-token C loop and the grouped numpy form of a small fp8 layer: the
    fp8 sums are exact in both, so they differ only where exp() rounds apart."""
    from oracle import native
    rng = np.random.default_rng(11)
    T, d, h, E, k = 9, 256, 384, 4, 2
    x = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).to(torch.bfloat16)
    wr = (rng.standard_normal((E, d)) * 0.1).astype(np.float32)
    b = (rng.standard_normal(E) * 0.1).astype(np.float32)
    experts = [native.fp8_expert((rng.standard_normal((h, d)) * 0.05).astype(np.float32),
                                 (rng.standard_normal((h, d)) * 0.05).astype(np.float32),
                                 (rng.standard_normal((d, h)) * 0.05).astype(np.float32), 2.0)
               for _ in range(E)]
    shared = tuple(torch.from_numpy((rng.standard_normal(s) * 0.05).astype(np.float32))
                   .to(torch.bfloat16) for s in ((h, d), (h, d), (d, h)))
    r_np = moe_forward(x.float().numpy(), wr, b, k, experts, shared)
    r_c = native.moe_forward_per_token(x, wr, b, k, experts, shared)
    np.testing.assert_array_equal(r_c.ids, r_np.ids)
    err = np.abs(r_c.y - r_np.y).max(axis=1) / np.abs(r_np.y).max(axis=1)
    assert err.max() < 1e-2, err.max()
    # most rows agree to the last bit of every bf16 rounding
    assert np.mean(err < 1e-12) >= 0.5, err

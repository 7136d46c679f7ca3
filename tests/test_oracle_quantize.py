"""Pins of the oracle's int4 group quantizer (CPU only).

The quantizer is int4_row_quantize from the discosf.com page, section
"FP8 / Int4 混合量化". It is pinned by:

* hand-worked groups (tests/golden/int4_groups.json);
* exact rational arithmetic: the code must equal round-half-even of the
  correctly rounded fp32 quotient, computed here with Python fractions, on
  random data and on crafted near-ties;
* invariants (scale recovery, code range, rounding error bound, round trip);
* the numpy form and the plain C loop agreeing bit for bit.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import dequantize, int4_group_quantize
from oracle import native

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "int4_groups.json")
G = 128
F32_1EM6 = np.float32(1e-6)


def _golden_groups():
    with open(GOLDEN) as f:
        spec = json.load(f)
    assert spec["group_size"] == G
    out = []
    for g in spec["groups"]:
        w = np.zeros(G, dtype=np.float32)
        codes = np.zeros(G, dtype=np.int8)
        if "fill" in g:
            w[:] = np.float32(g["fill"])
            codes[:] = g["codes_fill"]
        else:
            w[:len(g["values"])] = np.asarray(g["values"], dtype=np.float32)
            codes[:len(g["codes"])] = g["codes"]
        out.append((g["name"], w, np.uint32(int(g["scale_bits"], 16)), codes))
    return out


QUANTIZERS = {"numpy": int4_group_quantize, "c": native.quantize_int4}


# ------------------------------------------------------------ exact reference

def _fp32_round(q: Fraction) -> Fraction:
    """Correctly round a rational to the nearest fp32 (ties to even), normal range."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # choose e so that 2^23 <= a / 2^(e-23) < 2^24
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    assert -126 <= e <= 127, "outside the fp32 normal range"
    scaled = a / Fraction(2) ** (e - 23)  # in [2^23, 2^24)
    m = round(scaled)  # Fraction.__round__: half to even
    return sign * Fraction(m) * Fraction(2) ** (e - 23)


def _exact_group(w32: np.ndarray):
    """Scale and codes of one group by exact arithmetic on the fp32 inputs."""
    m = max(Fraction(float(abs(v))) for v in w32)
    m = max(m, Fraction(float(F32_1EM6)))
    s = m / 8  # exact: /8 of an fp32 is an fp32 (no underflow at these sizes)
    codes = []
    for v in w32:
        q32 = _fp32_round(Fraction(float(v)) / s)
        c = round(q32)  # half to even
        codes.append(min(7, max(-8, c)))
    return s, np.asarray(codes, dtype=np.int8)


# ---------------------------------------------------------------------- pins

@pytest.mark.parametrize("impl", sorted(QUANTIZERS))
def test_hand_worked_groups(impl):
    for name, w, scale_bits, codes in _golden_groups():
        c, s = QUANTIZERS[impl](w.reshape(1, G))
        assert s.shape == (1, 1)
        assert s.view(np.uint32)[0, 0] == scale_bits, f"group {name} scale"
        np.testing.assert_array_equal(c[0], codes, err_msg=f"group {name} codes")


def _near_tie_groups(rng):
    """Groups whose quotients sit at n + 0.5 and one fp32 ulp either side."""
    groups = []
    for gmax in (1.0, 0.7, 0.0123, 3.3e-3, 2.0e-6):
        s = np.float32(np.float32(gmax) / np.float32(8))
        vals = [np.float32(gmax)]
        for n in range(-8, 8):
            t = np.float32((n + 0.5) * float(s))
            vals += [t, np.nextafter(t, np.float32(np.inf)), np.nextafter(t, np.float32(-np.inf))]
        vals = [v for v in vals if abs(v) <= np.float32(gmax)]
        w = np.zeros(G, dtype=np.float32)
        w[:len(vals)] = vals[:G]
        rng.shuffle(w[1:])
        groups.append(w)
    return np.stack(groups)


@pytest.mark.parametrize("impl", sorted(QUANTIZERS))
def test_exact_rational_reference(impl):
    rng = np.random.default_rng(1)
    rand = (rng.standard_normal((6, G)) * 0.02).astype(np.float32)
    tiny = (rng.standard_normal((2, G)) * 1e-7).astype(np.float32)
    w = np.concatenate([rand, tiny, _near_tie_groups(rng)])
    c, s = QUANTIZERS[impl](w)
    for r in range(w.shape[0]):
        s_ref, c_ref = _exact_group(w[r])
        assert Fraction(float(s[r, 0])) == s_ref, f"row {r} scale"
        np.testing.assert_array_equal(c[r], c_ref, err_msg=f"row {r}")


def test_invariants_on_random_weights():
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((256, 1024)) * 0.02).astype(np.float32)
    w[3, 128:256] = 0.0            # an all-zero group
    w[7, :128] *= np.float32(1e-5)  # a group below the clamp
    c, s = int4_group_quantize(w)
    assert c.dtype == np.int8 and s.dtype == np.float32
    assert c.shape == w.shape and s.shape == (256, 8)
    assert c.min() >= -8 and c.max() <= 7
    grp = w.reshape(256, 8, G)
    m = np.abs(grp).max(axis=2)
    # scale recovers clamp(max|w|) exactly: /8 is exact in fp32
    np.testing.assert_array_equal((s * np.float32(8)).view(np.uint32),
                                  np.maximum(m, F32_1EM6).view(np.uint32))
    err = np.abs(grp.astype(np.float64) - c.reshape(grp.shape) * s[..., None].astype(np.float64))
    half = s[..., None].astype(np.float64) / 2
    clamped = c.reshape(grp.shape) == 7
    assert np.all(err[~clamped] <= half.repeat(G, -1)[~clamped] * (1 + 1e-6))
    assert np.all(err[clamped] <= 2 * half.repeat(G, -1)[clamped] * (1 + 1e-6))


def test_round_trip_of_representable_weights():
    rng = np.random.default_rng(3)
    codes = rng.integers(-8, 8, size=(64, 512)).astype(np.int8)
    codes[:, ::G] = -8  # every group reaches -8, so max|w| = 8 * scale
    scales = (2.0 ** rng.integers(-12, -2, size=(64, 4))
              * (1 + rng.integers(0, 2 ** 10, size=(64, 4)) / 2 ** 10)).astype(np.float32)
    w = dequantize(codes, scales).astype(np.float32)
    assert np.array_equal(w.astype(np.float64), dequantize(codes, scales))  # exact in fp32 too
    for impl in QUANTIZERS.values():
        c, s = impl(w)
        np.testing.assert_array_equal(c, codes)
        np.testing.assert_array_equal(s, scales)


def test_numpy_and_c_forms_agree_bitwise():
    rng = np.random.default_rng(4)
    w = (rng.standard_normal((512, 2048)) * 0.02).astype(np.float32)
    w[::17] *= np.float32(3e-5)
    ties = np.tile(_near_tie_groups(rng), (103, 1))[:512]
    w = np.concatenate([w, ties], axis=1)
    c1, s1 = int4_group_quantize(w)
    c2, s2 = native.quantize_int4(w)
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_array_equal(s1.view(np.uint32), s2.view(np.uint32))


def test_rejects_ragged_groups():
    with pytest.raises(ValueError):
        int4_group_quantize(np.zeros((2, 100), dtype=np.float32))

"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case patches one step of the numpy oracle with a plausible mistake (a
dropped term, a wrong sign, a transposed operand, a swapped branch, a wrong
rounding or clamp) and checks that at least one pin from
test_oracle_quantize / test_oracle_moe then fails. The mistakes live only in
this test, inside monkeypatch, on the CPU.
"""
import numpy as np
import pytest

import oracle.moe as M
import oracle.quantize as Q
import test_oracle_moe as pins_moe
import test_oracle_quantize as pins_q


def _quant_pins():
    pins_q.test_hand_worked_groups("numpy")
    pins_q.test_exact_rational_reference("numpy")
    pins_q.test_round_trip_of_representable_weights()


def _moe_pins():
    for k in (1, 2, 3):
        pins_moe.test_closed_form_permutation_layer("numpy", k)
    pins_moe.test_all_zero_router_ties_to_lowest_ids("numpy")
    pins_moe.test_zero_routed_weights_leave_the_shared_expert("numpy")
    pins_moe.test_single_expert_is_textbook_swiglu()
    pins_moe.test_representable_weights_match_fp32_weights_through_torch()
    pins_moe.test_topk_against_brute_force_with_ties()


def _swiglu_swapped(xrows, w1, w3, w2):
    x = M._f64(xrows)
    return (M.silu(x @ M._f64(w3).T) * (x @ M._f64(w1).T)) @ M._f64(w2).T


def _swiglu_w2_untransposed(xrows, w1, w3, w2):
    x = M._f64(xrows)
    return (M.silu(x @ M._f64(w1).T) * (x @ M._f64(w3).T)) @ M._f64(w2)


def _swiglu_w1_untransposed(xrows, w1, w3, w2):
    x = M._f64(xrows)
    return (M.silu(x @ M._f64(w1)) * (x @ M._f64(w3).T)) @ M._f64(w2).T


def _topk_ties_high(logits32, k):
    logits32 = np.asarray(logits32, dtype=np.float32)
    T, E = logits32.shape
    order = np.lexsort((-np.broadcast_to(np.arange(E), (T, E)), -logits32), axis=-1)
    return order[:, :k].astype(np.int32), np.zeros(T, np.float32)


_orig_router = M.router_logits
_orig_clip = np.clip


MUTATIONS = {
    # quantizer
    "scale divides by 7": (Q, "_EIGHT", np.float32(7.0), _quant_pins),
    "clamp applied after /8": (Q, "_CLAMP_MIN", np.float32(8e-6), _quant_pins),
    "round half away from zero": (Q.np, "rint", lambda a: np.trunc(a + np.copysign(0.5, a)),
                                  _quant_pins),
    "clamp to [-8, 8]": (Q.np, "clip", lambda a, lo, hi: _orig_clip(a, lo, 8), _quant_pins),
    # MoE forward
    "Swish dropped": (M, "silu", lambda z: np.asarray(z, dtype=np.float64), _moe_pins),
    "Swish on the V branch": (M, "swiglu", _swiglu_swapped, _moe_pins),
    "W2 not transposed": (M, "swiglu", _swiglu_w2_untransposed, _moe_pins),
    "W1 not transposed": (M, "swiglu", _swiglu_w1_untransposed, _moe_pins),
    "gate left out": (M, "gate_scores", lambda l: np.ones_like(np.asarray(l, np.float64)),
                      _moe_pins),
    "softmax-style gate exp(l)": (M, "gate_scores", lambda l: np.exp(np.asarray(l, np.float64)),
                                  _moe_pins),
    "scatter_add overwrites": (M, "scatter_add",
                               lambda y, t, w, o: y.__setitem__(t, w[:, None] * o), _moe_pins),
    "shared expert dropped": (M, "shared_forward",
                              lambda x, s1, s3, s2: 0.0 * M.swiglu(x, s1, s3, s2), _moe_pins),
    "router bias subtracted": (M, "router_logits",
                               lambda x, wr, b=None: _orig_router(
                                   x, wr, None if b is None else -np.asarray(b, np.float32)),
                               _moe_pins),
    "ties to the higher id": (M, "select_topk", _topk_ties_high, _moe_pins),
    "scale dropped in dequant": (M, "dequantize",
                                 lambda c, s, g=128: np.asarray(c, np.float64), _moe_pins),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    module, attr, value, pins = MUTATIONS[name]
    monkeypatch.setattr(module, attr, value)
    with pytest.raises(AssertionError):
        pins()


def test_pins_pass_unmutated():
    _quant_pins()
    _moe_pins()

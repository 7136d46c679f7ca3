"""Pins of the oracle's MoE forward (CPU only).

The layer is the discosf.com page's MoE forward (section "混合专家路由") with
SwiGLU experts (docs.ifdog.com page, section "SwiGLU：门控激活的数学"). Pins:

* closed form: experts whose W1, W3, W2 are scaled permutation matrices (and
  a router whose rows are scaled unit vectors) give an output that is known
  element by element. Distinct, non-involutive permutations make a transposed
  operand, swapped W1/W3, a wrong gate or a dropped shared expert visible;
* all-zero router: every logit ties, so ids are 0..k-1 and every gate is 0.5;
* x = 0 gives y = 0; zero routed weights give the shared expert alone;
* E = 1, k = 1 and int4-representable weights reduce to textbook SwiGLU,
  computed here with torch fp64 library routines on the original fp32 weights;
* permuting tokens permutes outputs; k = E sends every token everywhere;
* the grouped numpy form equals the per-token C loop;
* top-k against brute force over all k-subsets, margins by definition.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import native
from oracle.moe import Int4Expert, MoEResult, moe_forward, select_topk

G = 128


def _bf16(a):
    return torch.as_tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)


def _sig(z):
    return 1.0 / (1.0 + math.exp(-z))


# --------------------------------------------------------------- closed form

def _perm_matrix(n, perm, value):
    """W[i, perm[i]] = value, zeros elsewhere: (x @ W.T)[i] = value * x[perm[i]]."""
    w = np.zeros((n, n), dtype=np.float32)
    w[np.arange(n), perm] = value
    return w


class PermLayer:
    """A layer whose output is known in closed form (d = h = n)."""

    def __init__(self, n=256, E=3, k=1, T=6, seed=0, bias=True):
        rng = np.random.default_rng(seed)
        self.n, self.E, self.k, self.T = n, E, k, T
        # bf16-exact activations with distinct magnitudes
        self.x = np.round(rng.standard_normal((T, n)) * 8) / 8
        self.x = self.x.astype(np.float32)

        def perm():
            while True:
                p = rng.permutation(n)
                if np.any(p[p] != np.arange(n)):  # not an involution
                    return p
        # router: logit[t, e] = delta_e * x[t, j_e] + b_e
        self.j = rng.choice(n, size=E, replace=False)
        self.delta = 2.0 ** rng.integers(-3, 1, size=E)
        self.wr = np.zeros((E, n), dtype=np.float32)
        self.wr[np.arange(E), self.j] = self.delta
        self.b = (rng.integers(-4, 5, size=E) / 8).astype(np.float32) if bias else None
        # routed experts: negative powers of two so each row's only non-zero is
        # code -8 exactly (scale = |value| / 8), all other groups code 0
        self.p1 = [perm() for _ in range(E)]
        self.p3 = [perm() for _ in range(E)]
        self.p2 = [perm() for _ in range(E)]
        self.al = -(2.0 ** rng.integers(-2, 1, size=E))
        self.be = -(2.0 ** rng.integers(-2, 1, size=E))
        self.ga = -(2.0 ** rng.integers(-2, 1, size=E))
        self.experts = [Int4Expert.from_fp32(_perm_matrix(n, self.p1[e], self.al[e]),
                                             _perm_matrix(n, self.p3[e], self.be[e]),
                                             _perm_matrix(n, self.p2[e], self.ga[e]))
                        for e in range(E)]
        # shared expert in bf16 (0.5 and 0.25 are bf16-exact)
        self.q1, self.q3, self.q2 = perm(), perm(), perm()
        self.shared = (_bf16(_perm_matrix(n, self.q1, 0.5)), _bf16(_perm_matrix(n, self.q3, 0.25)),
                       _bf16(_perm_matrix(n, self.q2, 1.0)))

    def expected(self):
        n, E, k, T = self.n, self.E, self.k, self.T
        y = np.zeros((T, n))
        ids = np.zeros((T, k), dtype=np.int32)
        gates = np.zeros((T, k))
        for t in range(T):
            x = [float(v) for v in self.x[t]]
            logit = [self.delta[e] * x[self.j[e]] + (0.0 if self.b is None else float(self.b[e]))
                     for e in range(E)]
            order = sorted(range(E), key=lambda e: (-logit[e], e))
            for jj, e in enumerate(order[:k]):
                ids[t, jj] = e
                g = _sig(logit[e])
                gates[t, jj] = g
                for m in range(n):
                    nn = self.p2[e][m]
                    a = self.al[e] * x[self.p1[e][nn]]
                    b = self.be[e] * x[self.p3[e][nn]]
                    y[t, m] += g * self.ga[e] * (a * _sig(a)) * b
            for m in range(n):
                nn = self.q2[m]
                a = 0.5 * x[self.q1[nn]]
                b = 0.25 * x[self.q3[nn]]
                y[t, m] += (a * _sig(a)) * b
        return y, ids, gates


def _run(impl, *args, **kw) -> MoEResult:
    fn = moe_forward if impl == "numpy" else native.moe_forward_per_token
    return fn(*args, **kw)


IMPLS = ["numpy", "c"]


@pytest.mark.parametrize("impl", IMPLS)
@pytest.mark.parametrize("k", [1, 2, 3])
def test_closed_form_permutation_layer(impl, k):
    L = PermLayer(k=k, seed=10 + k)
    y_ref, ids_ref, g_ref = L.expected()
    r = _run(impl, L.x, L.wr, L.b, k, L.experts, L.shared)
    np.testing.assert_array_equal(r.ids, ids_ref)
    np.testing.assert_allclose(r.gates, g_ref, rtol=1e-13)
    np.testing.assert_allclose(r.y, y_ref, rtol=1e-12, atol=1e-14)


def test_closed_form_dequantization_is_exact():
    L = PermLayer(seed=5)
    w1, _, _ = L.experts[0].dequantized()
    np.testing.assert_array_equal(w1, _perm_matrix(L.n, L.p1[0], L.al[0]).astype(np.float64))


# -------------------------------------------------------------- special cases

def _random_layer(T=24, d=256, h=384, E=4, k=1, seed=0, scale=0.02):
    rng = np.random.default_rng(seed)
    x = _bf16(rng.standard_normal((T, d)))
    wr = (rng.standard_normal((E, d)) * scale).astype(np.float32)
    b = (rng.standard_normal(E) * 0.1).astype(np.float32)
    w = [[(rng.standard_normal(s) * scale).astype(np.float32) for s in ((h, d), (h, d), (d, h))]
         for _ in range(E)]
    experts = [Int4Expert.from_fp32(*ws) for ws in w]
    shared = tuple(_bf16(rng.standard_normal(s) * scale) for s in ((h, d), (h, d), (d, h)))
    return x, wr, b, experts, shared, w


@pytest.mark.parametrize("impl", IMPLS)
def test_all_zero_router_ties_to_lowest_ids(impl):
    x, wr, b, experts, shared, _ = _random_layer(E=5, k=3)
    r = _run(impl, x, np.zeros_like(wr), None, 3, experts, shared)
    np.testing.assert_array_equal(r.ids, np.tile([0, 1, 2], (x.shape[0], 1)))
    np.testing.assert_array_equal(r.gates, 0.5)
    xf = x.float().numpy().astype(np.float64)
    ref = sum(0.5 * oracle.swiglu(xf, *experts[e].dequantized()) for e in range(3))
    ref = ref + oracle.shared_forward(xf, *shared)
    np.testing.assert_allclose(r.y, ref, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("impl", IMPLS)
def test_zero_tokens_give_zero(impl):
    x, wr, b, experts, shared, _ = _random_layer(k=2)
    r = _run(impl, torch.zeros_like(x), wr, b, 2, experts, shared)
    assert np.all(r.y == 0.0)


@pytest.mark.parametrize("impl", IMPLS)
def test_zero_routed_weights_leave_the_shared_expert(impl):
    x, wr, b, experts, shared, _ = _random_layer(k=2)
    zero = [Int4Expert.from_fp32(np.zeros_like(e.c1, dtype=np.float32),
                                 np.zeros_like(e.c3, dtype=np.float32),
                                 np.zeros_like(e.c2, dtype=np.float32)) for e in experts]
    r = _run(impl, x, wr, b, 2, zero, shared)
    ref = oracle.shared_forward(x.float().numpy().astype(np.float64), *shared)
    np.testing.assert_allclose(r.y, ref, rtol=1e-12, atol=1e-15)
    assert np.abs(ref).max() > 0


def _torch_swiglu(x, w1, w3, w2):
    x, w1, w3, w2 = (torch.as_tensor(np.asarray(a, dtype=np.float64)) for a in (x, w1, w3, w2))
    return (torch.nn.functional.silu(x @ w1.T) * (x @ w3.T)) @ w2.T


def test_single_expert_is_textbook_swiglu():
    """E = 1, k = 1 with int4-representable weights: y = sigmoid(logit) * SwiGLU + SwiGLU_s."""
    rng = np.random.default_rng(7)
    T, d, h = 16, 256, 512
    def representable(shape):
        codes = rng.integers(-8, 8, size=shape).astype(np.int8)
        codes[..., ::G] = -8
        # short mantissas so that code * scale is exact in fp32
        s = (rng.integers(128, 256, size=shape[:-1] + (shape[-1] // G,)) * 2.0 ** -17).astype(np.float32)
        return oracle.dequantize(codes, s).astype(np.float32)
    w1, w3, w2 = representable((h, d)), representable((h, d)), representable((d, h))
    x = _bf16(rng.standard_normal((T, d)))
    wr = (rng.standard_normal((1, d)) * 0.02).astype(np.float32)
    b = np.asarray([0.3], dtype=np.float32)
    shared = tuple(_bf16(rng.standard_normal(s) * 0.02) for s in ((h, d), (h, d), (d, h)))
    ex = [Int4Expert.from_fp32(w1, w3, w2)]
    xf = x.float().numpy().astype(np.float64)
    logit = torch.as_tensor(xf) @ torch.as_tensor(wr.astype(np.float64)).T + float(b[0])
    gate = torch.sigmoid(logit.to(torch.float32).to(torch.float64))
    ref = gate * _torch_swiglu(xf, w1, w3, w2) + _torch_swiglu(
        xf, *(s.to(torch.float64).numpy() for s in shared))
    for impl in IMPLS:
        r = _run(impl, x, wr, b, 1, ex, shared)
        np.testing.assert_array_equal(r.ids, 0)
        np.testing.assert_allclose(r.y, ref.numpy(), rtol=1e-11, atol=1e-14)


def test_representable_weights_match_fp32_weights_through_torch():
    """Quantization is lossless on int4-representable weights, so the int4 layer
    equals the layer on the original fp32 weights, computed with torch fp64."""
    rng = np.random.default_rng(8)
    T, d, h, E, k = 20, 256, 256, 3, 2
    def representable(shape):
        codes = rng.integers(-8, 8, size=shape).astype(np.int8)
        codes[..., 5::G] = -8
        s = (2.0 ** rng.integers(-9, -6, size=shape[:-1] + (shape[-1] // G,))).astype(np.float32)
        return oracle.dequantize(codes, s).astype(np.float32)
    ws = [[representable(s) for s in ((h, d), (h, d), (d, h))] for _ in range(E)]
    x = _bf16(rng.standard_normal((T, d)))
    wr = (rng.standard_normal((E, d)) * 0.05).astype(np.float32)
    shared = tuple(_bf16(rng.standard_normal(s) * 0.02) for s in ((h, d), (h, d), (d, h)))
    r = moe_forward(x, wr, None, k, [Int4Expert.from_fp32(*w) for w in ws], shared)
    xf = torch.as_tensor(x.float().numpy().astype(np.float64))
    y = _torch_swiglu(xf, *(s.to(torch.float64).numpy() for s in shared))
    for t in range(T):
        for j in range(k):
            e = int(r.ids[t, j])
            g = torch.sigmoid(torch.tensor(float(r.logits[t, e]), dtype=torch.float64))
            y[t] += g * _torch_swiglu(xf[t:t + 1], *ws[e])[0]
    np.testing.assert_allclose(r.y, y.numpy(), rtol=1e-11, atol=1e-14)


def test_token_permutation_equivariance():
    x, wr, b, experts, shared, _ = _random_layer(T=32, k=2, seed=3)
    perm = np.random.default_rng(0).permutation(32)
    r = moe_forward(x, wr, b, 2, experts, shared)
    rp = moe_forward(x[torch.as_tensor(perm)], wr, b, 2, experts, shared)
    np.testing.assert_array_equal(rp.ids, r.ids[perm])
    np.testing.assert_allclose(rp.y, r.y[perm], rtol=1e-13, atol=1e-16)


def test_k_equals_e_uses_every_expert():
    x, wr, b, experts, shared, _ = _random_layer(E=3, k=3, seed=4)
    r = moe_forward(x, wr, b, 3, experts, shared)
    assert np.all(np.sort(r.ids, axis=1) == np.arange(3))
    assert np.all(np.isinf(r.margin))
    xf = x.float().numpy().astype(np.float64)
    ref = oracle.shared_forward(xf, *shared)
    for e in range(3):
        ref = ref + oracle.sigmoid(r.logits[:, e])[:, None] * oracle.swiglu(xf, *experts[e].dequantized())
    np.testing.assert_allclose(r.y, ref, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("k", [1, 2, 4])
def test_grouped_form_equals_per_token_loop(k):
    x, wr, b, experts, shared, _ = _random_layer(T=40, E=6, k=k, seed=20 + k)
    r1 = moe_forward(x, wr, b, k, experts, shared)
    r2 = native.moe_forward_per_token(x, wr, b, k, experts, shared)
    np.testing.assert_array_equal(r1.ids, r2.ids)
    np.testing.assert_array_equal(r1.logits, r2.logits)
    np.testing.assert_allclose(r1.y, r2.y, rtol=1e-11, atol=1e-16)
    # forced ids flow through both forms the same way
    forced = np.roll(r1.ids, 1, axis=1) if k > 1 else (r1.ids + 1) % 6
    f1 = moe_forward(x, wr, b, k, experts, shared, forced_ids=forced)
    f2 = native.moe_forward_per_token(x, wr, b, k, experts, shared, forced_ids=forced)
    np.testing.assert_allclose(f1.y, f2.y, rtol=1e-11, atol=1e-16)


# ------------------------------------------------------------------- top-k

def _brute_topk(row, k):
    """The k-subset whose every member beats every non-member (ties: lower id wins)."""
    E = len(row)
    beats = lambda a, b: row[a] > row[b] or (row[a] == row[b] and a < b)
    for sub in itertools.combinations(range(E), k):
        rest = [e for e in range(E) if e not in sub]
        if all(beats(a, b) for a in sub for b in rest):
            return sorted(sub, key=lambda e: (-row[e], e))
    raise AssertionError("no top-k subset")


def test_topk_against_brute_force_with_ties():
    rng = np.random.default_rng(5)
    logits = rng.integers(-3, 4, size=(200, 7)).astype(np.float32) / 4  # many ties
    logits[:50] = rng.standard_normal((50, 7)).astype(np.float32)
    for k in range(1, 8):
        ids, margin = select_topk(logits, k)
        for t in range(logits.shape[0]):
            assert list(ids[t]) == _brute_topk(list(logits[t]), k)
            srt = sorted(logits[t], reverse=True)
            want = np.inf if k == 7 else np.float32(srt[k - 1] - srt[k])
            assert margin[t] == want


def test_c_topk_matches_brute_force():
    rng = np.random.default_rng(6)
    logits = rng.integers(-2, 3, size=(100, 6)).astype(np.float32)
    L = native.lib()
    for k in (1, 2, 5, 6):
        for t in range(100):
            row = np.ascontiguousarray(logits[t])
            ids = np.zeros(k, dtype=np.int32)
            L.oracle_topk_token(row.ctypes.data, 6, k, ids.ctypes.data)
            assert list(ids) == _brute_topk(list(row), k)

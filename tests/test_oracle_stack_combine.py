"""Pins of the oracle's weighted combine (K >= 2), of the residual stack and of
the margins that decide which GPU results are compared element by element.

Show HN page "धीमे कंप्यूटर पर GLM 5.2 चलाना", section "implemented features",
router item: the chosen experts' outputs are added with their renormalised
weights times routed_scaling_factor, plus the shared expert.  The stack of
layers is the reading x <- x + MoE(rmsnorm(x)) (the pages describe one layer).

Each pin is written as a function of the oracle module, so that the tests at
the bottom can run it on copies of the oracle with a plausible mistake
planted (slot weights paired in reverse, no normalisation before a layer,
normalisation after the add, a margin off by one slot) and check that the
pin catches it.
"""
import math
import sys
import types

import numpy as np
import pytest
from scipy.special import expit

from oracle import moe_oracle as orc

ORACLE_SRC = orc.__file__


def _rand_experts(g, n, H, I, bits):
    lo, hi = orc.code_range(bits)
    ex = {}
    for e in range(n):
        d = {}
        for m, (r, c) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
            d["q_" + m] = orc.pack_rows(g.integers(lo, hi + 1, size=(r, c)), bits)
            d["s_" + m] = g.uniform(0.005, 0.02, size=r).astype(np.float32)
        ex[e] = d
    return ex


def _one_hot_output(m, d, j, a, bits):
    """o_r = sd[r] * sum_i qd[r, i] * silu(a sg[i] qg[i, j]) * a su[i] qu[i, j]:
    the expert's output for x = a * unit(j), from its codes, in fp64 with
    Python floats (no matrix routine)."""
    qg = m.unpack_rows(d["q_gate"], bits)
    qu = m.unpack_rows(d["q_up"], bits)
    qd = m.unpack_rows(d["q_down"], bits)
    I = qg.shape[0]
    hv = []
    for i in range(I):
        gi = a * float(d["s_gate"][i]) * int(qg[i, j])
        ui = a * float(d["s_up"][i]) * int(qu[i, j])
        hv.append(gi / (1.0 + math.exp(-gi)) * ui)
    out = np.zeros(qd.shape[0])
    for r in range(qd.shape[0]):
        out[r] = float(d["s_down"][r]) * sum(int(qd[r, i]) * hv[i] for i in range(I))
    return out


# ------------------------------------------------------------------ pins

def pin_two_expert_combine(m, bits=4):
    """K = 2 in one group, bias +10 on expert a and +9 on expert b (so a fills
    slot 0 and b slot 1), x = alpha * unit(j), router entries giving clearly
    different sigmoid scores s_a and s_b, distinct scales everywhere and a
    live shared expert.  Then the weights are rsf * s / (s_a + s_b), in slot
    order, and y = w0 * o_a + w1 * o_b + o_shared, every o from its codes."""
    g = np.random.default_rng(100 + bits)
    E, S, H, I = 8, 1, 48, 24
    ex = _rand_experts(g, E + S, H, I, bits)
    a_e, b_e, j, alpha, rsf = 6, 2, 11, 1.5, 2.5
    Wr = np.zeros((E, H), np.float32)
    Wr[a_e, j] = 1.2                 # s_a = sigmoid(1.8)
    Wr[b_e, j] = -0.8                # s_b = sigmoid(-1.2)
    bias = np.zeros(E, np.float32)
    bias[a_e], bias[b_e] = 10.0, 9.0
    x = np.zeros((1, H), np.float32)
    x[0, j] = alpha
    r = m.moe_layer(x, Wr, bias, ex.__getitem__, n_group=1, topk_group=1, top_k=2, n_shared=S, rsf=rsf, bits=bits)
    assert r.idx.tolist() == [[a_e, b_e]]
    sa, sb = 1.0 / (1.0 + math.exp(-1.8)), 1.0 / (1.0 + math.exp(1.2))
    w = r.w[0].astype(np.float64)
    assert abs(w[0] - rsf * sa / (sa + sb)) <= 1e-6 and abs(w[1] - rsf * sb / (sa + sb)) <= 1e-6
    want = (w[0] * _one_hot_output(m, ex[a_e], j, alpha, bits) + w[1] * _one_hot_output(m, ex[b_e], j, alpha, bits)
            + _one_hot_output(m, ex[E], j, alpha, bits))
    np.testing.assert_allclose(r.y[0], want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def pin_stack_zero_down_is_identity(m):
    """With every down-scale zero each layer's output is exactly zero, so the
    stack leaves x unchanged through every layer."""
    g = np.random.default_rng(7)
    E, S, H, I, L = 8, 1, 64, 32, 3
    layers = []
    for _ in range(L):
        ex = _rand_experts(g, E + S, H, I, 4)
        for d in ex.values():
            d["s_down"][:] = 0.0
        layers.append(((g.standard_normal((E, H)) * 0.05).astype(np.float32),
                       g.uniform(-0.1, 0.1, E).astype(np.float32), ex.__getitem__))
    x0 = g.standard_normal((2, H)).astype(np.float32)
    res = m.moe_stack(x0, layers, n_group=4, topk_group=2, top_k=2, n_shared=S, rsf=2.5, bits=4)
    for r in res:
        np.testing.assert_array_equal(r.y, x0.astype(np.float64))


def pin_stack_one_layer_closed_form(m, bits=4):
    """x0 = alpha * unit(j) through one layer with K = 1 forced by bias and a
    silent shared expert: rmsnorm(x0) = alpha' * unit(j) with alpha' =
    alpha / sqrt(alpha^2 / H + eps) (rounded to fp32, as the device holds it),
    so x1 = x0 + rsf * o_(e*)(alpha') with o from the codes."""
    g = np.random.default_rng(30 + bits)
    E, S, H, I = 8, 1, 64, 32
    ex = _rand_experts(g, E + S, H, I, bits)
    ex[E]["s_down"][:] = 0.0
    e_star, j, alpha, rsf, eps = 3, 40, 1.75, 2.5, 1e-6
    bias = np.zeros(E, np.float32)
    bias[e_star] = 10.0
    Wr = (g.standard_normal((E, H)) * 0.05).astype(np.float32)
    x0 = np.zeros((1, H), np.float32)
    x0[0, j] = alpha
    res = m.moe_stack(x0, [(Wr, bias, ex.__getitem__)], n_group=1, topk_group=1, top_k=1, n_shared=S, rsf=rsf,
                      bits=bits)
    a1 = float(np.float32(alpha / math.sqrt(alpha * alpha / H + eps)))
    want = x0[0].astype(np.float64) + rsf * _one_hot_output(m, ex[e_star], j, a1, bits)
    np.testing.assert_allclose(res[0].y[0], want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def pin_stack_sees_only_the_normalised_stream(m):
    """rmsnorm(c x) = rmsnorm(x) up to the epsilon, so scaling the residual
    stream by c = 64 must leave each layer's routing and MoE output unchanged
    (x1 - x0 scales not at all); routing or multiplying on the un-normalised
    stream would change both."""
    g = np.random.default_rng(12)
    E, S, H, I, T = 16, 1, 128, 32, 4
    ex = _rand_experts(g, E + S, H, I, 4)
    Wr = (g.standard_normal((E, H)) * 0.05).astype(np.float32)
    b = g.uniform(-0.1, 0.1, E).astype(np.float32)
    x0 = g.standard_normal((T, H)).astype(np.float32)
    kw = dict(n_group=4, topk_group=2, top_k=4, n_shared=S, rsf=2.5, bits=4)
    r1 = m.moe_stack(x0, [(Wr, b, ex.__getitem__)], **kw)[0]
    r64 = m.moe_stack(64.0 * x0, [(Wr, b, ex.__getitem__)], **kw)[0]
    sure = r1.margin >= 1e-4
    assert sure.sum() >= T - 1
    np.testing.assert_array_equal(r1.idx[sure], r64.idx[sure])
    y1 = r1.y - x0.astype(np.float64)
    y64 = r64.y - 64.0 * x0.astype(np.float64)
    for t in np.flatnonzero(sure):
        assert np.abs(y64[t] - y1[t]).max() <= 1e-4 * np.abs(y1[t]).max()


def pin_order_margin(m):
    """order_margin is the smallest gap between the corrected scores of
    consecutive chosen slots: a hand-worked row, then perturbations far below
    the margin never reorder the slots."""
    s = np.array([[0.50, 0.90, 0.70, 0.30, 0.62, 0.10, 0.20, 0.60]])
    b = np.zeros(8, np.float32)
    idx, _ = m.select_experts(s.astype(np.float32), b, 1, 1, 4, 2.5)
    assert idx[0].tolist() == [1, 2, 4, 7]                # c: 0.90, 0.70, 0.62, 0.60: gaps 0.2, 0.08, 0.02
    assert abs(m.order_margin(s, b, idx)[0] - 0.02) <= 1e-12
    one = np.array([[0, -1, -1, -1]], np.int32)
    assert m.order_margin(s, b, one)[0] == np.inf          # one kept slot: no order to decide
    g = np.random.default_rng(21)
    s64 = expit(3.9 * g.standard_normal((40, 64)))
    bb = g.uniform(-0.1, 0.1, 64).astype(np.float32)
    i0, _ = m.select_experts(s64.astype(np.float32), bb, 8, 4, 8, 2.5)
    om = m.order_margin(s64, bb, i0)
    sm = m.selection_margin(s64, bb, 8, 4, 8)
    for t in range(40):
        eps = min(om[t], sm[t]) / 8
        pert = (s64[t] + g.uniform(-eps, eps, 64)).astype(np.float32)[None]
        i1, _ = m.select_experts(pert, bb, 8, 4, 8, 2.5)
        np.testing.assert_array_equal(i1[0], i0[t])


def pin_topp_margin(m):
    """topp_margin is the smallest distance between a score-ordered prefix sum
    and p times the total (relative to the total) or between consecutive
    scores: a hand-worked row, then perturbations far below the margin never
    change the kept prefix."""
    s = np.array([[0.4, 0.3, 0.2, 0.1]])
    idx = np.array([[0, 1, 2, 3]], np.int32)
    # prefix sums 0.4, 0.7, 0.9, 1.0 against p * total = 0.65: nearest is 0.7 -> 0.05
    assert abs(m.topp_margin(s, idx, 0.65)[0] - 0.05) <= 1e-12
    # against 0.95: the prefix sums are 0.05 away, the score gaps 0.1 apart
    assert abs(m.topp_margin(s, idx, 0.95)[0] - 0.05) <= 1e-12
    assert m.topp_margin(s, idx, 1.0)[0] == np.inf
    g = np.random.default_rng(23)
    s64 = expit(2.0 * g.standard_normal((40, 32)))
    bb = g.uniform(-0.1, 0.1, 32).astype(np.float32)
    for p in (0.3, 0.6, 0.85):
        ik, _ = m.select_experts(s64.astype(np.float32), bb, 4, 2, 6, 2.5)
        tm = m.topp_margin(s64, ik, p)
        sm = m.selection_margin(s64, bb, 4, 2, 6)
        i0, _, k0 = m.select_experts_topp(s64.astype(np.float32), bb, 4, 2, 6, 2.5, p)
        for t in range(40):
            eps = min(tm[t] * 0.3, sm[t]) / 8                 # total <= 6: absolute <= relative margin * total / 20
            pert = (s64[t] + g.uniform(-eps, eps, 32)).astype(np.float32)[None]
            i1, _, k1 = m.select_experts_topp(pert, bb, 4, 2, 6, 2.5, p)
            assert k1[0] == k0[t]
            assert sorted(i1[0].tolist()) == sorted(i0[t].tolist())


PINS = {
    "two_expert_combine": pin_two_expert_combine,
    "stack_zero_down": pin_stack_zero_down_is_identity,
    "stack_closed_form": pin_stack_one_layer_closed_form,
    "stack_scale_invariance": pin_stack_sees_only_the_normalised_stream,
    "order_margin": pin_order_margin,
    "topp_margin": pin_topp_margin,
}


@pytest.mark.parametrize("bits", [4, 8, 2])
def test_two_expert_combine_closed_form(bits):
    pin_two_expert_combine(orc, bits)


def test_stack_with_zero_down_scales_is_identity():
    pin_stack_zero_down_is_identity(orc)


@pytest.mark.parametrize("bits", [4, 2])
def test_stack_one_layer_closed_form(bits):
    pin_stack_one_layer_closed_form(orc, bits)


def test_stack_sees_only_the_normalised_stream():
    pin_stack_sees_only_the_normalised_stream(orc)


def test_order_margin():
    pin_order_margin(orc)


def test_topp_margin():
    pin_topp_margin(orc)


# ------------------------------------------------- planted mistakes are caught

def _mutant(old: str, new: str) -> types.ModuleType:
    """A copy of the oracle with one source fragment replaced."""
    with open(ORACLE_SRC) as f:
        src = f.read()
    assert src.count(old) == 1, old
    name = "oracle_mutant"
    mod = types.ModuleType(name)
    sys.modules[name] = mod                 # dataclasses look their module up while the class is built
    try:
        exec(compile(src.replace(old, new), name, "exec"), mod.__dict__)
    finally:
        del sys.modules[name]
    return mod


MUTANTS = {
    # the routed slots' weights paired with the experts in reverse slot order
    "weights_reversed": ("coef = float(w[t, slot]) if slot < top_k else 1.0",
                         "coef = float(w[t, top_k - 1 - slot]) if slot < top_k else 1.0",
                         ["two_expert_combine"]),
    # the layer routes and multiplies on the raw residual stream
    "no_norm": ("xn = rmsnorm(x).astype(np.float32)", "xn = x.astype(np.float32)",
                ["stack_closed_form", "stack_scale_invariance"]),
    # the stream is normalised after the residual add
    "norm_after_add": ("x = x + r.y", "x = rmsnorm(x + r.y)", ["stack_zero_down", "stack_closed_form"]),
    # the order margin skips the last gap
    "order_margin_short": ("d = v[:-1] - v[1:]", "d = (v[:-1] - v[1:])[:-1] if len(v) > 2 else np.array([np.inf])",
                           ["order_margin"]),
    # the top-p margin measured against p of the total without the prefix sums' nearest point
    "topp_margin_first_only": ("m = np.min(np.abs(cum - top_p * total)) / max(total, 1e-300)",
                               "m = np.abs(cum[0] - top_p * total) / max(total, 1e-300)", ["topp_margin"]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_fail_a_pin(name):
    old, new, pins = MUTANTS[name]
    mod = _mutant(old, new)
    for p in pins:
        with pytest.raises(AssertionError):
            PINS[p](mod)


def test_unmutated_copy_passes_every_pin():
    mod = _mutant("def sigmoid(z):", "def sigmoid(z):")
    for p in PINS.values():
        p(mod)

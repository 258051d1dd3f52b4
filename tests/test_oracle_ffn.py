"""Pins of the oracle's expert arithmetic and of the whole layer.

Closed forms (one-hot input, all-equal codes), invariants (relabelling the
experts, the shared expert's weight of one) and the figures the pages print
for the int4 expert record (ideipro.ru article; Show HN page "धीमे कंप्यूटर पर
GLM 5.2 चलाना", section "disk streaming आधारित MoE execution तरीका").
"""
import math
import os

import numpy as np
import pytest
from scipy.special import expit

from oracle import moe_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _figures():
    out = {}
    with open(os.path.join(GOLDEN, "page_figures.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v, tol = (p.strip() for p in line.split("|"))
                out[k] = (float(v), float(tol))
    return out


def test_expert_record_matches_page_figures():
    fig = _figures()
    per_expert = orc.expert_bytes(6144, 2048, 4)
    assert per_expert == 18_915_328
    v, tol = fig["expert_mb_int4"]
    assert abs(per_expert / 1e6 - v) <= tol * v
    per_token = fig["moe_layers"][0] * fig["experts_per_token_per_layer"][0] * per_expert
    v, tol = fig["gb_per_token_cold"]
    assert abs(per_token / 1e9 - v) <= tol * v


def test_silu_matches_library():
    g = np.linspace(-60, 60, 1201)
    np.testing.assert_allclose(orc.silu(g), g * expit(g), rtol=1e-14, atol=1e-300)
    assert orc.silu(0.0) == 0.0


def _rand_layer(g, E, S, H, I, bits, scale_shared=True):
    lo, hi = orc.code_range(bits)
    ex = {}
    for e in range(E + S):
        d = {}
        for m, (r, c) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
            d["q_" + m] = orc.pack_rows(g.integers(lo, hi + 1, size=(r, c)), bits)
            d["s_" + m] = g.uniform(0.005, 0.02, size=r).astype(np.float32)
        ex[e] = d
    return ex


@pytest.mark.parametrize("bits", [4, 8, 2])
def test_one_hot_token_closed_form(bits):
    """K = 1, one group, a +10 bias on expert e*, shared down-scales zero and
    x = a * unit(j): the layer output reduces to a sum over the j-th columns of
    gate and up:  y_r = rsf * sd[r] * sum_i qd[r, i] * silu(a sg[i] qg[i, j]) * a su[i] qu[i, j]."""
    g = np.random.default_rng(bits)
    E, S, H, I = 8, 1, 64, 32
    ex = _rand_layer(g, E, S, H, I, bits)
    ex[E]["s_down"][:] = 0.0
    e_star, j, a, rsf = 5, 17, 1.75, 2.5
    bias = np.zeros(E, np.float32)
    bias[e_star] = 10.0
    Wr = g.standard_normal((E, H)).astype(np.float32) * 0.05
    x = np.zeros((1, H), np.float32)
    x[0, j] = a
    r = orc.moe_layer(x, Wr, bias, ex.__getitem__, n_group=1, topk_group=1, top_k=1,
                      n_shared=S, rsf=rsf, bits=bits)
    assert r.idx.tolist() == [[e_star]]
    d = ex[e_star]
    qg = orc.unpack_rows(d["q_gate"], bits)
    qu = orc.unpack_rows(d["q_up"], bits)
    qd = orc.unpack_rows(d["q_down"], bits)
    want = np.zeros(H)
    for row in range(H):
        acc = 0.0
        for i in range(I):
            gi = a * float(d["s_gate"][i]) * int(qg[i, j])
            ui = a * float(d["s_up"][i]) * int(qu[i, j])
            acc += int(qd[row, i]) * (gi / (1.0 + math.exp(-gi))) * ui
        want[row] = rsf * float(d["s_down"][row]) * acc
    np.testing.assert_allclose(r.y[0], want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


@pytest.mark.parametrize("n_shared", [0, 1, 2])
def test_all_equal_closed_form(n_shared):
    """Every code c0, every scale sigma, x = 1: every expert gives the same o
    with o_r = sigma * I * c0 * silu(sigma H c0) * sigma H c0, and the routed
    weights sum to rsf, so y = (rsf + n_shared) * o."""
    E, H, I, bits, c0, sig, rsf = 16, 64, 32, 4, -3, 0.0125, 2.5
    packed = {m: orc.pack_rows(np.full(shape, c0), bits)
              for m, shape in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I)))}
    d = {"q_" + m: packed[m] for m in packed}
    d.update({"s_gate": np.full(I, sig, np.float32), "s_up": np.full(I, sig, np.float32),
              "s_down": np.full(H, sig, np.float32)})
    sig = float(np.float32(sig))
    Wr = np.random.default_rng(1).standard_normal((E, H)).astype(np.float32)
    x = np.ones((1, H), np.float32)
    r = orc.moe_layer(x, Wr, np.zeros(E, np.float32), lambda e: d, n_group=4, topk_group=2,
                      top_k=4, n_shared=n_shared, rsf=rsf, bits=bits)
    gv = sig * H * c0
    o = sig * I * c0 * (gv / (1 + math.exp(-gv))) * gv
    wsum = float(r.w.astype(np.float64).sum())
    np.testing.assert_allclose(wsum, rsf, rtol=4 * 2.4e-7)
    np.testing.assert_allclose(r.y[0], (wsum + n_shared) * o, rtol=1e-12)


def test_relabelling_experts_leaves_output_unchanged():
    """Swapping two groups of experts together with their router rows and bias
    changes the chosen ids but not the output."""
    g = np.random.default_rng(9)
    E, S, H, I, G = 16, 1, 64, 32, 4
    ex = _rand_layer(g, E, S, H, I, 4)
    Wr = (g.standard_normal((E, H)) * 0.05).astype(np.float32)
    b = g.uniform(-0.1, 0.1, E).astype(np.float32)
    x = g.standard_normal((3, H)).astype(np.float32)
    kw = dict(n_group=G, topk_group=2, top_k=4, n_shared=S, rsf=2.5, bits=4)
    r0 = orc.moe_layer(x, Wr, b, ex.__getitem__, **kw)
    perm = np.r_[np.arange(8, 12), np.arange(4, 8), np.arange(0, 4), np.arange(12, 16)]
    ex2 = {e: ex[int(perm[e])] if e < E else ex[e] for e in range(E + S)}
    r1 = orc.moe_layer(x, Wr[perm], b[perm], ex2.__getitem__, **kw)
    np.testing.assert_allclose(r1.y, r0.y, rtol=1e-12, atol=1e-12)
    assert sorted(perm[r1.idx].ravel().tolist()) == sorted(r0.idx.ravel().tolist())


def test_shared_expert_has_unit_weight():
    """Zeroing every routed down-scale leaves exactly the shared expert's output."""
    g = np.random.default_rng(4)
    E, S, H, I = 16, 1, 64, 32
    ex = _rand_layer(g, E, S, H, I, 4)
    for e in range(E):
        ex[e]["s_down"][:] = 0
    Wr = (g.standard_normal((E, H)) * 0.05).astype(np.float32)
    x = g.standard_normal((2, H)).astype(np.float32)
    r = orc.moe_layer(x, Wr, np.zeros(E, np.float32), ex.__getitem__, n_group=4, topk_group=2,
                      top_k=4, n_shared=S, rsf=2.5, bits=4)
    d = ex[E]
    for t in range(2):
        o, _ = orc.swiglu_expert(x[t], orc.dequantize(d["q_gate"], d["s_gate"], 4),
                                 orc.dequantize(d["q_up"], d["s_up"], 4),
                                 orc.dequantize(d["q_down"], d["s_down"], 4))
        np.testing.assert_array_equal(r.y[t], o)


def test_rmsnorm_closed_form():
    x = np.full((1, 64), -3.0)
    np.testing.assert_allclose(orc.rmsnorm(x), -1.0 / math.sqrt(1.0 + 1e-6 / 9.0), rtol=1e-15)
    v = np.random.default_rng(0).standard_normal((4, 128))
    r = orc.rmsnorm(v)
    np.testing.assert_allclose(np.mean(r * r, axis=1), 1.0 / (1.0 + 1e-6 / np.mean(v * v, axis=1)),
                               rtol=1e-12)

"""The two CPU implementations of the layer against each other (no GPU).

oracle/moe_oracle.py (NumPy) and oracle/moe_ref.c (plain C) were written
separately from the same definitions (Show HN page "धीमे कंप्यूटर पर GLM 5.2
चलाना", implemented features: the router, quantisation and batch-union
items); they share no code.  On small layers, including the tiny
configuration that the oracle is pinned on, they must choose the same
experts in the same slot order with bit-identical fp32 weights, and agree on
h and y to fp64 rounding (1e-12 relative: both compute in double, only the
summation order differs).
"""
import numpy as np
import pytest

from oracle import moe_oracle as orc
from oracle import moe_ref
from quantized_moe_decode_route_amd import synth

REL = 1e-12

CASES = {
    # name: (T, H, I, E, G, TG, K, S, bits, seed)
    "tiny_seed0": (1, 256, 128, 16, 4, 2, 4, 1, 4, 0),
    "tiny_seed1": (1, 256, 128, 16, 4, 2, 4, 1, 4, 1),
    "tiny_t4": (4, 256, 128, 16, 4, 2, 4, 1, 4, 2),
    "t3_s2_q8": (3, 192, 96, 24, 4, 2, 5, 2, 8, 3),
    "t2_q2_noshared": (2, 320, 64, 12, 3, 2, 3, 0, 2, 4),
    "one_group": (3, 128, 64, 10, 1, 1, 4, 1, 4, 5),
    "every_group": (2, 128, 32, 16, 8, 8, 16, 1, 4, 6),
}


def _run_both(name, threads=1):
    T, H, I, E, G, TG, K, S, b, seed = CASES[name]
    cfg = synth.MoEConfig(name, T, H, I, E, G, TG, K, S, b, seed=seed)
    x = synth.token_pool(cfg, T)
    rw, bias = synth.router_weight(cfg, 0), synth.router_bias(cfg, 0)
    experts = {e: synth.expert_arrays(cfg, 0, e) for e in range(E + S)}
    r = orc.moe_layer(x, rw, bias, experts.__getitem__, n_group=G, topk_group=TG, top_k=K, n_shared=S,
                      rsf=cfg.rsf, bits=b)
    c = moe_ref.layer(x, rw, bias, experts, n_group=G, topk_group=TG, top_k=K, n_shared=S, rsf=cfg.rsf, bits=b,
                      threads=threads)
    return r, c


def _rel(a, b):
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300))


@pytest.mark.parametrize("name", sorted(CASES))
def test_two_cpu_implementations_agree(name):
    r, c = _run_both(name)
    np.testing.assert_allclose(c.scores64, r.scores64, rtol=1e-14, atol=0)
    np.testing.assert_array_equal(c.idx, r.idx)
    np.testing.assert_array_equal(c.w, r.w)
    assert _rel(c.h, r.h) <= REL
    assert _rel(c.y, r.y) <= REL


def test_threads_do_not_change_the_result():
    """OpenMP splits rows between threads; every row is still one sequential sum."""
    _, c1 = _run_both("tiny_t4", threads=1)
    _, c4 = _run_both("tiny_t4", threads=4)
    np.testing.assert_array_equal(c1.y, c4.y)
    np.testing.assert_array_equal(c1.h, c4.h)


def test_missing_selected_expert_is_an_error():
    T, H, I, E, G, TG, K, S, b, seed = CASES["tiny_seed0"]
    cfg = synth.MoEConfig("m", T, H, I, E, G, TG, K, S, b, seed=seed)
    x = synth.token_pool(cfg, T)
    experts = {E: synth.expert_arrays(cfg, 0, E)}          # only the shared expert
    with pytest.raises(RuntimeError):
        moe_ref.layer(x, synth.router_weight(cfg, 0), synth.router_bias(cfg, 0), experts, n_group=G,
                      topk_group=TG, top_k=K, n_shared=S, rsf=cfg.rsf, bits=b)
